// Scratch memory of kvq_decode_attn_noalloc, the decode entry point that allocates nothing.
//
// The decode kernel needs a workspace: per (batch, kv_head) an arrival counter and the chunk
// cursors, and the split-K partials (m, l, o) of its work items.  kvq_decode_attn takes it
// from the caller; for callers that cannot allocate it lives here, in a file-scope device
// array of kNoAllocScratchBytes.  Each GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` is only a stand-in for the symbol: its device
// address on the current GPU comes from hipGetSymbolAddress, looked up once per device and
// kept, and only that address is ever handed to a kernel.
//
// Every call on a GPU uses that GPU's one array: calls that overlap in time on one GPU (two
// streams, or two threads) race on it.  The counters and cursors must start at zero; the
// array is cleared once per device by a fill kernel on the first call's stream, and every
// decode call leaves them at zero again when it ends.  The partials need no clearing.
#include "kvq_internal.h"

#include <mutex>
#include <vector>

namespace kvq {
namespace {

__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

__global__ void zero_fill(uint4 *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

std::mutex g_mu;
std::vector<void *> g_scratch;   // per device id: that device's address of `scratch` (null until set up)

}  // namespace

hipError_t noalloc_scratch(void **ptr, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_mu);
  if ((int)g_scratch.size() <= dev) g_scratch.resize((size_t)dev + 1, nullptr);
  if (!g_scratch[(size_t)dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    zero_fill<<<256, 256, 0, s>>>((uint4 *)p, kNoAllocScratchBytes / sizeof(uint4));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch[(size_t)dev] = p;
  }
  *ptr = g_scratch[(size_t)dev];
  return hipSuccess;
}

}  // namespace kvq
