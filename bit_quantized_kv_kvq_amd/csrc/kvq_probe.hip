// Achievable HBM read rate of one launch: a plain grid-stride stream of 16-byte loads, the
// denominator the decode kernel's effective rate is compared with (the decode path reads the
// whole cache once per step: page "KV Cache量化实战：Model Optimizer为大模型长上下文省下50%显存",
// section on why long context runs out of memory first).  Every 32-bit word of the buffer is
// read exactly once; each lane writes the XOR of the words it read, so the XOR of the sink
// equals the XOR of the buffer (which the tests check) and no load can be dropped.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Eight independent nontemporal 16-byte loads in flight per lane and iteration: of the shapes
// measured on a 4 GiB buffer (1024-8192 workgroups, 4-16 loads per lane, with and without the
// nontemporal policy: 5.4-6.5 TB/s) the fastest.
constexpr int kProbeUnroll = 8;
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4 *__restrict__ p, int64_t n, uint32_t *sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * stride < n; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= fold(v[u]);
  }
  for (; i < n; i += stride) acc ^= fold(__builtin_nontemporal_load(p + i));
  sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s) {
  read_probe_kernel<<<kProbeBlocks, kProbeThreads, 0, s>>>((const u32x4 *)buf, (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace kvq
