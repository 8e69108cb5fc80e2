// Achievable HBM read rate of one launch: a plain grid-stride stream of 16-byte loads, the
// denominator the decode kernel's effective rate is compared with (the decode path reads the
// whole cache once per step: page "KV Cache量化实战：Model Optimizer为大模型长上下文省下50%显存",
// section on why long context runs out of memory first).  Every 32-bit word of the buffer is
// read exactly once; each lane writes the XOR of the words it read, so the XOR of the sink
// equals the XOR of the buffer (which the tests check) and no load can be dropped.
#include "kvq_internal.h"

namespace kvq {
namespace {

__device__ __forceinline__ uint32_t fold(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4 *__restrict__ p, int64_t n, uint32_t *sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  // four independent loads in flight per lane and iteration
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
  }
  for (; i < n; i += stride) acc ^= fold(p[i]);
  sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s) {
  read_probe_kernel<<<kProbeBlocks, kProbeThreads, 0, s>>>((const uint4 *)buf, (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace kvq
