// Copy of new fp16 tokens into the residual of one (batch, kv_head) (page "KV缓存量化技术：
// 提升大模型长文本生成效率" §2.2: the newest tokens stay unquantized in a residual cache),
// shared by the append's copy kernel, the flush that refills the residual it has just read, and
// the decode launch that copies its step's tokens.
//
// The residual holds K as rows [R][128] and V as [R/16][128][16] (16 consecutive slots of one
// dim together).  K rows are copied as 16-byte words.  V is transposed on the way: a run of 8
// slots that starts at a multiple of 8 is one 16-byte store, gathered from 8 source rows with
// 2-byte loads that are coalesced across the dims; the slots before the first such run and
// after the last one are stored one value at a time.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kvq {
namespace {

// Tokens [0, count) of k ([count][128] fp16, 16-byte aligned rows) go to K slots
// [slot0, slot0 + count) of the residual at `res`, by threads tid = 0 .. nthr - 1.
__device__ __forceinline__ void residual_store_k(const uint16_t *k, int count, int slot0, uint8_t *res, int tid,
                                                 int nthr) {
  uint16_t *rk = (uint16_t *)res;
  for (int e = tid; e < count * 16; e += nthr) {
    const int t = e >> 4, ch = e & 15;
    *(uint4 *)(rk + (int64_t)(slot0 + t) * 128 + ch * 8) = *(const uint4 *)(k + (int64_t)t * 128 + ch * 8);
  }
}

// Tokens [0, count) of v ([count][128] fp16) go to V slots [slot0, slot0 + count) of the
// residual at `res` (R slots); only those slots' values are written.
__device__ __forceinline__ void residual_store_v(const uint16_t *v, int count, int slot0, uint8_t *res, int R, int tid,
                                                 int nthr) {
  uint16_t *rv = (uint16_t *)(res + (int64_t)R * 256);
  const int head = min(count, (8 - (slot0 & 7)) & 7);   // slots before the first 8-aligned run
  const int nrun = (count - head) >> 3;
  const int tail0 = head + 8 * nrun;                     // first token after the runs
  for (int e = tid; e < nrun * 128; e += nthr) {
    const int t0 = head + 8 * (e >> 7), d = e & 127, s0 = slot0 + t0;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)v[(int64_t)(t0 + 2 * i) * 128 + d] | ((uint32_t)v[(int64_t)(t0 + 2 * i + 1) * 128 + d] << 16);
    *(uint4 *)(rv + ((int64_t)(s0 >> 4) * 128 + d) * 16 + (s0 & 15)) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  const int nloose = head + (count - tail0);
  for (int e = tid; e < nloose * 128; e += nthr) {
    const int i = e >> 7, d = e & 127;
    const int t = i < head ? i : tail0 + (i - head), s = slot0 + t;
    rv[((int64_t)(s >> 4) * 128 + d) * 16 + (s & 15)] = v[(int64_t)t * 128 + d];
  }
}

// Both halves: tokens [0, count) of k and v into slots [slot0, slot0 + count).
__device__ __forceinline__ void residual_store(const uint16_t *k, const uint16_t *v, int count, int slot0,
                                               uint8_t *res, int R, int tid, int nthr) {
  residual_store_k(k, count, slot0, res, tid, nthr);
  residual_store_v(v, count, slot0, res, R, tid, nthr);
}

}  // namespace
}  // namespace kvq
