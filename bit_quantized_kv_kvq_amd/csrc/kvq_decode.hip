// Fused dequant + single-token decode attention of libkvq (gfx950).
//
// Every decode step reads the whole cached history (page "KV Cache量化实战：Model Optimizer
// 为大模型长上下文省下50%显存", section on why long context runs out of memory first) and the
// dequantized K/V take part in attention (page "NVFP4 KV缓存技术详解" §2.1).  The kernel
// streams the packed blocks once and dequantizes in registers; no fp16 copy of the cache is
// ever written.
//
// One launch per call.  A workgroup (4 waves) owns a work item: a run of 128-slot blocks of
// one tier of one (batch, kv_head), and the last item of each (batch, kv_head) also covers
// the fp16 residual.  Blocks stream HBM -> LDS through 16-byte LDS-DMA loads into a ring of
// four buffers (three for INT8), so up to three blocks are in flight while the waves compute
// on the fourth.  Wave w
// handles slots 32w..32w+31 of every block for all G query heads of the kv head (GQA: each
// byte is read once per group).  At the end of an item the four waves merge their running
// softmax states in LDS, the workgroup writes one partial (m, l, o) and bumps an arrival
// counter; the last workgroup of a (batch, kv_head) merges all partials with a log-sum-exp
// reduction and writes the output.  The partials and the counter use agent-scope atomics
// only: no device-wide fence (which would write back and invalidate the L2 of the XCD).
//
// Matrix cores, per 32 slots of a wave (v_mfma_f32_16x16x32_f16):
//  QK^T  A = K codes (16 slots x 32 dims), B = Q^T (32 dims x 16 heads; heads >= G are zero);
//        lane (c, g) = (lane & 15, lane >> 4) feeds slot c and receives the logits of slots
//        4g..4g+3 of the tile for head c.
//  PV    O^T += V^T P: A = V codes (16 dims x 32 slots), B = P (32 slots x 16 heads); lane
//        (c, g) feeds dim c of the tile and the 8 slots whose logits it holds, and accumulates
//        O^T[dims 4g..4g+3][head c].
// Affine: the MFMA takes exact code integers as fp16 (some scaled by 16).  K: codes c,
// logit = S0 (dot0 - Z0 qsum0) + S1 (dot1 - Z1 qsum1) per 64-dim group.  V: codes c - C with
// C = 2^(n-1); the scale S of each (slot, group) is folded into P and the zero point enters as
// o -= sum_t P'_t (Z_t - C).
// NVFP4: E2M1 codes and E4M3 scales are converted by the hardware to fp16 and multiplied
// (exact: at most 6 significant bits, magnitude in [2^-10, 2688]).
#include "kvq_internal.h"

#include <algorithm>
#include <cmath>

namespace kvq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kNegInf = -INFINITY;

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u(half2_t h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ half8_t h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(half8_t, u32x4{a, b, c, d});
}
__device__ __forceinline__ float lo_f(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFF)); }
__device__ __forceinline__ float hi_f(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16)); }
__device__ __forceinline__ uint32_t pk(float a, float b) { return as_u(half2_t{(_Float16)a, (_Float16)b}); }

__device__ __forceinline__ float4_t mfma(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// fp16 pair (1024 + f_lo, 1024 + f_hi) of the two fields selected by mask, minus 1024 + off:
// exact (f - off, or 16 f - off for a mask shifted by 4 bits).
// (x & mask) | magic in one v_and_or_b32; gfx950 VOP3 reads at most one scalar operand, so the
// magic constant lives in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic_v) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(magic_v));
  return r;
}
template <int OFF = 0>
__device__ __forceinline__ uint32_t field_pair(uint32_t x, uint32_t mask) {
  constexpr _Float16 k = (_Float16)(1024.0f + OFF);
  return as_u(as_h2(and_or(x, mask, 0x64006400u)) - half2_t{k, k});
}

// ---------------------------------------------------------------- operand unpack per format
// The K operand takes the codes c as they are; the V operand takes c - C (C = 2^(n-1)), so
// that the PV sums stay centred and the zero-point term sum P'(Z - C) stays small over long
// contexts (no cancellation between two large sums).
// INT4 word -> [n0, n4, 16n1, 16n5, n2, n6, 16n3, 16n7] - C (n_v = nibble v; 16 C on the
// scaled positions)
template <bool CENTER>
__device__ __forceinline__ half8_t unpack_int4(uint32_t x) {
  const uint32_t y = x >> 8;
  constexpr int C1 = CENTER ? 8 : 0, C16 = CENTER ? 128 : 0;
  return h8(field_pair<C1>(x, 0x000F000Fu), field_pair<C16>(x, 0x00F000F0u), field_pair<C1>(y, 0x000F000Fu),
            field_pair<C16>(y, 0x00F000F0u));
}
// INT2 word -> lo = crumbs [0,8,1,9,2,10,3,11], hi = [4,12,5,13,6,14,7,15] (minus C)
template <bool CENTER>
__device__ __forceinline__ void unpack_int2(uint32_t x, half8_t &lo, half8_t &hi) {
  constexpr int C = CENTER ? 2 : 0;
  lo = h8(field_pair<C>(x, 0x00030003u), field_pair<C>(x >> 2, 0x00030003u), field_pair<C>(x >> 4, 0x00030003u),
          field_pair<C>(x >> 6, 0x00030003u));
  hi = h8(field_pair<C>(x >> 8, 0x00030003u), field_pair<C>(x >> 10, 0x00030003u), field_pair<C>(x >> 12, 0x00030003u),
          field_pair<C>(x >> 14, 0x00030003u));
}
// INT8 word pair -> [w0.b0, w0.b2, w0.b1, w0.b3, w1.b0, w1.b2, w1.b1, w1.b3] (minus C)
template <bool CENTER>
__device__ __forceinline__ half8_t unpack_int8(uint32_t w0, uint32_t w1) {
  constexpr int C = CENTER ? 128 : 0;
  return h8(field_pair<C>(w0, 0x00FF00FFu), field_pair<C>(w0 >> 8, 0x00FF00FFu), field_pair<C>(w1, 0x00FF00FFu),
            field_pair<C>(w1 >> 8, 0x00FF00FFu));
}
// NVFP4 word (8 E2M1 codes, nibble order) times per-pair fp16 scales
__device__ __forceinline__ half8_t unpack_fp4(uint32_t x, uint32_t s01, uint32_t s23, uint32_t s45, uint32_t s67) {
  const uint32_t a = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 0));
  const uint32_t b = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 1));
  const uint32_t c = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2));
  const uint32_t d = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 3));
  return h8(as_u(as_h2(a) * as_h2(s01)), as_u(as_h2(b) * as_h2(s23)), as_u(as_h2(c) * as_h2(s45)), as_u(as_h2(d) * as_h2(s67)));
}
// two E4M3 bytes (bits 0-15 of x, sel = false; bits 16-31, sel = true) -> fp16 pair (exact)
__device__ __forceinline__ uint32_t e4m3_pair(uint32_t x, bool sel) {
  return as_u(sel ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true)
                  : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false));
}

// ---------------------------------------------------------------- Q operand per format
// Dim fed by B element e of k-step j in lane quarter g, and whether the A element it meets
// carries a factor 16 (then B holds q / 16).
template <int FMT>
__device__ __forceinline__ int q_dim(int g, int j, int e, bool &scaled) {
  const int G = j >> 1, h = j & 1;
  scaled = false;
  if constexpr (FMT == kFmtInt4) {
    scaled = ((e >> 1) & 1) != 0;
    return 64 * G + 16 * g + 8 * h + (e >> 1) + 4 * (e & 1);
  } else if constexpr (FMT == kFmtInt2) {
    return 64 * G + 16 * g + 4 * h + (e >> 1) + 8 * (e & 1);
  } else if constexpr (FMT == kFmtInt8) {
    return 64 * G + 16 * g + 4 * (2 * h + (e >> 2)) + ((e >> 1) & 1) + 2 * (e & 1);
  } else {
    return 32 * g + 8 * j + e;   // NVFP4 and the fp16 residual: natural order
  }
}

// The 32 dims a lane quarter g feeds: affine formats dims 16g..16g+15 and 64+16g..64+16g+15
// (local index 16G + m); NVFP4 and fp16 dims 32g..32g+31 (local index dim - 32g).
template <int FMT>
__device__ __forceinline__ void load_q(const uint16_t *qrow, bool valid, int g, half8_t (&qb)[4], float &qs0, float &qs1) {
  constexpr bool kAff = FMT == kFmtInt2 || FMT == kFmtInt4 || FMT == kFmtInt8;
  uint4 raw[4];
  if constexpr (kAff) {
    raw[0] = *(const uint4 *)(qrow + 16 * g);
    raw[1] = *(const uint4 *)(qrow + 16 * g + 8);
    raw[2] = *(const uint4 *)(qrow + 64 + 16 * g);
    raw[3] = *(const uint4 *)(qrow + 64 + 16 * g + 8);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = *(const uint4 *)(qrow + 32 * g + 8 * i);
  }
  _Float16 loc[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half8_t v = __builtin_bit_cast(half8_t, raw[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) loc[8 * i + e] = valid ? v[e] : (_Float16)0.0f;
  }
  qs0 = 0.0f;
  qs1 = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bool scaled;
      const int d = q_dim<FMT>(g, j, e, scaled);
      const int li = kAff ? 16 * (d >> 6) + (d & 15) : d - 32 * g;
      _Float16 v = loc[li];
      if (scaled) v = v * (_Float16)0.0625f;
      qb[j][e] = v;
      const float eff = scaled ? 16.0f * (float)v : (float)v;    // the q the MFMA effectively uses
      if (j < 2) qs0 += eff; else qs1 += eff;
    }
  }
  // group sums over the four lane quarters (lanes c, c+16, c+32, c+48 hold one head)
  qs0 += __shfl_xor(qs0, 16);
  qs0 += __shfl_xor(qs0, 32);
  qs1 += __shfl_xor(qs1, 16);
  qs1 += __shfl_xor(qs1, 32);
}

// ---------------------------------------------------------------- LDS DMA
// 16 bytes per lane from global `src` to LDS address lds + 16 * lane (wave-uniform lds).
// M0 is saved and restored around the load so the compiler's use of it is undisturbed.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
    case 15: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 17: asm volatile("s_waitcnt vmcnt(17)" ::: "memory"); break;
    case 18: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
    case 19: asm volatile("s_waitcnt vmcnt(19)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
  }
}

// Barrier without a memory fence: LDS-DMA completion is established by each wave's own
// vmcnt wait before it; the empty asm statements keep the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------- running softmax state
struct State {
  float m = kNegInf;   // running max (log2 domain) of head c, same on the 4 lane quarters
  float l = 0.0f;      // this lane's share of sum p
  float z1 = 0.0f, z16 = 0.0f;   // affine V: this lane's share of sum P' Z (group 0 / 1 folded below)
  float z1b = 0.0f, z16b = 0.0f;
  float4_t o[8];       // O^T[dims 16k + 4g + i][head c]
};

// Update the running max with 8 logits (slots (tt, i) = (e >> 2, e & 3)) and return the
// probabilities; positions whose A element is scaled by 16 (mask bit e) get p / 16.
__device__ __forceinline__ void softmax_step(State &st, const float (&s)[8], float (&p)[8], bool valid_head,
                                             unsigned scaled_mask) {
  float mt = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
  mt = fmaxf(mt, __shfl_xor(mt, 16));
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  const bool grow = valid_head && mt > st.m;
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    const float m_new = fmaxf(st.m, mt);
    const float alpha = (m_new == kNegInf) ? 1.0f : __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
    st.z1 *= alpha; st.z16 *= alpha; st.z1b *= alpha; st.z16b *= alpha;
#pragma unroll
    for (int k = 0; k < 8; ++k) st.o[k] *= alpha;
    st.m = m_new;
  }
  const float m0 = st.m == kNegInf ? 0.0f : st.m;
  const float m4 = m0 + 4.0f;
  float ls = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bool sc = (scaled_mask >> e) & 1;
    p[e] = __builtin_amdgcn_exp2f(s[e] - (sc ? m4 : m0));   // v_exp_f32; results below 2^-126 flush to 0
    ls = sc ? fmaf(16.0f, p[e], ls) : ls + p[e];
  }
  st.l += ls;
}

// ---------------------------------------------------------------- one 32-slot step per format
// blk: LDS copy of the block; w: wave; TAIL: only the first nvalid slots of the block hold
// tokens (the last block of a tier).
template <int NB, bool TAIL>
__device__ __forceinline__ void affine_step(const uint8_t *blk, int w, int g, int c, const half8_t (&qb)[4], float qs0,
                                            float qs1, float sl2, bool valid_head, int nvalid, State &st) {
  constexpr int kRow = 16 * NB;                      // K row bytes
  constexpr int kKm = 2048 * NB, kVc = 2048 * NB + 1024, kVm = 4096 * NB + 1024;
  const int lane = 16 * g + c;
  float s[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tau = 2 * w + tt;
    const uint8_t *row = blk + (32 * w + 16 * tt + c) * kRow + g * (4 * NB);
    float4_t a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = a0;
    if constexpr (NB == 4) {
      const uint4 x = *(const uint4 *)row;
      a0 = mfma(unpack_int4<false>(x.x), qb[0], a0);
      a0 = mfma(unpack_int4<false>(x.y), qb[1], a0);
      a1 = mfma(unpack_int4<false>(x.z), qb[2], a1);
      a1 = mfma(unpack_int4<false>(x.w), qb[3], a1);
    } else if constexpr (NB == 2) {
      const uint2 x = *(const uint2 *)row;
      half8_t l0, h0, l1, h1;
      unpack_int2<false>(x.x, l0, h0);
      unpack_int2<false>(x.y, l1, h1);
      a0 = mfma(l0, qb[0], a0);
      a0 = mfma(h0, qb[1], a0);
      a1 = mfma(l1, qb[2], a1);
      a1 = mfma(h1, qb[3], a1);
    } else {
      const uint4 x = *(const uint4 *)row, y = *(const uint4 *)(row + 16);
      a0 = mfma(unpack_int8<false>(x.x, x.y), qb[0], a0);
      a0 = mfma(unpack_int8<false>(x.z, x.w), qb[1], a0);
      a1 = mfma(unpack_int8<false>(y.x, y.y), qb[2], a1);
      a1 = mfma(unpack_int8<false>(y.z, y.w), qb[3], a1);
    }
    const uint4 ks = *(const uint4 *)(blk + kKm + tau * 128 + 16 * g);        // (S0, S1) of slots 4g+i
    const uint4 kz = *(const uint4 *)(blk + kKm + tau * 128 + 64 + 16 * g);   // (Z0, Z1)
    const uint32_t sw[4] = {ks.x, ks.y, ks.z, ks.w}, zw[4] = {kz.x, kz.y, kz.z, kz.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float u0 = fmaf(-lo_f(zw[i]), qs0, a0[i]);
      const float u1 = fmaf(-hi_f(zw[i]), qs1, a1[i]);
      float v = fmaf(hi_f(sw[i]), u1, lo_f(sw[i]) * u0) * sl2;
      if (TAIL && 16 * tau + 4 * g + i >= nvalid) v = kNegInf;
      s[4 * tt + i] = v;
    }
  }
  float p[8];
  constexpr unsigned kScaled = NB == 4 ? 0xCCu : 0u;   // INT4: positions i = 2, 3 of both tiles
  softmax_step(st, s, p, valid_head, kScaled);

  // P' = p * S per group, and the zero-point sums sum P' (Z - C)
  half8_t pb[2];
  {
    uint32_t pw[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint4 vm0 = *(const uint4 *)(blk + kVm + ((2 * w + tt) * 4 + g) * 32);        // S_G0[0..3], S_G1[0..3]
      const uint4 vz = *(const uint4 *)(blk + kVm + ((2 * w + tt) * 4 + g) * 32 + 16);    // Z_G0[0..3], Z_G1[0..3]
      constexpr _Float16 kC = (_Float16)(1 << (NB - 1));
      const half2_t cc = {kC, kC};
      const uint4 vm1 = {as_u(as_h2(vz.x) - cc), as_u(as_h2(vz.y) - cc), as_u(as_h2(vz.z) - cc), as_u(as_h2(vz.w) - cc)};
      // p * S in fp32, rounded once to fp16
      const float *pp = p + 4 * tt;
      const uint32_t a01 = pk(pp[0] * lo_f(vm0.x), pp[1] * hi_f(vm0.x)), a23 = pk(pp[2] * lo_f(vm0.y), pp[3] * hi_f(vm0.y));
      const uint32_t b01 = pk(pp[0] * lo_f(vm0.z), pp[1] * hi_f(vm0.z)), b23 = pk(pp[2] * lo_f(vm0.w), pp[3] * hi_f(vm0.w));
      pw[0][2 * tt + 0] = a01; pw[0][2 * tt + 1] = a23;
      pw[1][2 * tt + 0] = b01; pw[1][2 * tt + 1] = b23;
      if constexpr (NB == 4) {
        st.z1 = __builtin_amdgcn_fdot2(as_h2(a01), as_h2(vm1.x), st.z1, false);
        st.z16 = __builtin_amdgcn_fdot2(as_h2(a23), as_h2(vm1.y), st.z16, false);
        st.z1b = __builtin_amdgcn_fdot2(as_h2(b01), as_h2(vm1.z), st.z1b, false);
        st.z16b = __builtin_amdgcn_fdot2(as_h2(b23), as_h2(vm1.w), st.z16b, false);
      } else {
        st.z1 = __builtin_amdgcn_fdot2(as_h2(a01), as_h2(vm1.x), st.z1, false);
        st.z1 = __builtin_amdgcn_fdot2(as_h2(a23), as_h2(vm1.y), st.z1, false);
        st.z1b = __builtin_amdgcn_fdot2(as_h2(b01), as_h2(vm1.z), st.z1b, false);
        st.z1b = __builtin_amdgcn_fdot2(as_h2(b23), as_h2(vm1.w), st.z1b, false);
      }
    }
    pb[0] = h8(pw[0][0], pw[0][1], pw[0][2], pw[0][3]);
    pb[1] = h8(pw[1][0], pw[1][1], pw[1][2], pw[1][3]);
  }

  // V codes of this lane: [part w][chunk r][lane][16 B]
  constexpr int kChunks = NB / 2;
  const uint8_t *vc = blk + kVc + (w * kChunks * 64 + lane) * 16;
  if constexpr (NB == 4) {
    const uint4 x0 = *(const uint4 *)vc, x1 = *(const uint4 *)(vc + 1024);
    st.o[0] = mfma(unpack_int4<true>(x0.x), pb[0], st.o[0]);
    st.o[1] = mfma(unpack_int4<true>(x0.y), pb[0], st.o[1]);
    st.o[2] = mfma(unpack_int4<true>(x0.z), pb[0], st.o[2]);
    st.o[3] = mfma(unpack_int4<true>(x0.w), pb[0], st.o[3]);
    st.o[4] = mfma(unpack_int4<true>(x1.x), pb[1], st.o[4]);
    st.o[5] = mfma(unpack_int4<true>(x1.y), pb[1], st.o[5]);
    st.o[6] = mfma(unpack_int4<true>(x1.z), pb[1], st.o[6]);
    st.o[7] = mfma(unpack_int4<true>(x1.w), pb[1], st.o[7]);
  } else if constexpr (NB == 2) {
    const uint4 x = *(const uint4 *)vc;
    const uint32_t ws[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      half8_t lo, hi;
      unpack_int2<true>(ws[u], lo, hi);
      st.o[2 * u] = mfma(lo, pb[u >> 1], st.o[2 * u]);
      st.o[2 * u + 1] = mfma(hi, pb[u >> 1], st.o[2 * u + 1]);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint4 x = *(const uint4 *)(vc + r * 1024);
      st.o[2 * r] = mfma(unpack_int8<true>(x.x, x.y), pb[r >> 1], st.o[2 * r]);
      st.o[2 * r + 1] = mfma(unpack_int8<true>(x.z, x.w), pb[r >> 1], st.o[2 * r + 1]);
    }
  }
}

template <bool TAIL>
__device__ __forceinline__ void nvfp4_step(const uint8_t *blk, int w, int g, int c, const half8_t (&qb)[4], float sl2,
                                           bool valid_head, int nvalid, State &st) {
  const int lane = 16 * g + c;
  float s[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = 32 * w + 16 * tt + c;
    const uint4 x = *(const uint4 *)(blk + t * 64 + 16 * g);                  // dims 32g .. 32g+31
    const uint32_t sb = *(const uint16_t *)(blk + kNvKs + t * 8 + 2 * g);     // scales of blocks 2g, 2g+1
    const uint32_t s0 = e4m3_pair((sb & 0xFFu) * 0x0101u, false);             // (s_2g, s_2g)
    const uint32_t s1 = e4m3_pair((sb >> 8) * 0x0101u, false);                // (s_2g+1, s_2g+1)
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = mfma(unpack_fp4(x.x, s0, s0, s0, s0), qb[0], acc);
    acc = mfma(unpack_fp4(x.y, s0, s0, s0, s0), qb[1], acc);
    acc = mfma(unpack_fp4(x.z, s1, s1, s1, s1), qb[2], acc);
    acc = mfma(unpack_fp4(x.w, s1, s1, s1, s1), qb[3], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = acc[i] * sl2;
      if (TAIL && 16 * (2 * w + tt) + 4 * g + i >= nvalid) v = kNegInf;
      s[4 * tt + i] = v;
    }
  }
  float p[8];
  softmax_step(st, s, p, valid_head, 0u);
  const half8_t pb = h8(pk(p[0], p[1]), pk(p[2], p[3]), pk(p[4], p[5]), pk(p[6], p[7]));
  const uint8_t *vc = blk + kNvVc + (w * 2 * 64 + lane) * 16;
  const uint8_t *vs = blk + kNvVs + (4 * w + g) * 64;                          // [k][e] scale bytes
  const uint4 x0 = *(const uint4 *)vc, x1 = *(const uint4 *)(vc + 1024);
  const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint2 sc = *(const uint2 *)(vs + 8 * k);
    const half8_t a = unpack_fp4(xw[k], e4m3_pair(sc.x, false), e4m3_pair(sc.x, true), e4m3_pair(sc.y, false),
                                 e4m3_pair(sc.y, true));
    st.o[k] = mfma(a, pb, st.o[k]);
  }
}

// fp16 residual, 32 slots u*32 .. u*32+31 (direct global loads; R slots allocated, r used).
__device__ __forceinline__ void residual_step(const uint8_t *res, int R, int r, int u, int g, int c, const half8_t (&qb)[4],
                                              float sl2, bool valid_head, State &st) {
  const int ntiles = R / 16;
  float s[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tau = 2 * u + tt;
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (tau < ntiles) {
      const int t = 16 * tau + c;
      const uint4 *row = (const uint4 *)(res + t * 256 + 64 * g);   // dims 32g .. 32g+31
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma(__builtin_bit_cast(half8_t, row[j]), qb[j], acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = 16 * tau + 4 * g + i;
      s[4 * tt + i] = (tau < ntiles && slot < r) ? acc[i] * sl2 : kNegInf;
    }
  }
  float p[8];
  softmax_step(st, s, p, valid_head, 0u);
  const half8_t pb = h8(pk(p[0], p[1]), pk(p[2], p[3]), pk(p[4], p[5]), pk(p[6], p[7]));
  const uint8_t *vres = res + (int64_t)R * 256;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int d = 16 * k + c;
    uint32_t v[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tau = 2 * u + tt;
      if (tau < ntiles) {
        const uint2 x = *(const uint2 *)(vres + ((tau * kHeadDim + d) * 16 + 4 * g) * 2);
        v[2 * tt] = x.x;
        v[2 * tt + 1] = x.y;
        // slots past r may hold stale bits (even NaN): zero them
        const int s0 = 16 * tau + 4 * g;
        if (s0 + 0 >= r) v[2 * tt] &= 0xFFFF0000u;
        if (s0 + 1 >= r) v[2 * tt] &= 0x0000FFFFu;
        if (s0 + 2 >= r) v[2 * tt + 1] &= 0xFFFF0000u;
        if (s0 + 3 >= r) v[2 * tt + 1] &= 0x0000FFFFu;
      }
    }
    st.o[k] = mfma(h8(v[0], v[1], v[2], v[3]), pb, st.o[k]);
  }
}

// ---------------------------------------------------------------- the kernel
struct Item {
  int bh, part, seg;          // seg = -1: residual only
  int64_t blk_lo, blk_hi;     // blocks of the segment
  bool has_res;
};

__device__ __forceinline__ Item decode_item(const DecodeArgs &a, int wg) {
  const int nbh = a.B * a.H;
  Item it;
  it.bh = wg % nbh;
  it.part = a.items_total - 1 - wg / nbh;      // the residual-carrying last part starts first
  it.seg = -1;
  it.blk_lo = it.blk_hi = 0;
  for (int s = 0; s < a.nseg; ++s) {
    const DecodeSeg &sg = a.seg[s];
    if (it.part >= sg.part0 && it.part < sg.part0 + sg.items) {
      it.seg = s;
      const int64_t nblk = (sg.ntok + kBlock - 1) / kBlock;
      it.blk_lo = (int64_t)(it.part - sg.part0) * sg.blocks_per_item;
      it.blk_hi = min(nblk, it.blk_lo + sg.blocks_per_item);
    }
  }
  it.has_res = a.res_ntok > 0 && it.part == a.items_total - 1;
  return it;
}

__device__ __forceinline__ int block_bytes_of(int fmt) { return (int)block_bytes(fmt); }

// LDS ring depth: four blocks (three in flight) when two workgroups still fit in a CU.
__host__ __device__ __forceinline__ int ring_depth(int bb) { return bb <= 18432 ? 4 : 3; }

template <int FMT>
__device__ void stream_segment(const DecodeArgs &a, const DecodeSeg &sg, const Item &it, uint8_t *smem, int w, int g, int c,
                               bool valid_head, State &st) {
  const int lane = 16 * g + c;
  const int bb = block_bytes_of(FMT);
  const int ndma = bb / 1024;                                 // 1 KB per wave instruction
  const int mine = (ndma - w + kWaves - 1) / kWaves;          // instructions this wave issues per block
  const int b = it.bh / a.H, h = it.bh % a.H;
  const uint16_t *qrow = a.q + ((int64_t)b * a.H * a.G + (int64_t)h * a.G + (valid_head ? c : 0)) * kHeadDim;
  half8_t qb[4];
  float qs0, qs1;
  load_q<FMT>(qrow, valid_head, g, qb, qs0, qs1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  const uint8_t *gbase = sg.base + (int64_t)it.bh * sg.bh_stride + it.blk_lo * (int64_t)bb + lane * 16;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const int nbuf = ring_depth(bb);
  const int n = (int)(it.blk_hi - it.blk_lo);
  auto issue = [&](int i) {
    const uint8_t *src = gbase + (int64_t)i * bb;
    const uint32_t dst = lds0 + (uint32_t)((i % nbuf) * bb);
    for (int j = w; j < ndma; j += kWaves) dma16(src + j * 1024, __builtin_amdgcn_readfirstlane(dst + j * 1024));
  };
  for (int i = 0; i < nbuf - 1 && i < n; ++i) issue(i);
  // valid slots in the last block of the segment (128 when it is full)
  const int64_t nblk_seg = (sg.ntok + kBlock - 1) / kBlock;
  const int tail_valid = (int)(sg.ntok - (nblk_seg - 1) * kBlock);
  const bool has_tail = it.blk_hi == nblk_seg && tail_valid < kBlock;
  const int nfull = has_tail ? n - 1 : n;
  int buf = 0;
  for (int i = 0; i < n; ++i) {
    // blocks i+1 .. i+nbuf-2 may still be in flight
    wait_vmcnt(mine * min(nbuf - 2, n - 1 - i));
    barrier();
    if (i + nbuf - 1 < n) issue(i + nbuf - 1);
    const uint8_t *blk = smem + buf * bb;
    buf = buf + 1 == nbuf ? 0 : buf + 1;
    if (i < nfull) {
      if constexpr (FMT == kFmtNvfp4) nvfp4_step<false>(blk, w, g, c, qb, a.scale_log2, valid_head, kBlock, st);
      else affine_step<FMT, false>(blk, w, g, c, qb, qs0, qs1, a.scale_log2, valid_head, kBlock, st);
    } else {
      if constexpr (FMT == kFmtNvfp4) nvfp4_step<true>(blk, w, g, c, qb, a.scale_log2, valid_head, tail_valid, st);
      else affine_step<FMT, true>(blk, w, g, c, qb, qs0, qs1, a.scale_log2, valid_head, tail_valid, st);
    }
  }
  barrier();   // every wave is done with the ring before it is reused
  if constexpr (FMT != kFmtNvfp4) {
    // fold the zero points into o: o[d] -= sum_t P'_t (Z_t - C) of the group of d
    float zg0 = st.z1 + 16.0f * st.z16, zg1 = st.z1b + 16.0f * st.z16b;
    zg0 += __shfl_xor(zg0, 16);
    zg0 += __shfl_xor(zg0, 32);
    zg1 += __shfl_xor(zg1, 16);
    zg1 += __shfl_xor(zg1, 32);
#pragma unroll
    for (int k = 0; k < 8; ++k) st.o[k] -= (k < 4 ? zg0 : zg1);
    st.z1 = st.z16 = st.z1b = st.z16b = 0.0f;
  }
}

__global__ __launch_bounds__(kThreads, 2) void decode_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const bool valid_head = c < a.G;
  const Item it = decode_item(a, blockIdx.x);
  State st;
#pragma unroll
  for (int k = 0; k < 8; ++k) st.o[k] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  if (it.seg >= 0) {
    const DecodeSeg &sg = a.seg[it.seg];
    switch (sg.fmt) {
      case kFmtInt2: stream_segment<kFmtInt2>(a, sg, it, smem, w, g, c, valid_head, st); break;
      case kFmtInt4: stream_segment<kFmtInt4>(a, sg, it, smem, w, g, c, valid_head, st); break;
      case kFmtInt8: stream_segment<kFmtInt8>(a, sg, it, smem, w, g, c, valid_head, st); break;
      default: stream_segment<kFmtNvfp4>(a, sg, it, smem, w, g, c, valid_head, st); break;
    }
  }
  if (it.has_res) {
    const int b = it.bh / a.H, h = it.bh % a.H;
    const uint16_t *qrow = a.q + ((int64_t)b * a.H * a.G + (int64_t)h * a.G + (valid_head ? c : 0)) * kHeadDim;
    half8_t qb[4];
    float qs0, qs1;
    load_q<kFmtFp16>(qrow, valid_head, g, qb, qs0, qs1);
    const uint8_t *res = a.res_base + (int64_t)it.bh * a.res_bh_stride;
    const int nsteps = (a.res_ntok + 31) / 32;
    for (int u = w; u < nsteps; u += kWaves) residual_step(res, a.res_len, a.res_ntok, u, g, c, qb, a.scale_log2, valid_head, st);
  }

  // ---- merge the four waves in LDS: per wave m[16], l[16], o[16][128]
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  float *wm = (float *)smem;                       // [4][16]
  float *wl = wm + kWaves * 16;                    // [4][16]
  float *wo = wl + kWaves * 16;                    // [4][16][128]
  if (g == 0) {
    wm[w * 16 + c] = st.m;
    wl[w * 16 + c] = l;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) *(float4_t *)(wo + ((w * 16 + c) * kHeadDim + 16 * k + 4 * g)) = st.o[k];
  __syncthreads();

  const int G = a.G;
  float *part = a.partials + ((int64_t)it.bh * kMaxParts + it.part) * G * kPartialStride;
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kThreads) {
    const int hc = idx >> 7, d = idx & 127;
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, wm[v * 16 + hc]);
    float O = 0.0f, L = 0.0f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float mv = wm[v * 16 + hc];
      const float wt = mv == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mv - M);
      O += wt * wo[(v * 16 + hc) * kHeadDim + d];
      L += wt * wl[v * 16 + hc];
    }
    // Partials are written with agent-scope stores, which go past this XCD's L2, so the
    // merging workgroup (possibly on another XCD) reads them without any L2 write-back.
    float *pp = part + hc * kPartialStride;
    __hip_atomic_store(pp + 4 + d, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == 0) {
      __hip_atomic_store(pp, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(pp + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ---- arrival; the last workgroup of this (batch, kv_head) merges every partial.
  // Every thread waits for its own partial stores to complete before the barrier; thread 0
  // then counts the arrival with an agent-scope atomic.  The merging workgroup reads the
  // partials with agent-scope loads issued after it has seen the final count.
  __shared__ int s_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t *cnt = a.counters + it.bh;
    uint64_t cur = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t next;
    for (;;) {
      next = ((uint32_t)(cur >> 32) == a.epoch) ? cur + 1 : (((uint64_t)a.epoch << 32) | 1u);
      if (__hip_atomic_compare_exchange_strong(cnt, &cur, next, __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        break;
    }
    s_last = (int)(uint32_t)next == a.items_total;
  }
  __syncthreads();
  if (!s_last) return;

  const int P = a.items_total;
  const float *parts = a.partials + (int64_t)it.bh * kMaxParts * G * kPartialStride;
  float *sm_m = (float *)smem;            // [P][G]
  float *sm_w = sm_m + P * G;             // [P][G] weights, after the max is known
  float *sm_l = sm_w + P * G;             // [P][G]
  float *sm_inv = sm_l + P * G;           // [G]
  for (int idx = threadIdx.x; idx < P * G; idx += kThreads) {
    const float *pp = parts + (int64_t)idx * kPartialStride;       // part idx / G, head idx % G
    sm_m[idx] = __hip_atomic_load(pp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm_l[idx] = __hip_atomic_load(pp + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int hc = threadIdx.x;
    float M = kNegInf;
    for (int p = 0; p < P; ++p) M = fmaxf(M, sm_m[p * G + hc]);
    float L = 0.0f;
    for (int p = 0; p < P; ++p) {
      const float mv = sm_m[p * G + hc];
      const float wt = mv == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mv - M);
      sm_w[p * G + hc] = wt;
      L += wt * sm_l[p * G + hc];
    }
    sm_inv[hc] = 1.0f / L;
  }
  __syncthreads();
  const int b = it.bh / a.H, h = it.bh % a.H;
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kThreads) {
    const int hc = idx >> 7, d = idx & 127;
    float O = 0.0f;
#pragma unroll 8
    for (int p = 0; p < P; ++p)
      O += sm_w[p * G + hc] * __hip_atomic_load(parts + (int64_t)(p * G + hc) * kPartialStride + 4 + d, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    const float r = O * sm_inv[hc];
    const int64_t o = ((int64_t)b * a.H * G + (int64_t)h * G + hc) * kHeadDim + d;
    if (a.out_fp32) ((float *)a.out)[o] = r;
    else ((_Float16 *)a.out)[o] = (_Float16)r;
  }
}

}  // namespace

size_t decode_lds_bytes(const DecodeArgs &a) {
  size_t ring = 0;
  for (int s = 0; s < a.nseg; ++s) {
    const int bb = (int)block_bytes(a.seg[s].fmt);
    ring = std::max(ring, (size_t)ring_depth(bb) * bb);
  }
  const size_t merge = (size_t)kWaves * (16 + 16 + 16 * kHeadDim) * sizeof(float);
  return std::max(ring, merge);
}

hipError_t launch_decode(const DecodeArgs &a, int num_wg, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)decode_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const size_t lds = decode_lds_bytes(a);
  decode_kernel<<<(unsigned)num_wg, kThreads, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvq
