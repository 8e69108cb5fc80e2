// Fused dequant + single-token decode attention of libkvq (gfx950).
//
// Every decode step reads the whole cached history (page "KV Cache量化实战：Model Optimizer
// 为大模型长上下文省下50%显存", section on why long context runs out of memory first) and the
// dequantized K/V take part in attention (page "NVFP4 KV缓存技术详解" §2.1).  The kernel
// streams the packed blocks once and dequantizes in registers; no fp16 copy of the cache is
// ever written.
//
// Work split (flash-decode): a work item is a run of 128-slot blocks of one tier (or the
// fp16 residual) of one (batch, kv_head); one 64-lane wave handles one item for all G query
// heads of that kv head (GQA grouping: each K/V byte is read once per group).  The item
// writes an unnormalised partial (m, l, o) in the log2 domain; a merge kernel combines the
// partials with a log-sum-exp reduction.
//
// Matrix cores: 32 slots per step.
//  QK^T  v_mfma_f32_16x16x32_f16, A = K (16 tokens x 32 dims), B = Q^T (32 dims x 16 heads,
//        heads >= G are zero).  Lane l (g = l/16, c = l%16) feeds token c of the tile and
//        receives logits of tokens 4g..4g+3 for head c.
//  PV    v_mfma_f32_16x16x32_f16 computing O^T, A = V^T (16 dims x 32 tokens), B = P (32
//        tokens x 16 heads); lane l feeds dim c of the 16-dim tile and the 8 tokens of lane
//        quarter g, and accumulates O^T[dims 4g..4g+3][head c] -- the same head as its logits.
// Affine K: the MFMA takes the exact integers (q - Z) as fp16 and S is applied per group
// after the dot.  Affine V: the MFMA takes (q - Z) and S is folded into P per group.
// NVFP4: E2M1 codes are converted by the hardware FP4->fp16 conversion and multiplied by
// the E4M3 scale, both exact in fp16 with a 2^-8 factor that is undone on the output.
#include "kvq_internal.h"

#include <cmath>

namespace kvq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -INFINITY;

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u(half2_t h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ half8_t pack8(half2_t a, half2_t b, half2_t c, half2_t d) {
  half8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// (1024 + c_lo, 1024 + c_hi) as fp16 from the n-bit fields at bit `sh` of both halves.
template <int NB>
__device__ __forceinline__ half2_t magic_pair(uint32_t w, int sh) {
  constexpr uint32_t mask = ((1u << NB) - 1) * 0x00010001u;
  return as_h2(((w >> sh) & mask) | 0x64006400u);
}

// fp16 bits of (E4M3 value) * 2^-8 for the two bytes held in bits 0-7 and 16-23 of x.
__device__ __forceinline__ half2_t e4m3_pair_scaled(uint32_t x) {
  return as_h2(((x & 0x007F007Fu) << 7) | ((x & 0x00800080u) << 8));
}

__device__ __forceinline__ float wave_max_lanes16(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float wave_sum_lanes16(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Running softmax state of one lane: head c, its O^T accumulators for dims 16k + 4g + i.
struct State {
  float m = kNegInf, l = 0.0f;
  float4_t o[8];
};

// Online softmax update for 8 logits (two 16-token tiles, tokens 4g+i of each) and the
// probabilities p that feed the PV product.
__device__ __forceinline__ void softmax_step(State &st, float (&s)[8], float (&p)[8]) {
  float mt = s[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mt = fmaxf(mt, s[i]);
  mt = wave_max_lanes16(mt);
  const float m_new = fmaxf(st.m, mt);
  const bool none = m_new == kNegInf;
  const float alpha = none ? 1.0f : exp2f(st.m - m_new);
  st.l *= alpha;
#pragma unroll
  for (int k = 0; k < 8; ++k) st.o[k] *= alpha;
  st.m = m_new;
  float ls = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = none ? 0.0f : exp2f(s[i] - m_new);
    ls += p[i];
  }
  st.l += ls;
}

__device__ __forceinline__ float4_t mfma32(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ Q operands per format
// Dims that k-step j (of 4) feeds from lane quarter g, in the order the K unpack produces.
template <int FMT>
__device__ __forceinline__ int q_dim(int g, int j, int e) {
  if constexpr (FMT == kFmtInt4) {
    // step j: group j/2, dims 64*(j/2) + 16g + 8*(j%2) + [0,4,1,5,2,6,3,7][e]
    const int perm = (e & 1) * 4 + (e >> 1);
    return 64 * (j >> 1) + 16 * g + 8 * (j & 1) + perm;
  } else if constexpr (FMT == kFmtInt2) {
    // one 32-bit word = dims 64*(j/2) + 16g + 0..15; pairs (c_s, c_{s+8}), step uses s = 4*(j%2) + 0..3
    const int s = 4 * (j & 1) + (e >> 1);
    return 64 * (j >> 1) + 16 * g + s + 8 * (e & 1);
  } else if constexpr (FMT == kFmtInt8) {
    // two words per step; per word pairs (b0,b2), (b1,b3)
    const int w = e >> 2, ee = e & 3;
    const int perm = (ee & 1) * 2 + (ee >> 1);
    return 64 * (j >> 1) + 16 * g + 8 * (j & 1) + 4 * w + perm;
  } else {
    // NVFP4 and fp16: dims 32g + 8j + e in natural order
    return 32 * g + 8 * j + e;
  }
}

template <int FMT>
__device__ __forceinline__ void load_q(const uint16_t *qrow, bool valid, int g, half8_t (&qb)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) qb[j][e] = valid ? __builtin_bit_cast(_Float16, qrow[q_dim<FMT>(g, j, e)]) : (_Float16)0.0f;
}

// ------------------------------------------------------------------ affine step (32 slots)
template <int NB>
__device__ __forceinline__ void affine_step(const uint8_t *blk, int u, int64_t slot_base, int64_t ntok, int g, int c,
                                            const half8_t (&qb)[4], float scale_log2, State &st) {
  constexpr int kRow = 16 * NB;
  const uint8_t *km = blk + aff_km(NB);
  float s[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tau = 2 * u + tt;
    const int t = 16 * tau + c;                              // token this lane feeds
    const uint8_t *row = blk + t * kRow;
    const uint2 meta = *(const uint2 *)(km + t * 8);         // S0 Z0 S1 Z1
    float4_t acc[2];
#pragma unroll
    for (int gr = 0; gr < 2; ++gr) {
      const uint16_t zb = (uint16_t)(gr ? (meta.y >> 16) : (meta.x >> 16));
      const _Float16 zc = (_Float16)(1024.0f + h2f(zb));
      const half2_t zc2 = {zc, zc};
      half8_t a[2];
      if constexpr (NB == 4) {
        const uint2 w = *(const uint2 *)(row + 32 * gr + 8 * g);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint32_t x = hh ? w.y : w.x;
          a[hh] = pack8(magic_pair<4>(x, 0) - zc2, magic_pair<4>(x, 4) - zc2, magic_pair<4>(x, 8) - zc2, magic_pair<4>(x, 12) - zc2);
        }
      } else if constexpr (NB == 2) {
        const uint32_t x = *(const uint32_t *)(row + 16 * gr + 4 * g);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          a[hh] = pack8(magic_pair<2>(x, 8 * hh + 0) - zc2, magic_pair<2>(x, 8 * hh + 2) - zc2,
                        magic_pair<2>(x, 8 * hh + 4) - zc2, magic_pair<2>(x, 8 * hh + 6) - zc2);
      } else {
        const uint4 w = *(const uint4 *)(row + 64 * gr + 16 * g);
        a[0] = pack8(magic_pair<8>(w.x, 0) - zc2, magic_pair<8>(w.x, 8) - zc2, magic_pair<8>(w.y, 0) - zc2, magic_pair<8>(w.y, 8) - zc2);
        a[1] = pack8(magic_pair<8>(w.z, 0) - zc2, magic_pair<8>(w.z, 8) - zc2, magic_pair<8>(w.w, 0) - zc2, magic_pair<8>(w.w, 8) - zc2);
      }
      float4_t z4 = {0.0f, 0.0f, 0.0f, 0.0f};
      z4 = mfma32(a[0], qb[2 * gr + 0], z4);
      acc[gr] = mfma32(a[1], qb[2 * gr + 1], z4);
    }
    // logits of tokens 16*tau + 4g + i for head c: sum over groups of S * dot
    const uint4 m0 = *(const uint4 *)(km + (16 * tau + 4 * g) * 8);
    const uint4 m1 = *(const uint4 *)(km + (16 * tau + 4 * g) * 8 + 16);
    const uint32_t mw[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float S0 = h2f((uint16_t)(mw[2 * i] & 0xFFFF)), S1 = h2f((uint16_t)(mw[2 * i + 1] & 0xFFFF));
      const float v = (S0 * acc[0][i] + S1 * acc[1][i]) * scale_log2;
      const int64_t slot = slot_base + 16 * tau + 4 * g + i;
      s[4 * tt + i] = slot < ntok ? v : kNegInf;
    }
  }
  float p[8];
  softmax_step(st, s, p);

  // P folded with the V scale of each group; Z pairs of the lane's 8 tokens per group
  const uint8_t *vm = blk + aff_vm(NB);
  half8_t pb[2];
  half2_t zc[2][4];
#pragma unroll
  for (int gr = 0; gr < 2; ++gr) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint4 e = *(const uint4 *)(vm + ((gr * 4 + g) * 8 + 2 * u + tt) * 16);
      const uint32_t sw[2] = {e.x, e.y};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float S = h2f((uint16_t)((sw[i >> 1] >> (16 * (i & 1))) & 0xFFFF));
        pb[gr][4 * tt + i] = (_Float16)(p[4 * tt + i] * S);
      }
      const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
      zc[gr][2 * tt + 0] = as_h2(e.z) + k1024;
      zc[gr][2 * tt + 1] = as_h2(e.w) + k1024;
    }
  }
  const uint8_t *vc = blk + aff_vc(NB);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int gr = k >> 2;
    const uint8_t *vrow = vc + (16 * k + c) * kRow + g * (4 * NB);   // lane quarter of the dim row
    half8_t a;
    if constexpr (NB == 4) {
      const uint32_t x = *(const uint32_t *)(vrow + 4 * u);
      a = pack8(magic_pair<4>(x, 0) - zc[gr][0], magic_pair<4>(x, 4) - zc[gr][1], magic_pair<4>(x, 8) - zc[gr][2],
                magic_pair<4>(x, 12) - zc[gr][3]);
    } else if constexpr (NB == 2) {
      const uint32_t x = *(const uint32_t *)(vrow + 4 * (u >> 1));
      const int sh = 8 * (u & 1);
      a = pack8(magic_pair<2>(x, sh + 0) - zc[gr][0], magic_pair<2>(x, sh + 2) - zc[gr][1],
                magic_pair<2>(x, sh + 4) - zc[gr][2], magic_pair<2>(x, sh + 6) - zc[gr][3]);
    } else {
      const uint2 x = *(const uint2 *)(vrow + 8 * u);
      a = pack8(magic_pair<8>(x.x, 0) - zc[gr][0], magic_pair<8>(x.x, 8) - zc[gr][1], magic_pair<8>(x.y, 0) - zc[gr][2],
                magic_pair<8>(x.y, 8) - zc[gr][3]);
    }
    st.o[k] = mfma32(a, pb[gr], st.o[k]);
  }
}

// ------------------------------------------------------------------ NVFP4 step (32 slots)
template <int BYTE>
__device__ __forceinline__ half2_t fp4_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, BYTE);
}

__device__ __forceinline__ void nvfp4_step(const uint8_t *blk, int u, int64_t slot_base, int64_t ntok, int g, int c,
                                           const half8_t (&qb)[4], float scale_log2, State &st) {
  float s[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tau = 2 * u + tt;
    const int t = 16 * tau + c;
    const uint4 w = *(const uint4 *)(blk + t * 64 + 16 * g);                 // dims 32g .. 32g+31
    const uint32_t sb = *(const uint16_t *)(blk + kNvKs + t * 8 + 2 * g);    // scales of blocks 2g, 2g+1
    const half2_t sc0 = e4m3_pair_scaled((sb & 0xFF) * 0x00010001u);
    const half2_t sc1 = e4m3_pair_scaled((sb >> 8) * 0x00010001u);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const half2_t sc = j < 2 ? sc0 : sc1;
      const half8_t a = pack8(fp4_pair<0>(ws[j]) * sc, fp4_pair<1>(ws[j]) * sc, fp4_pair<2>(ws[j]) * sc, fp4_pair<3>(ws[j]) * sc);
      acc = mfma32(a, qb[j], acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t slot = slot_base + 16 * tau + 4 * g + i;
      s[4 * tt + i] = slot < ntok ? acc[i] * (scale_log2 * 256.0f) : kNegInf;
    }
  }
  float p[8];
  softmax_step(st, s, p);
  // B operand order follows the FP4 byte pairs of the V word: tokens (tau, i) =
  // (2u,0) (2u,2) (2u+1,0) (2u+1,2) (2u,1) (2u,3) (2u+1,1) (2u+1,3)
  half8_t pb;
  pb[0] = (_Float16)p[0]; pb[1] = (_Float16)p[2]; pb[2] = (_Float16)p[4]; pb[3] = (_Float16)p[6];
  pb[4] = (_Float16)p[1]; pb[5] = (_Float16)p[3]; pb[6] = (_Float16)p[5]; pb[7] = (_Float16)p[7];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t x = *(const uint32_t *)(blk + kNvVc + (16 * k + c) * 64 + 16 * g + 4 * u);
    const uint2 sv = *(const uint2 *)(blk + kNvVs + k * 128 + 32 * g + 8 * u);   // scales (2u,0..3) (2u+1,0..3)
    const half2_t s02 = e4m3_pair_scaled(sv.x & 0x00FF00FFu);
    const half2_t s13 = e4m3_pair_scaled((sv.x >> 8) & 0x00FF00FFu);
    const half2_t s46 = e4m3_pair_scaled(sv.y & 0x00FF00FFu);
    const half2_t s57 = e4m3_pair_scaled((sv.y >> 8) & 0x00FF00FFu);
    const half8_t a = pack8(fp4_pair<0>(x) * s02, fp4_pair<1>(x) * s46, fp4_pair<2>(x) * s13, fp4_pair<3>(x) * s57);
    st.o[k] = mfma32(a, pb, st.o[k]);
  }
}

// ------------------------------------------------------------------ fp16 residual step (32 slots)
__device__ __forceinline__ void fp16_step(const uint8_t *res, int R, int u, int64_t ntok, int g, int c,
                                          const half8_t (&qb)[4], float scale_log2, State &st) {
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
      for (int j = 0; j < 4; ++j) acc = mfma32(__builtin_bit_cast(half8_t, row[j]), qb[j], acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t slot = 16 * tau + 4 * g + i;
      s[4 * tt + i] = (tau < ntiles && slot < ntok) ? acc[i] * scale_log2 : kNegInf;
    }
  }
  float p[8];
  softmax_step(st, s, p);
  half8_t pb;
#pragma unroll
  for (int i = 0; i < 8; ++i) pb[i] = (_Float16)p[i];
  const uint8_t *vres = res + (int64_t)R * 256;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int d = 16 * k + c;
    half4_t v[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tau = 2 * u + tt;
      v[tt] = half4_t{0, 0, 0, 0};
      if (tau < ntiles) {
        const uint2 x = *(const uint2 *)(vres + ((tau * kHeadDim + d) * 16 + 4 * g) * 2);
        v[tt] = __builtin_bit_cast(half4_t, x);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * tau + 4 * g + i >= ntok) v[tt][i] = (_Float16)0.0f;   // slots past r may hold stale bits
      }
    }
    half8_t a;
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = v[0][i]; a[4 + i] = v[1][i]; }
    st.o[k] = mfma32(a, pb, st.o[k]);
  }
}

// ------------------------------------------------------------------ partial kernel
template <int FMT>
__global__ __launch_bounds__(64) void decode_partial_kernel(DecodeArgs a, DecodeSeg seg) {
  const int item = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, g = lane >> 4, c = lane & 15;
  const int G = a.G, Hq = a.H * a.G;
  const bool head_ok = c < G;
  const uint16_t *qrow = a.q + ((int64_t)b * Hq + h * G + c) * kHeadDim;
  half8_t qb[4];
  load_q<FMT>(qrow, head_ok, g, qb);

  State st;
#pragma unroll
  for (int k = 0; k < 8; ++k) st.o[k] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const uint8_t *bh = seg.base + ((int64_t)b * a.H + h) * seg.bh_stride;
  float out_scale = 1.0f;
  if constexpr (FMT == kFmtFp16) {
    const int nsteps = (int)((seg.ntok + 31) / 32);
    for (int u = 0; u < nsteps; ++u) fp16_step(bh, seg.res_len, u, seg.ntok, g, c, qb, a.scale_log2, st);
  } else {
    const int64_t nblk = (seg.ntok + kBlock - 1) / kBlock;
    const int64_t blk_lo = (int64_t)item * seg.units_per_item;
    const int64_t blk_hi = min(nblk, blk_lo + seg.units_per_item);
    for (int64_t bi = blk_lo; bi < blk_hi; ++bi) {
      const uint8_t *blk = bh + bi * (int64_t)block_bytes(FMT);
      const int64_t slot_base = bi * kBlock;
#pragma unroll 1
      for (int u = 0; u < 4; ++u) {
        if constexpr (FMT == kFmtNvfp4) nvfp4_step(blk, u, slot_base, seg.ntok, g, c, qb, a.scale_log2, st);
        else affine_step<FMT>(blk, u, slot_base, seg.ntok, g, c, qb, a.scale_log2, st);
      }
    }
    if constexpr (FMT == kFmtNvfp4) out_scale = 256.0f;
  }
  const float l = wave_sum_lanes16(st.l);
  if (head_ok) {
    float *dst = a.partials + (((int64_t)(seg.item0 + item) * a.B + b) * Hq + h * G + c) * kPartialStride;
    if (g == 0) { dst[0] = st.m; dst[1] = l; }
#pragma unroll
    for (int k = 0; k < 8; ++k) *(float4_t *)(dst + 4 + 16 * k + 4 * g) = st.o[k] * out_scale;
  }
}

// ------------------------------------------------------------------ merge kernel
__global__ __launch_bounds__(128) void merge_kernel(DecodeArgs a, void *out, int out_fp32) {
  const int bq = blockIdx.x;              // b * Hq + hq
  const int d = threadIdx.x;
  const int Hq = a.H * a.G;
  const int64_t stride = (int64_t)a.B * Hq * kPartialStride;
  const float *p = a.partials + (int64_t)bq * kPartialStride;
  float m = kNegInf;
  for (int i = 0; i < a.n_items_total; ++i) m = fmaxf(m, p[i * stride]);
  float num = 0.0f, den = 0.0f;
  for (int i = 0; i < a.n_items_total; ++i) {
    const float *pi = p + i * stride;
    const float mi = pi[0];
    const float w = mi == kNegInf ? 0.0f : exp2f(mi - m);
    den += w * pi[1];
    num += w * pi[4 + d];
  }
  const float r = num / den;
  if (out_fp32) ((float *)out)[(int64_t)bq * kHeadDim + d] = r;
  else ((_Float16 *)out)[(int64_t)bq * kHeadDim + d] = (_Float16)r;
}

}  // namespace

hipError_t launch_decode_segment(const DecodeArgs &a, const DecodeSeg &seg, hipStream_t s) {
  dim3 grid((unsigned)seg.n_items, (unsigned)a.H, (unsigned)a.B);
  switch (seg.fmt) {
    case kFmtInt2: decode_partial_kernel<kFmtInt2><<<grid, 64, 0, s>>>(a, seg); break;
    case kFmtInt4: decode_partial_kernel<kFmtInt4><<<grid, 64, 0, s>>>(a, seg); break;
    case kFmtInt8: decode_partial_kernel<kFmtInt8><<<grid, 64, 0, s>>>(a, seg); break;
    case kFmtNvfp4: decode_partial_kernel<kFmtNvfp4><<<grid, 64, 0, s>>>(a, seg); break;
    case kFmtFp16: decode_partial_kernel<kFmtFp16><<<grid, 64, 0, s>>>(a, seg); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const DecodeArgs &a, void *out, int out_fp32, hipStream_t s) {
  merge_kernel<<<(unsigned)(a.B * a.H * a.G), kHeadDim, 0, s>>>(a, out, out_fp32);
  return hipGetLastError();
}

}  // namespace kvq
