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
// Affine: the MFMA takes the raw codes as fp16 subnormals (c * 2^-24, some scaled by 16 for
// INT4, by 4 for INT2).  K:
// logit = S0 (dot0 - Z0 qsum0) + S1 (dot1 - Z1 qsum1) per 64-dim group, in units of 2^-24.  V:
// the scale S of each (slot, group) is folded into P and the zero point enters as
// o = 2^24 o - sum_t P'_t Z_t at the end of the work item.
// NVFP4: E2M1 codes and E4M3 scales are converted by the hardware to fp16 and multiplied
// (exact: at most 6 significant bits, magnitude in [2^-10, 2688]).
#include "kvq_internal.h"
#include "kvq_fp_codes.h"
#include "kvq_rescopy.h"

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
// Formats whose P operand is p itself (NVFP4, MXFP4, FP8, FP16) keep their reference max until
// a logit exceeds it by 2^8 in p: the state is rescaled about once per work item instead of at
// most blocks of a short item, and P <= 256 stays exact in fp16 range (products with V codes
// at most 65504 * 256 in fp32).  Affine formats fold S into P' = p S, so their slack is 0.
constexpr float kSlackLog2 = 8.0f;

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u(half2_t h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ half8_t h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(half8_t, u32x4{a, b, c, d});
}
__device__ __forceinline__ uint32_t pk(float a, float b) { return as_u(half2_t{(_Float16)a, (_Float16)b}); }

__device__ __forceinline__ float4_t mfma(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ half4_t h4(uint32_t a, uint32_t b) { return __builtin_bit_cast(half4_t, u32x2{a, b}); }
__device__ __forceinline__ float4_t mfma16(half4_t a, half4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
// PV over both 16-slot subtiles of a wave in one 16x16x32 step: k element e of lane quarter g
// is slot 4g + (e & 3) of subtile e >> 2, so A = (codes of subtile 0, codes of subtile 1) and
// B = the lane's P where its column's subtile matches (zeros in the other half).
__device__ __forceinline__ float4_t mfma_pv2(half4_t a0, half4_t a1, half4_t b0, half4_t b1, float4_t c) {
  return mfma(__builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7), __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7), c);
}

// fp16 pair (1024 + f_lo, 1024 + f_hi) of the two fields selected by mask, minus 1024 + off:
// exact (f - off, or 16 f - off for a mask shifted by 4 bits).
// ---------------------------------------------------------------- operand unpack per format
// Affine codes enter the MFMA as fp16 subnormals: the 16-bit halves of (x & mask) are the raw
// codes c, i.e. the values c * 2^-24 (16 c * 2^-24 for a mask shifted by 4 bits), which the
// matrix core multiplies exactly.  One v_and per pair; the factor 2^24 is carried by the
// softmax scale and removed from the PV sums once per work item.
// INT4 word -> [n0, n4, 16n1, 16n5, n2, n6, 16n3, 16n7] * 2^-24 (n_v = nibble v)
__device__ __forceinline__ half8_t unpack_int4(uint32_t x) {
  const uint32_t y = x >> 8;
  return h8(x & 0x000F000Fu, x & 0x00F000F0u, y & 0x000F000Fu, y & 0x00F000F0u);
}
// INT2 word -> lo = crumbs [c0, c8, 4c1, 4c9, c2, c10, 4c3, 4c11] * 2^-24, hi = the same for
// crumbs 4..7 / 12..15: the odd crumb of each nibble is masked in place (times 4), as INT4's
// high nibble is taken times 16, so the scaled elements sit where INT4's do (3 shifts and 8
// ands per word instead of 7 and 8)
__device__ __forceinline__ void unpack_int2(uint32_t x, half8_t &lo, half8_t &hi) {
  const uint32_t x4 = x >> 4, x8 = x >> 8, x12 = x >> 12;
  lo = h8(x & 0x00030003u, x & 0x000C000Cu, x4 & 0x00030003u, x4 & 0x000C000Cu);
  hi = h8(x8 & 0x00030003u, x8 & 0x000C000Cu, x12 & 0x00030003u, x12 & 0x000C000Cu);
}
// INT2 K word with per-token groups -> the same crumbs in the same order as unpack_int2, with
// the three crumbs in bits 0..5 of each half masked in place (times 1, 4, 16), the next three
// after one shift by 6, the last two after a shift by 12 (2 shifts and 8 ands per word):
// lo = [c0, c8, 4c1, 4c9, 16c2, 16c10, c3, c11], hi = [4c4, 4c12, 16c5, 16c13, c6, c14, 4c7, 4c15]
// (factors at most 16 apart within one MFMA operand, as INT4's)
__device__ __forceinline__ void unpack_int2_k(uint32_t x, half8_t &lo, half8_t &hi) {
  const uint32_t x6 = x >> 6, x12 = x >> 12;
  lo = h8(x & 0x00030003u, x & 0x000C000Cu, x & 0x00300030u, x6 & 0x00030003u);
  hi = h8(x6 & 0x000C000Cu, x6 & 0x00300030u, x12 & 0x00030003u, x12 & 0x000C000Cu);
}
// log2 of the factor that the scaled A elements carry (INT4 16, INT2 4; none for the others)
template <int FMT>
constexpr int kSh = FMT == kFmtInt4 ? 4 : FMT == kFmtInt2 ? 2 : 0;
// log2 of the factor of K operand element e of the word's first (hh = 0) or second (hh = 1)
// operand: INT2 with per-token groups as unpack_int2_k; otherwise (e >> 1) odd: INT4 4, INT2
// 2, else 0
template <int FMT, int GS>
__device__ __forceinline__ constexpr int k_elem_sh(int hh, int e) {
  if constexpr (FMT == kFmtInt2 && GS != kKc) {
    constexpr int lo_sh[4] = {0, 2, 4, 0}, hi_sh[4] = {2, 4, 0, 2};
    return hh ? hi_sh[e >> 1] : lo_sh[e >> 1];
  }
  return ((e >> 1) & 1) ? kSh<FMT> : 0;
}
// INT8 word pair -> [w0.b0, w0.b2, w0.b1, w0.b3, w1.b0, w1.b2, w1.b1, w1.b3]
__device__ __forceinline__ half8_t unpack_int8(uint32_t w0, uint32_t w1) {
  return h8(w0 & 0x00FF00FFu, (w0 >> 8) & 0x00FF00FFu, w1 & 0x00FF00FFu, (w1 >> 8) & 0x00FF00FFu);
}
constexpr float kSub = 5.9604644775390625e-08f;   // 2^-24, the value of fp16 bit pattern 1
constexpr float kInvSub = 16777216.0f;            // 2^24
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

// MXFP4 scales.  The scaled conversion multiplies by 2^(e - 127), e the exponent field of its
// f32 scale, and reads no other bit of it (measured over every exponent 101..140, the range of
// fp16 data, with sign and mantissa bits set and clear); the products are exact, subnormal fp16
// results included.  So an E8M0 byte only has to be moved into bits 23..30: one shift, whatever
// lands in the other bits.
__device__ __forceinline__ float e8m0_f32(uint32_t d, int k) {
  return __uint_as_float(k == 3 ? d >> 1 : d << (23 - 8 * k));
}
// 8 E2M1 codes of one word (nibble order) times the power-of-two scale X
__device__ __forceinline__ half8_t unpack_mx(uint32_t x, float X) {
  return h8(as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, X, 0)), as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, X, 1)),
            as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, X, 2)), as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, X, 3)));
}
// MXFP4 V of dim block m: byte 8m + e of the lane string holds slot e at dims 16(2m) + c (low
// nibble) and 16(2m+1) + c (high nibble), under the slot's own scale.  Each byte converts under
// its scale into (tile 2m, tile 2m+1) of slot e; byte permutes regroup the halves into the
// operands of tile 2m (lo[0..3]: slots (0,1), (2,3), (4,5), (6,7)) and tile 2m+1 (hi[0..3]).
__device__ __forceinline__ void mx_v_tiles(uint32_t x0, uint32_t x1, uint32_t s0, uint32_t s1, uint32_t (&lo)[4],
                                           uint32_t (&hi)[4]) {
  uint32_t r[8];
  r[0] = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x0, e8m0_f32(s0, 0), 0));
  r[1] = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x0, e8m0_f32(s0, 1), 1));
  r[2] = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x0, e8m0_f32(s0, 2), 2));
  r[3] = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x0, e8m0_f32(s0, 3), 3));
  r[4] = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x1, e8m0_f32(s1, 0), 0));
  r[5] = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x1, e8m0_f32(s1, 1), 1));
  r[6] = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x1, e8m0_f32(s1, 2), 2));
  r[7] = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x1, e8m0_f32(s1, 3), 3));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[i] = __builtin_amdgcn_perm(r[2 * i + 1], r[2 * i], 0x05040100u);
    hi[i] = __builtin_amdgcn_perm(r[2 * i + 1], r[2 * i], 0x07060302u);
  }
}

// FP8 word pair -> the 8 values in byte order [w0.b0, w0.b1, w0.b2, w0.b3, w1.b0, ..., w1.b3]
__device__ __forceinline__ half8_t unpack_fp8(uint32_t w0, uint32_t w1) {
  return h8(e4m3_pair(w0, false), e4m3_pair(w0, true), e4m3_pair(w1, false), e4m3_pair(w1, true));
}

// ---------------------------------------------------------------- cross-quarter reductions
// Reduce over lanes {c, c+16, c+32, c+48} (the four lane quarters holding one head).  The
// partner values come from the lane-swap instructions (v_permlane16_swap / v_permlane32_swap:
// with both operands x, the two results hold x of rows (0, 1) or (2, 3), resp. of halves
// (lo, hi), on every lane), so no LDS round trip; both results enter in the same order on every
// lane, so all lanes of a head get the same bits.
__device__ __forceinline__ void xor16_pair(float x, float &a, float &b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void xor32_pair(float x, float &a, float &b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float quad_max(float x) {
  float a, b;
  xor16_pair(x, a, b);
  xor32_pair(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float quad_sum(float x) {
  float a, b;
  xor16_pair(x, a, b);
  xor32_pair(a + b, a, b);
  return a + b;
}
// Value of lane c ^ 8 within the lane's row of 16 (DPP row rotation by 8).
__device__ __forceinline__ float row_xor8(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
}
// Over all 64 lanes (the final merge, once per (batch, kv_head) and call): DPP rotations by
// 8, 4, 2 and 1 within each row of 16, then the two lane swaps.  Every lane gets the max; for
// the sum the lanes of a row add in different orders, and lane 0's value is the one used.
__device__ __forceinline__ float row_ror(float x, int k) {
  switch (k) {
    case 8: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
    case 4: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, false));
    case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x122, 0xF, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x121, 0xF, 0xF, false));
  }
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int k = 8; k >= 1; k >>= 1) x = fmaxf(x, row_ror(x, k));
  return quad_max(x);
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int k = 8; k >= 1; k >>= 1) x += row_ror(x, k);
  return quad_sum(x);
}
// Over the eight lanes {c, c^8} x quarters that hold one head in the paired-subtile layout.
__device__ __forceinline__ float head_max2(float x) { return quad_max(fmaxf(x, row_xor8(x))); }
__device__ __forceinline__ float head_sum2(float x) { return quad_sum(x + row_xor8(x)); }

// ---------------------------------------------------------------- Q operand per format
// Dim fed by B element e of k-step j in lane quarter g, and the log2 sh of the factor the A
// element it meets carries (then B holds q / 2^sh).
template <int FMT, int GS>
__device__ __forceinline__ int q_dim(int g, int j, int e, int &sh) {
  const int G = j >> 1, h = j & 1;
  sh = k_elem_sh<FMT, GS>(h, e);
  if constexpr (is_affine(FMT) && GS == 32) {
    return 32 * j + 8 * g + e;   // groups of 32: k-step j feeds dims 32j + 8g .. +7 (group j)
  } else if constexpr (FMT == kFmtInt4) {
    return 64 * G + 16 * g + 8 * h + (e >> 1) + 4 * (e & 1);
  } else if constexpr (FMT == kFmtInt2) {
    return 64 * G + 16 * g + 4 * h + (e >> 1) + 8 * (e & 1);
  } else if constexpr (FMT == kFmtInt8) {
    return 64 * G + 16 * g + 4 * (2 * h + (e >> 2)) + ((e >> 1) & 1) + 2 * (e & 1);
  } else if constexpr (FMT == kFmtFp8) {
    return 64 * G + 16 * g + 8 * h + e;   // INT8 lane fields, converted in byte order
  } else {
    return 32 * g + 8 * j + e;   // NVFP4 and the fp16 residual: natural order
  }
}

// Affine group of MFMA k-step j (groups of 32: one per step; 64: steps 2G, 2G + 1; 128: all)
// and of V dim tile k (dims 16k .. 16k + 15).
// (kKc, per-channel K, has V groups of 64 and no K groups along head_dim.)
template <int GS>
__device__ __forceinline__ constexpr int k_group(int j) { return GS == 32 ? j : (GS == 64 || GS == kKc) ? j >> 1 : 0; }
template <int GS>
__device__ __forceinline__ constexpr int v_group(int k) { return GS == 32 ? k >> 1 : (GS == 64 || GS == kKc) ? k >> 2 : 0; }
template <int GS>
constexpr int kGroups = GS == kKc ? 2 : kHeadDim / GS;   // per-token groups along head_dim

// INT4 and INT2 meet half of the query row with codes taken times 2^kSh (the masked high
// fields), so that half enters the MFMA as q / 2^kSh.  Divided as it stands, a query entry
// below 2^(kSh - 14) would become an fp16 subnormal and lose relative precision (the oracle
// uses q exactly).  So each head's row is first scaled by a power of two 2^t that puts its
// largest magnitude M into [2^14, 2^15): every entry >= M 2^-24 then keeps its full fp16
// precision after the division, and smaller ones are off by at most M 2^-35 (both roundings
// are exact otherwise: a power-of-two scaling).  The logits come out 2^t larger, which the
// softmax scale and the max take back (t >= 0 keeps every entry finite).  Per-channel K
// multiplies q by the block's per-dim S first, where no fixed shift is safe from overflow.
template <int FMT, int GS>
constexpr bool kQShift = kSh<FMT> != 0 && GS != kKc;
// 2^t for a row maximum M (the same on every lane of the head: M is reduced over them)
__device__ __forceinline__ float q_shift_scale(float M) {
  if (!(M > 0.0f)) return 1.0f;
  const int E = (int)((__float_as_uint(M) >> 23) & 0xFFu) - 127;   // M = 2^E (1 + f), normal in fp32
  const int t = max(0, 14 - E);
  return __uint_as_float((uint32_t)(127 + t) << 23);
}

// The 32 dims a lane quarter g feeds: affine formats (groups of 64 or 128) and FP8 dims
// 16g..16g+15 and 64+16g..64+16g+15 (local index 16G + m); affine groups of 32 dims 32j + 8g
// .. +7 (local index 8j + m); NVFP4 and fp16 dims 32g..32g+31 (local index dim - 32g).
template <int FMT, int GS>
__device__ __forceinline__ void load_q(const uint16_t *qrow, bool valid, int g, half8_t (&qb)[4], float (&qs)[4],
                                       float &qscale) {
  constexpr bool kLay32 = is_affine(FMT) && GS == 32;
  constexpr bool kLay64 = !kLay32 && (is_affine(FMT) || FMT == kFmtFp8);
  uint4 raw[4];
  if constexpr (kLay32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) raw[j] = *(const uint4 *)(qrow + 32 * j + 8 * g);
  } else if constexpr (kLay64) {
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
  qscale = 1.0f;
  if constexpr (kQShift<FMT, GS>) {
    _Float16 mh = (_Float16)0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) mh = __builtin_fmaxf16(mh, __builtin_fabsf16(loc[i]));
    qscale = q_shift_scale(quad_max((float)mh));   // the four quarters hold the head's 128 dims
  }
#pragma unroll
  for (int G = 0; G < 4; ++G) qs[G] = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int sh;
      const int d = q_dim<FMT, GS>(g, j, e, sh);
      const int li = kLay32 ? 8 * (d >> 5) + (d & 7) : kLay64 ? 16 * (d >> 6) + (d & 15) : d - 32 * g;
      _Float16 v = loc[li];
      if constexpr (kQShift<FMT, GS>) v = (_Float16)((float)v * (qscale * (1.0f / (float)(1 << sh))));
      else if (sh) v = v * (_Float16)(1.0f / (float)(1 << sh));
      qb[j][e] = v;
      const float eff = (float)(1 << sh) * (float)v;    // the q the MFMA effectively uses
      qs[k_group<GS>(j)] += eff;
    }
  }
  // group sums over the four lane quarters (lanes c, c+16, c+32, c+48 hold one head), in the
  // 2^-24 units of the subnormal code operands
#pragma unroll
  for (int G = 0; G < kGroups<GS>; ++G) qs[G] = quad_sum(qs[G]) * kSub;
}

// ---------------------------------------------------------------- LDS DMA
// 16 bytes per lane from global sbase + voff (wave-uniform 64-bit base in scalar registers,
// per-lane 32-bit offset) to LDS address lds + 16 * lane (wave-uniform lds).  With the base in
// scalar registers the per-block address arithmetic is scalar work, not three vector
// instructions per load.  M0 is saved and restored around the load so the compiler's use of
// it is undisturbed.  The cache bytes are read once per call: the load carries the
// nontemporal policy (nt), with which a plain read stream of 4 GiB ran at 6.4-6.5 TB/s against
// 5.6-6.0 TB/s without.
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

// N (1..4) chunk loads of one wave as dma16, chunk t from sbase + t * STRIDE to LDS lds + t *
// STRIDE, with M0 saved once and restored once around all of them
template <int N, int STRIDE>
__device__ __forceinline__ void dma16_run(const uint8_t *sbase, uint32_t voff, uint32_t lds) {
  static_assert(N >= 1 && N <= 4, "one to four chunks");
  const uint8_t *s1 = sbase + STRIDE, *s2 = sbase + 2 * STRIDE, *s3 = sbase + 3 * STRIDE;
  const uint32_t l1 = lds + STRIDE, l2 = lds + 2 * STRIDE, l3 = lds + 3 * STRIDE;
  uint32_t saved;
  if constexpr (N == 1) {
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds)
        : "memory");
  } else if constexpr (N == 2) {
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %4 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds), "s"(s1), "s"(l1)
        : "memory");
  } else if constexpr (N == 3) {
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %4 nt\n\t"
        "s_mov_b32 m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %6 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds), "s"(s1), "s"(l1), "s"(s2), "s"(l2)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %4 nt\n\t"
        "s_mov_b32 m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %6 nt\n\t"
        "s_mov_b32 m0, %9\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %8 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds), "s"(s1), "s"(l1), "s"(s2), "s"(l2), "s"(s3), "s"(l3)
        : "memory");
  }
}

// N (1..8) chunk loads as dma16_run, in statements of four
template <int N, int STRIDE>
__device__ __forceinline__ void dma16_runs(const uint8_t *sbase, uint32_t voff, uint32_t lds) {
  if constexpr (N <= 4) {
    dma16_run<N, STRIDE>(sbase, voff, lds);
  } else {
    dma16_run<4, STRIDE>(sbase, voff, lds);
    dma16_run<N - 4, STRIDE>(sbase + 4 * STRIDE, voff, lds + 4 * STRIDE);
  }
}

// vmcnt(N) for a count known at compile time
template <int N>
__device__ __forceinline__ void wait_vmcnt_c() {
  static_assert(N >= 0 && N <= 63, "the vmcnt field holds 0..63");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
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
    case 20: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
    case 21: asm volatile("s_waitcnt vmcnt(21)" ::: "memory"); break;
    case 22: asm volatile("s_waitcnt vmcnt(22)" ::: "memory"); break;
    case 23: asm volatile("s_waitcnt vmcnt(23)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;   // never weaker than asked
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
  float m = kNegInf;   // reference max of the unscaled logits of head c, same on the 4 lane quarters
  float slack = 0.0f;  // logits up to m + slack keep the reference (p <= 2^kSlackLog2 then)
  float l = 0.0f;      // this lane's share of sum p
  float z[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};   // affine V: this lane's share of
                       // sum P' Z of group G (z[2G]; the scaled positions of INT4 / INT2 in z[2G + 1])
  float4_t o[8];       // O^T[dims 16k + 4g + i][head c]
  float nm = 0.0f;     // -m sl2 (0 while m = -inf): the exponent offset of softmax_step2, set with
                       // m and the scale sl2 in use (set_nm)
  uint64_t vmask = 0;  // lanes of the wave whose head is valid (wave-uniform)
};
__device__ __forceinline__ void set_nm(State &st, float sl2) { st.nm = st.m == kNegInf ? 0.0f : -st.m * sl2; }

// Update the running max with 8 unscaled logits (slots (tt, i) = (e >> 2, e & 3)) and return
// p = exp2(sl2 (s - m)), sl2 = softmax_scale * log2(e) > 0; positions whose A element is scaled
// by 2^SH (mask bit e) get p / 2^SH.
template <int SH = 0>
__device__ __forceinline__ void softmax_step(State &st, const float (&s)[8], float (&p)[8], bool valid_head,
                                             unsigned scaled_mask, float sl2) {
  // Fast path: no logit of a valid head exceeds the reference max by more than the slack, so
  // the reference and every accumulator stay as they are and no cross-lane reduction is
  // needed.  Otherwise the new max of each head is reduced over its four lane quarters and the
  // state is rescaled to it.  (The reference only has to be common to l and o; with a slack,
  // p may exceed 1 by at most 2^kSlackLog2.)
  const float ml = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
  if (__builtin_amdgcn_ballot_w64(valid_head && ml > st.m + st.slack) != 0) {
    const float mt = quad_max(ml);
    const float m_new = fmaxf(st.m, mt);
    const float alpha = (m_new == kNegInf) ? 1.0f : __builtin_amdgcn_exp2f((st.m - m_new) * sl2);
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.z[i] *= alpha;
#pragma unroll
    for (int k = 0; k < 8; ++k) st.o[k] *= alpha;
    st.m = m_new;
  }
  const float nm = st.m == kNegInf ? 0.0f : -st.m * sl2;
  const float nm4 = nm - (float)SH;
  float ls = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bool sc = (scaled_mask >> e) & 1;
    p[e] = __builtin_amdgcn_exp2f(fmaf(s[e], sl2, sc ? nm4 : nm));   // v_exp_f32; results below 2^-126 flush to 0
    ls = sc ? fmaf((float)(1 << SH), p[e], ls) : ls + p[e];
  }
  st.l += ls;
}

// ---------------------------------------------------------------- one 32-slot step per format
// blk: LDS copy of the block; w: wave; TAIL: only the first nvalid slots of the block hold
// tokens (the last block of a tier).
struct QOp {
  half8_t qb[4];
  float qs[4];             // per-group sums of the effective q (zero-point terms)
  float qscale = 1.0f;     // 2^t the query row was scaled by (kQShift formats; else 1)
};

// N consecutive 32-bit words from LDS (N = 2, 4 or 8)
template <int N>
__device__ __forceinline__ void lds_words(const uint8_t *p, uint32_t (&w)[N]) {
  if constexpr (N == 2) {
    const uint2 x = *(const uint2 *)p;
    w[0] = x.x; w[1] = x.y;
  } else {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint4 x = *(const uint4 *)(p + 16 * i);
      w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
    }
  }
}
// fp16 half h of a word as an f32 operand (folds into v_fma_mix as a converted source)
__device__ __forceinline__ float half_of(uint32_t word, int h) { return (float)as_h2(word)[h]; }
// fp16 pair (fp16(p0 S.lo), fp16(p1 S.hi)): each product rounded to f32, then to fp16 (written
// as fused multiply-adds with +0 so that each is one v_fma_mix with the fp16 half as a source)
__device__ __forceinline__ uint32_t pk_scaled(float p0, float p1, uint32_t s) {
  return pk(__builtin_fmaf(p0, half_of(s, 0), 0.0f), __builtin_fmaf(p1, half_of(s, 1), 0.0f));
}

// Per-channel K: add a Q operand's sum of (qh + ql) Z over its 8 elements into b1 (or b16 for
// the INT4 / INT2 elements 2, 3, 6, 7, which meet codes times 16 / 4)
template <bool kScaledOdd>
__device__ __forceinline__ void kc_zero_point(half8_t qh, half8_t ql, uint4 zv, float &b1, float &b16) {
  const uint4 hw = __builtin_bit_cast(uint4, qh), lw = __builtin_bit_cast(uint4, ql);
  const uint32_t h[4] = {hw.x, hw.y, hw.z, hw.w}, l[4] = {lw.x, lw.y, lw.z, lw.w}, z[4] = {zv.x, zv.y, zv.z, zv.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float &b = (kScaledOdd && (k & 1)) ? b16 : b1;
    b = __builtin_amdgcn_fdot2(as_h2(h[k]), as_h2(z[k]), b, false);
    b = __builtin_amdgcn_fdot2(as_h2(l[k]), as_h2(z[k]), b, false);
  }
}

template <int NB, int GS, bool TAIL>
__device__ __forceinline__ void affine_step(const uint8_t *blk, int w, int g, int c, const QOp &q, float sl2,
                                            bool valid_head, int nvalid, State &st) {
  constexpr bool kKcK = GS == kKc;          // K per channel: one (S, Z) per dim for the whole block
  constexpr int NG = kGroups<GS>;           // per-token groups (of V; also of K unless per channel)
  constexpr int kKm = 2048 * NB;
  constexpr int kVc = kKcK ? 2048 * NB + 512 : 2048 * NB + 512 * NG;
  constexpr int kVm = kKcK ? 4096 * NB + 512 : 4096 * NB + 512 * NG;
  const int lane = 16 * g + c;
  const half8_t (&qb)[4] = q.qb;

  // Everything that does not depend on the softmax state first (LDS reads, the V operands),
  // so that it overlaps the K -> logits -> max chain.
  // V codes of this lane: [part w][chunk r][lane][16 B]
  constexpr int kChunks = NB / 2;
  const uint8_t *vc = blk + kVc + (w * kChunks * 64 + lane) * 16;
  half8_t va[8];
  if constexpr (NB == 4) {
    const uint4 x0 = *(const uint4 *)vc, x1 = *(const uint4 *)(vc + 1024);
    va[0] = unpack_int4(x0.x); va[1] = unpack_int4(x0.y);
    va[2] = unpack_int4(x0.z); va[3] = unpack_int4(x0.w);
    va[4] = unpack_int4(x1.x); va[5] = unpack_int4(x1.y);
    va[6] = unpack_int4(x1.z); va[7] = unpack_int4(x1.w);
  } else if constexpr (NB == 2) {
    const uint4 x = *(const uint4 *)vc;
    const uint32_t ws[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) unpack_int2(ws[u], va[2 * u], va[2 * u + 1]);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint4 x = *(const uint4 *)(vc + r * 1024);
      va[2 * r] = unpack_int8(x.x, x.y);
      va[2 * r + 1] = unpack_int8(x.z, x.w);
    }
  }
  // V metadata of slots 4g + i (i = 0..3) of each tile: S of group G at half 4G + i, then the Z
  uint32_t vsw[2][2 * NG], vzw[2][2 * NG];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const uint8_t *m = blk + kVm + ((2 * w + tt) * 4 + g) * 16 * NG;
    lds_words<2 * NG>(m, vsw[tt]);
    lds_words<2 * NG>(m + 8 * NG, vzw[tt]);
  }

  // Per-channel K: the block's per-dim S is folded into Q as two fp16 terms, qh = RN(q S) and
  // ql = q S - qh (exact through a fused multiply-add: an fp16 product has at most 22
  // significant bits), so the logits keep the accuracy of an fp32 product; the head's
  // sum_d q_d S_d Z_d, the same for every token of the block, leaves each logit.
  half8_t qkh[4], qkl[4];
  float bq = 0.0f;
  if constexpr (kKcK) {
    const uint8_t *km = blk + kKm + 64 * g;            // (S, Z) in operand order: 32g + 8j + e
    float b1 = 0.0f, b16 = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 sv = *(const uint4 *)(km + 16 * j), zv = *(const uint4 *)(km + 256 + 16 * j);
      const half8_t s8 = __builtin_bit_cast(half8_t, sv);
      qkh[j] = qb[j] * s8;
      qkl[j] = __builtin_elementwise_fma(qb[j], s8, -qkh[j]);
      kc_zero_point<NB == 4 || NB == 2>(qkh[j], qkl[j], zv, b1, b16);
    }
    bq = quad_sum(fmaf((float)(NB == 4 ? 16 : 4), b16, b1)) * kSub;   // in the 2^-24 units of the logits
  }

  float s[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tau = 2 * w + tt;
    // K codes: [part w][tile tt][chunk][lane][min(16, 4n) bytes]; op[j] feeds k-step j
    const uint8_t *row = blk + (tau * (NB == 8 ? 2 : 1) * 64 + lane) * (NB == 2 ? 8 : 16);
    half8_t op[4];
    if constexpr (NB == 4) {
      const uint4 x = *(const uint4 *)row;
      op[0] = unpack_int4(x.x); op[1] = unpack_int4(x.y); op[2] = unpack_int4(x.z); op[3] = unpack_int4(x.w);
    } else if constexpr (NB == 2) {
      const uint2 x = *(const uint2 *)row;
      if constexpr (kKcK) {
        unpack_int2(x.x, op[0], op[1]);
        unpack_int2(x.y, op[2], op[3]);
      } else {
        unpack_int2_k(x.x, op[0], op[1]);
        unpack_int2_k(x.y, op[2], op[3]);
      }
    } else {
      const uint4 x = *(const uint4 *)row, y = *(const uint4 *)(row + 1024);
      op[0] = unpack_int8(x.x, x.y); op[1] = unpack_int8(x.z, x.w);
      op[2] = unpack_int8(y.x, y.y); op[3] = unpack_int8(y.z, y.w);
    }
    if constexpr (kKcK) {
      float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f}, accl = acc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = mfma(op[j], qkh[j], acc);
        accl = mfma(op[j], qkl[j], accl);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = (acc[i] + accl[i]) - bq;
        if (TAIL && 16 * tau + 4 * g + i >= nvalid) v = kNegInf;
        s[4 * tt + i] = v;
      }
      continue;
    }
    float4_t acc[NG];
#pragma unroll
    for (int G = 0; G < NG; ++G) acc[G] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[k_group<GS>(j)] = mfma(op[j], qb[j], acc[k_group<GS>(j)]);
    // (S, Z) of slots 16 tau + 4g + i, group G at half NG i + G
    uint32_t ksw[2 * NG], kzw[2 * NG];
    lds_words<2 * NG>(blk + kKm + tau * 64 * NG + 8 * NG * g, ksw);
    lds_words<2 * NG>(blk + kKm + tau * 64 * NG + 32 * NG + 8 * NG * g, kzw);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.0f;
#pragma unroll
      for (int G = 0; G < NG; ++G) {
        const int hx = NG * i + G;
        const float u = __builtin_fmaf(-half_of(kzw[hx >> 1], hx & 1), q.qs[G], acc[G][i]);
        v = __builtin_fmaf(half_of(ksw[hx >> 1], hx & 1), u, G == 0 ? 0.0f : v);
      }
      if (TAIL && 16 * tau + 4 * g + i >= nvalid) v = kNegInf;
      s[4 * tt + i] = v;
    }
  }
  float p[8];
  constexpr int SH = NB == 4 ? 4 : NB == 2 ? 2 : 0;
  constexpr unsigned kScaled = SH != 0 ? 0xCCu : 0u;   // INT4 / INT2: positions i = 2, 3 of both tiles
  softmax_step<SH>(st, s, p, valid_head, kScaled, sl2);

  // P' = p * S per group (one fp16 rounding), and the zero-point sums sum P' Z
  half8_t pb[NG];
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    uint32_t pw[4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const float *pp = p + 4 * tt;
      const uint32_t s01 = vsw[tt][2 * G], s23 = vsw[tt][2 * G + 1];
      const uint32_t a01 = pk_scaled(pp[0], pp[1], s01), a23 = pk_scaled(pp[2], pp[3], s23);
      pw[2 * tt] = a01;
      pw[2 * tt + 1] = a23;
      const half2_t z01 = as_h2(vzw[tt][2 * G]), z23 = as_h2(vzw[tt][2 * G + 1]);
      if constexpr (NB == 4 || NB == 2) {
        st.z[2 * G] = __builtin_amdgcn_fdot2(as_h2(a01), z01, st.z[2 * G], false);
        st.z[2 * G + 1] = __builtin_amdgcn_fdot2(as_h2(a23), z23, st.z[2 * G + 1], false);
      } else {
        st.z[2 * G] = __builtin_amdgcn_fdot2(as_h2(a01), z01, st.z[2 * G], false);
        st.z[2 * G] = __builtin_amdgcn_fdot2(as_h2(a23), z23, st.z[2 * G], false);
      }
    }
    pb[G] = h8(pw[0], pw[1], pw[2], pw[3]);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) st.o[k] = mfma(va[k], pb[v_group<GS>(k)], st.o[k]);
}

template <bool TAIL>
__device__ __forceinline__ void nvfp4_step(const uint8_t *blk, int w, int g, int c, const QOp &q, float sl2,
                                           bool valid_head, int nvalid, State &st) {
  const int lane = 16 * g + c;
  const half8_t (&qb)[4] = q.qb;
  float s[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tl = (2 * w + tt) * 64 + lane;
    const uint4 x = *(const uint4 *)(blk + tl * 16);                          // dims 32g .. 32g+31 of slot c
    const uint32_t sb = *(const uint16_t *)(blk + kNvKs + tl * 2);            // scales of blocks 2g, 2g+1
    const uint32_t s0 = e4m3_pair((sb & 0xFFu) * 0x0101u, false);             // (s_2g, s_2g)
    const uint32_t s1 = e4m3_pair((sb >> 8) * 0x0101u, false);                // (s_2g+1, s_2g+1)
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = mfma(unpack_fp4(x.x, s0, s0, s0, s0), qb[0], acc);
    acc = mfma(unpack_fp4(x.y, s0, s0, s0, s0), qb[1], acc);
    acc = mfma(unpack_fp4(x.z, s1, s1, s1, s1), qb[2], acc);
    acc = mfma(unpack_fp4(x.w, s1, s1, s1, s1), qb[3], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = acc[i];
      if (TAIL && 16 * (2 * w + tt) + 4 * g + i >= nvalid) v = kNegInf;
      s[4 * tt + i] = v;
    }
  }
  float p[8];
  softmax_step(st, s, p, valid_head, 0u, sl2);
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

// FP8 (E4M3 codes with scale 1, INT8's byte positions): the values are exact fp16, so the
// logits are the plain dot products and P multiplies the converted codes directly.  The
// convert yields a word's bytes in order (b0, b1, b2, b3) where INT8's unpack yields operand
// positions (b0, b2, b1, b3), so the Q dims and the P operand follow that order.
template <bool TAIL>
__device__ __forceinline__ void fp8_step(const uint8_t *blk, int w, int g, int c, const QOp &q, float sl2,
                                         bool valid_head, int nvalid, State &st) {
  const int lane = 16 * g + c;
  const half8_t (&qb)[4] = q.qb;
  const uint8_t *vc = blk + kF8Vc + (w * 4 * 64 + lane) * 16;
  half8_t va[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint4 x = *(const uint4 *)(vc + r * 1024);
    va[2 * r] = unpack_fp8(x.x, x.y);
    va[2 * r + 1] = unpack_fp8(x.z, x.w);
  }
  float s[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tau = 2 * w + tt;
    const uint8_t *row = blk + (tau * 2 * 64 + lane) * 16;
    const uint4 x = *(const uint4 *)row, y = *(const uint4 *)(row + 1024);
    float4_t a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = a0;
    a0 = mfma(unpack_fp8(x.x, x.y), qb[0], a0);
    a0 = mfma(unpack_fp8(x.z, x.w), qb[1], a0);
    a1 = mfma(unpack_fp8(y.x, y.y), qb[2], a1);
    a1 = mfma(unpack_fp8(y.z, y.w), qb[3], a1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = a0[i] + a1[i];
      if (TAIL && 16 * tau + 4 * g + i >= nvalid) v = kNegInf;
      s[4 * tt + i] = v;
    }
  }
  float p[8];
  softmax_step(st, s, p, valid_head, 0u, sl2);
  const half8_t pb = h8(pk(p[0], p[2]), pk(p[1], p[3]), pk(p[4], p[6]), pk(p[5], p[7]));
#pragma unroll
  for (int k = 0; k < 8; ++k) st.o[k] = mfma(va[k], pb, st.o[k]);
}

// MXFP4: K lanes hold one 32-dim block of one slot, so its codes convert under a single scale
// (no multiply); V as in mx_v_tiles.
template <bool TAIL>
__device__ __forceinline__ void mxfp4_step(const uint8_t *blk, int w, int g, int c, const QOp &q, float sl2,
                                           bool valid_head, int nvalid, State &st) {
  const int lane = 16 * g + c;
  const half8_t (&qb)[4] = q.qb;
  half8_t va[8];
  {
    const uint8_t *vc = blk + kMxVc + (w * 2 * 64 + lane) * 16;
    const uint4 x0 = *(const uint4 *)vc, x1 = *(const uint4 *)(vc + 1024);
    const uint4 s01 = *(const uint4 *)(blk + kMxVs + (4 * w + g) * 32);        // [m][e], m = 0, 1
    const uint4 s23 = *(const uint4 *)(blk + kMxVs + (4 * w + g) * 32 + 16);   // m = 2, 3
    const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    const uint32_t sw[8] = {s01.x, s01.y, s01.z, s01.w, s23.x, s23.y, s23.z, s23.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t lo[4], hi[4];
      mx_v_tiles(xw[2 * m], xw[2 * m + 1], sw[2 * m], sw[2 * m + 1], lo, hi);
      va[2 * m] = h8(lo[0], lo[1], lo[2], lo[3]);
      va[2 * m + 1] = h8(hi[0], hi[1], hi[2], hi[3]);
    }
  }
  float s[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tl = (2 * w + tt) * 64 + lane;
    const uint4 x = *(const uint4 *)(blk + tl * 16);                          // dims 32g .. 32g+31 of slot c
    const float X = e8m0_f32((uint32_t)blk[kMxKs + tl], 0);
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = mfma(unpack_mx(x.x, X), qb[0], acc);
    acc = mfma(unpack_mx(x.y, X), qb[1], acc);
    acc = mfma(unpack_mx(x.z, X), qb[2], acc);
    acc = mfma(unpack_mx(x.w, X), qb[3], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = acc[i];
      if (TAIL && 16 * (2 * w + tt) + 4 * g + i >= nvalid) v = kNegInf;
      s[4 * tt + i] = v;
    }
  }
  float p[8];
  softmax_step(st, s, p, valid_head, 0u, sl2);
  const half8_t pb = h8(pk(p[0], p[1]), pk(p[2], p[3]), pk(p[4], p[5]), pk(p[6], p[7]));
#pragma unroll
  for (int k = 0; k < 8; ++k) st.o[k] = mfma(va[k], pb, st.o[k]);
}

// FP16 blocks: the operands are the stored values (K lane chunks of dims 32g + 8i .. +7 in
// natural order, V chunks of 8 slots at one dim), so a step is two MFMA chains and the softmax.
template <bool TAIL>
__device__ __forceinline__ void fp16_step(const uint8_t *blk, int w, int g, int c, const QOp &q, float sl2,
                                          bool valid_head, int nvalid, State &st) {
  const int lane = 16 * g + c;
  const half8_t (&qb)[4] = q.qb;
  const uint8_t *vc = blk + kF16Vc + (w * 8 * 64 + lane) * 16;
  half8_t va[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) va[k] = *(const half8_t *)(vc + k * 1024);
  float s[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tau = 2 * w + tt;
    const uint8_t *row = blk + (tau * 4 * 64 + lane) * 16;
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = mfma(*(const half8_t *)(row + i * 1024), qb[i], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = acc[i];
      if (TAIL && 16 * tau + 4 * g + i >= nvalid) v = kNegInf;
      s[4 * tt + i] = v;
    }
  }
  float p[8];
  softmax_step(st, s, p, valid_head, 0u, sl2);
  const half8_t pb = h8(pk(p[0], p[1]), pk(p[2], p[3]), pk(p[4], p[5]), pk(p[6], p[7]));
#pragma unroll
  for (int k = 0; k < 8; ++k) st.o[k] = mfma(va[k], pb, st.o[k]);
}

// fp16 residual, 32 slots u*32 .. u*32+31 (direct global loads; R slots allocated, r used).
__device__ __forceinline__ void residual_step(const uint8_t *res, int R, int r, int u, int g, int c, const QOp &q,
                                              float sl2, bool valid_head, State &st) {
  const half8_t (&qb)[4] = q.qb;
  const int ntiles = R / 16;
  // every K and V load of the step goes out first (one wait for memory); a tile past the
  // residual reads the last tile instead and is masked below
  uint4 kx[2][4];
  uint2 vx[8][2];
  const uint8_t *vres = res + (int64_t)R * 256;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tau = min(2 * u + tt, ntiles - 1);
    const uint4 *row = (const uint4 *)(res + (16 * tau + c) * 256 + 64 * g);   // dims 32g .. 32g+31
#pragma unroll
    for (int j = 0; j < 4; ++j) kx[tt][j] = row[j];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tau = min(2 * u + tt, ntiles - 1);
      vx[k][tt] = *(const uint2 *)(vres + ((tau * kHeadDim + 16 * k + c) * 16 + 4 * g) * 2);
    }
  float s[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tau = 2 * u + tt;
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (tau < ntiles) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma(__builtin_bit_cast(half8_t, kx[tt][j]), qb[j], acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = 16 * tau + 4 * g + i;
      s[4 * tt + i] = (tau < ntiles && slot < r) ? acc[i] : kNegInf;
    }
  }
  float p[8];
  softmax_step(st, s, p, valid_head, 0u, sl2);
  const half8_t pb = h8(pk(p[0], p[1]), pk(p[2], p[3]), pk(p[4], p[5]), pk(p[6], p[7]));
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint32_t v[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tau = 2 * u + tt;
      if (tau < ntiles) {
        const uint2 x = vx[k][tt];
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

// ================================================================ paired subtiles (G <= 8)
// A wave's 32 slots are two 16-slot subtiles s = 0, 1.  The QK^T MFMA puts (subtile, head)
// in its 16 columns, c = 8s + h, and splits its 32-wide k range by lane quarter: quarters
// 2s and 2s+1 feed the tokens of subtile s (each quarter 8 of the 16 dims of a k-step), and
// the Q operand is block diagonal (zero where the quarter's subtile is not the column's).
// So every column carries a real head when G = 8 (half of them when G = 4) and each lane
// holds 4 logits, not 8.  PV uses v_mfma_f32_16x16x16_f16 once per subtile s0 computing
// O^T: A = the V codes of subtile s0, B = P' of the lanes whose column subtile is s0 (zero
// elsewhere); each lane accumulates its own column (subtile, head), and the two subtile
// columns of a head are summed at the end.
struct QOp2 {
  half8_t qb[8];
  float qs[4];
  float qscale = 1.0f;     // as in QOp
};

// Dim (index into the lane's 64 loaded dims) fed by B element e of k-step j, and the log2 of
// the factor of the A element it meets.  Affine formats and FP8: the lane holds dims 64G + 16(2q + gi) + m
// at local index 32G + 16gi + m (G, gi in {0,1}); natural formats dims 64q + i at index i.
// B operand idx feeds k-step j = 2(idx >> 2) + (idx & 1) of lane quarter 2q + gi, gi = (idx >> 1) & 1.
template <int FMT, int GS>
__device__ __forceinline__ int q_loc2(int j, int e, int &sh) {
  const int G = j >> 2, gi = (j >> 1) & 1, hh = j & 1;
  sh = k_elem_sh<FMT, GS>(hh, e);
  if constexpr (is_affine(FMT) && GS == 32) {
    return 8 * (2 * (2 * G + hh) + gi) + e;   // groups of 32: dims 32 step + 8(2q + gi) + e
  } else if constexpr (FMT == kFmtInt4) {
    return 32 * G + 16 * gi + 8 * hh + (e >> 1) + 4 * (e & 1);
  } else if constexpr (FMT == kFmtInt2) {
    return 32 * G + 16 * gi + 4 * hh + (e >> 1) + 8 * (e & 1);
  } else if constexpr (FMT == kFmtInt8) {
    return 32 * G + 16 * gi + 4 * (2 * hh + (e >> 2)) + ((e >> 1) & 1) + 2 * (e & 1);
  } else if constexpr (FMT == kFmtFp8) {
    return 32 * G + 16 * gi + 8 * hh + e;
  } else {
    return 8 * j + e;
  }
}

template <int FMT, int GS>
__device__ __forceinline__ void load_q2(const uint16_t *qrow, bool valid, int g, int c, QOp2 &q) {
  constexpr bool kLay32 = is_affine(FMT) && GS == 32;
  constexpr bool kLay64 = !kLay32 && (is_affine(FMT) || FMT == kFmtFp8);
  const int qq = g & 1;
  const bool active = valid && (c >> 3) == (g >> 1);
  uint4 raw[8];
  if constexpr (kLay32) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) raw[2 * j + gi] = *(const uint4 *)(qrow + 32 * j + 8 * (2 * qq + gi));
  } else if constexpr (kLay64) {
#pragma unroll
    for (int G = 0; G < 2; ++G)
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const uint16_t *r = qrow + 64 * G + 16 * (2 * qq + gi);
        raw[4 * G + 2 * gi] = *(const uint4 *)r;
        raw[4 * G + 2 * gi + 1] = *(const uint4 *)(r + 8);
      }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) raw[i] = *(const uint4 *)(qrow + 64 * qq + 8 * i);
  }
  _Float16 loc[64];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const half8_t v = __builtin_bit_cast(half8_t, raw[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) loc[8 * i + e] = active ? v[e] : (_Float16)0.0f;
  }
  q.qscale = 1.0f;
  if constexpr (kQShift<FMT, GS>) {
    // the two active quarters of the lane's column hold the head's two halves (the others zeros)
    _Float16 mh = (_Float16)0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) mh = __builtin_fmaxf16(mh, __builtin_fabsf16(loc[i]));
    q.qscale = q_shift_scale(quad_max((float)mh));
  }
  float qs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int sh;
      _Float16 v = loc[q_loc2<FMT, GS>(j, e, sh)];
      if constexpr (kQShift<FMT, GS>) v = (_Float16)((float)v * (q.qscale * (1.0f / (float)(1 << sh))));
      else if (sh) v = v * (_Float16)(1.0f / (float)(1 << sh));
      q.qb[j][e] = v;
      const float eff = (float)(1 << sh) * (float)v;
      qs[k_group<GS>(2 * (j >> 2) + (j & 1))] += eff;
    }
  }
#pragma unroll
  for (int G = 0; G < 4; ++G) q.qs[G] = G < kGroups<GS> ? quad_sum(qs[G]) * kSub : 0.0f;
}

// Running max / probabilities for 4 logits (slots i of the lane's subtile); scaled_mask bit i
// marks positions whose V operand carries a factor 2^SH (p / 2^SH there).
template <int SH = 0>
__device__ __forceinline__ void softmax_step2(State &st, const float (&s)[4], float (&p)[4], unsigned scaled_mask,
                                              float sl2) {
  const float ml = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  // (the compare's lane mask as it is, masked by the valid heads')
  if ((__builtin_amdgcn_ballot_w64(ml > st.m + st.slack) & st.vmask) != 0) {
    const float m_new = fmaxf(st.m, head_max2(ml));
    const float alpha = (m_new == kNegInf) ? 1.0f : __builtin_amdgcn_exp2f((st.m - m_new) * sl2);
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.z[i] *= alpha;
#pragma unroll
    for (int k = 0; k < 8; ++k) st.o[k] *= alpha;
    st.m = m_new;
    set_nm(st, sl2);
  }
  const float nm = st.nm;
  const float nm4 = nm - (float)SH;
  float ls = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool sc = (scaled_mask >> i) & 1;
    p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], sl2, sc ? nm4 : nm));
    if (i == 0) ls = sc ? (float)(1 << SH) * p[i] : p[i];
    else ls = sc ? fmaf((float)(1 << SH), p[i], ls) : ls + p[i];
  }
  st.l += ls;
}

// V operand of subtile s0 from the lane's words (tokens i = 0..3), raw codes as subnormals
// (INT4: [c0, c1, 16 c2, 16 c3]; INT2: [c0, c1, 4 c2, 4 c3])
template <int NB>
__device__ __forceinline__ half4_t v_operand2(const uint32_t *vw, int k, int s0);

template <>
__device__ __forceinline__ half4_t v_operand2<4>(const uint32_t *vw, int k, int s0) {
  const uint32_t x = s0 ? vw[k] >> 8 : vw[k];
  return h4(x & 0x000F000Fu, x & 0x00F000F0u);
}
template <>
__device__ __forceinline__ half4_t v_operand2<2>(const uint32_t *vw, int k, int s0) {
  // word k >> 1 holds tiles 2(k>>1) + a; pairs (crumb s, crumb s+8), s = 4a + 2 s0 + {0, 1},
  // the second pair in place (times 4: slots i = 2, 3 carry P / 4).  The word is shifted by 8
  // for a = 1 only: subtile 1's crumbs are masked in place, times 16, so that the columns of
  // subtile 1 accumulate 16 times their sums (taken out at the end of the tier, exactly).
  const uint32_t x = (k & 1) ? vw[k >> 1] >> 8 : vw[k >> 1];
  return s0 ? h4(x & 0x00300030u, x & 0x00C000C0u) : h4(x & 0x00030003u, x & 0x000C000Cu);
}
template <>
__device__ __forceinline__ half4_t v_operand2<8>(const uint32_t *vw, int k, int s0) {
  const uint32_t x = vw[2 * k + s0];
  return h4(x & 0x00FF00FFu, (x >> 8) & 0x00FF00FFu);
}

template <int NB, int GS, bool TAIL>
__device__ __forceinline__ void affine_step2(const uint8_t *blk, int w, int g, int c, const QOp2 &q, float sl2,
                                             int nvalid, State &st) {
  constexpr bool kKcK = GS == kKc;
  constexpr int NG = kGroups<GS>;
  constexpr int kKm = 2048 * NB;
  constexpr int kVc = kKcK ? 2048 * NB + 512 : 2048 * NB + 512 * NG;
  constexpr int kVm = kKcK ? 4096 * NB + 512 : 4096 * NB + 512 * NG;
  const int lane = 16 * g + c;
  const int qq = g & 1, sa = g >> 1;           // A operand: this lane feeds subtile sa, dim half qq
  const int sc = c >> 3;                       // output column subtile

  // V codes of this lane ([part w][chunk][lane][16 B]) and the metadata of the column's slots
  constexpr int kChunks = NB / 2;
  uint32_t vw[2 * NB];
  {
    const uint8_t *vc = blk + kVc + (w * kChunks * 64 + lane) * 16;
#pragma unroll
    for (int r = 0; r < kChunks; ++r) {
      const uint4 x = *(const uint4 *)(vc + r * 1024);
      vw[4 * r] = x.x; vw[4 * r + 1] = x.y; vw[4 * r + 2] = x.z; vw[4 * r + 3] = x.w;
    }
  }
  const int tau_c = 2 * w + sc;
  uint32_t vsw[2 * NG], vzw[2 * NG], ksw[2 * NG], kzw[2 * NG];
  lds_words<2 * NG>(blk + kVm + (tau_c * 4 + g) * 16 * NG, vsw);            // S of group G, slot 4g + i: half 4G + i
  lds_words<2 * NG>(blk + kVm + (tau_c * 4 + g) * 16 * NG + 8 * NG, vzw);   // the Z likewise
  if constexpr (!kKcK) {
    lds_words<2 * NG>(blk + kKm + tau_c * 64 * NG + 8 * NG * g, ksw);       // (S, Z) of slots 4g + i: half NG i + G
    lds_words<2 * NG>(blk + kKm + tau_c * 64 * NG + 32 * NG + 8 * NG * g, kzw);
  }
  // Per-channel K: the block's per-dim S folded into this lane's Q elements (quarters 2qq + gi)
  // and the head's sum_d q_d S_d Z_d
  half8_t qkh[8], qkl[8];
  float bq = 0.0f;
  if constexpr (kKcK) {
    float b1 = 0.0f, b16 = 0.0f;
#pragma unroll
    for (int idx = 0; idx < 8; ++idx) {
      const int j = 2 * (idx >> 2) + (idx & 1), gq = 2 * qq + ((idx >> 1) & 1);
      const uint8_t *km = blk + kKm + 64 * gq + 16 * j;
      const uint4 sv = *(const uint4 *)km, zv = *(const uint4 *)(km + 256);
      const half8_t s8 = __builtin_bit_cast(half8_t, sv);
      qkh[idx] = q.qb[idx] * s8;
      qkl[idx] = __builtin_elementwise_fma(q.qb[idx], s8, -qkh[idx]);
      kc_zero_point<NB == 4 || NB == 2>(qkh[idx], qkl[idx], zv, b1, b16);
    }
    bq = quad_sum(fmaf((float)(NB == 4 ? 16 : 4), b16, b1)) * kSub;
  }

  // QK^T: lane feeds token (subtile sa, row c) from the lane strings of quarters 2qq + gi:
  // op[gi][j] feeds k-step j
  const int tau_a = 2 * w + sa;
  half8_t op[2][4];
  if constexpr (NB == 4) {
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const uint4 x = *(const uint4 *)(blk + (tau_a * 64 + 16 * (2 * qq + gi) + c) * 16);
      op[gi][0] = unpack_int4(x.x); op[gi][1] = unpack_int4(x.y);
      op[gi][2] = unpack_int4(x.z); op[gi][3] = unpack_int4(x.w);
    }
  } else if constexpr (NB == 2) {
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const uint2 x = *(const uint2 *)(blk + (tau_a * 64 + 16 * (2 * qq + gi) + c) * 8);
      if constexpr (kKcK) {
        unpack_int2(x.x, op[gi][0], op[gi][1]);
        unpack_int2(x.y, op[gi][2], op[gi][3]);
      } else {
        unpack_int2_k(x.x, op[gi][0], op[gi][1]);
        unpack_int2_k(x.y, op[gi][2], op[gi][3]);
      }
    }
  } else {
    // chunk r of (tile, lane') at ((tile * 2 + r) * 64 + lane') * 16
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const uint8_t *k = blk + ((tau_a * 2) * 64 + 16 * (2 * qq + gi) + c) * 16;
      const uint4 x = *(const uint4 *)k, y = *(const uint4 *)(k + 1024);
      op[gi][0] = unpack_int8(x.x, x.y); op[gi][1] = unpack_int8(x.z, x.w);
      op[gi][2] = unpack_int8(y.x, y.y); op[gi][3] = unpack_int8(y.z, y.w);
    }
  }
  float4_t acc[NG];
#pragma unroll
  for (int G = 0; G < NG; ++G) acc[G] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int idx = 0; idx < 8; ++idx) {
    const int j = 2 * (idx >> 2) + (idx & 1), gi = (idx >> 1) & 1;
    if constexpr (kKcK) {
      acc[0] = mfma(op[gi][j], qkh[idx], acc[0]);        // the two terms of q S (acc[1] is free)
      acc[1] = mfma(op[gi][j], qkl[idx], acc[1]);
    } else {
      acc[k_group<GS>(j)] = mfma(op[gi][j], q.qb[idx], acc[k_group<GS>(j)]);
    }
  }
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = 0.0f;
    if constexpr (kKcK) {
      v = (acc[0][i] + acc[1][i]) - bq;
      if (TAIL && 16 * tau_c + 4 * g + i >= nvalid) v = kNegInf;
      s[i] = v;
      continue;
    }
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      const int hx = NG * i + G;
      const float u = __builtin_fmaf(-half_of(kzw[hx >> 1], hx & 1), q.qs[G], acc[G][i]);
      v = __builtin_fmaf(half_of(ksw[hx >> 1], hx & 1), u, G == 0 ? 0.0f : v);
    }
    if (TAIL && 16 * tau_c + 4 * g + i >= nvalid) v = kNegInf;
    s[i] = v;
  }
  float p[4];
  constexpr int SH = NB == 4 ? 4 : NB == 2 ? 2 : 0;
  constexpr unsigned kScaled = SH != 0 ? 0xCu : 0u;   // INT4 / INT2: positions i = 2, 3
  softmax_step2<SH>(st, s, p, kScaled, sl2);

  // P' = p * S per group (one fp16 rounding) and the zero-point sums sum P' Z; PV as
  // O^T += V^T P per subtile s0: A = V codes of s0, B = this lane's P' where its column
  // subtile is s0 (else zero); the accumulator rows are dims, its column the lane's head.
  half4_t pa[NG][2];
#pragma unroll
  for (int G = 0; G < NG; ++G) {
    const uint32_t a01 = pk_scaled(p[0], p[1], vsw[2 * G]);
    const uint32_t a23 = pk_scaled(p[2], p[3], vsw[2 * G + 1]);
    if constexpr (NB == 4 || NB == 2) {
      st.z[2 * G] = __builtin_amdgcn_fdot2(as_h2(a01), as_h2(vzw[2 * G]), st.z[2 * G], false);
      st.z[2 * G + 1] = __builtin_amdgcn_fdot2(as_h2(a23), as_h2(vzw[2 * G + 1]), st.z[2 * G + 1], false);
    } else {
      st.z[2 * G] = __builtin_amdgcn_fdot2(as_h2(a01), as_h2(vzw[2 * G]), st.z[2 * G], false);
      st.z[2 * G] = __builtin_amdgcn_fdot2(as_h2(a23), as_h2(vzw[2 * G + 1]), st.z[2 * G], false);
    }
    pa[G][0] = sc == 0 ? h4(a01, a23) : h4(0u, 0u);
    pa[G][1] = sc == 1 ? h4(a01, a23) : h4(0u, 0u);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    st.o[k] = mfma_pv2(v_operand2<NB>(vw, k, 0), v_operand2<NB>(vw, k, 1), pa[v_group<GS>(k)][0], pa[v_group<GS>(k)][1],
                       st.o[k]);
  }
}

template <bool TAIL>
__device__ __forceinline__ void nvfp4_step2(const uint8_t *blk, int w, int g, int c, const QOp2 &q, float sl2,
                                            int nvalid, State &st) {
  const int lane = 16 * g + c;
  const int qq = g & 1, sa = g >> 1, sc = c >> 3;
  const int tau_a = 2 * w + sa, tau_c = 2 * w + sc;
  const int l0 = tau_a * 64 + 16 * (2 * qq) + c, l1 = l0 + 16;
  const uint4 x0 = *(const uint4 *)(blk + l0 * 16), x1 = *(const uint4 *)(blk + l1 * 16);
  const uint32_t sb0 = *(const uint16_t *)(blk + kNvKs + l0 * 2), sb1 = *(const uint16_t *)(blk + kNvKs + l1 * 2);
  const uint32_t s00 = e4m3_pair((sb0 & 0xFFu) * 0x0101u, false), s01 = e4m3_pair((sb0 >> 8) * 0x0101u, false);
  const uint32_t s10 = e4m3_pair((sb1 & 0xFFu) * 0x0101u, false), s11 = e4m3_pair((sb1 >> 8) * 0x0101u, false);
  const uint4 vx0 = *(const uint4 *)(blk + kNvVc + (w * 2 * 64 + lane) * 16);
  const uint4 vx1 = *(const uint4 *)(blk + kNvVc + (w * 2 * 64 + lane) * 16 + 1024);
  const uint32_t vw[8] = {vx0.x, vx0.y, vx0.z, vx0.w, vx1.x, vx1.y, vx1.z, vx1.w};
  const uint8_t *vs = blk + kNvVs + (4 * w + g) * 64;                          // [k][e] scale bytes

  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  acc = mfma(unpack_fp4(x0.x, s00, s00, s00, s00), q.qb[0], acc);
  acc = mfma(unpack_fp4(x0.y, s00, s00, s00, s00), q.qb[1], acc);
  acc = mfma(unpack_fp4(x0.z, s01, s01, s01, s01), q.qb[2], acc);
  acc = mfma(unpack_fp4(x0.w, s01, s01, s01, s01), q.qb[3], acc);
  acc = mfma(unpack_fp4(x1.x, s10, s10, s10, s10), q.qb[4], acc);
  acc = mfma(unpack_fp4(x1.y, s10, s10, s10, s10), q.qb[5], acc);
  acc = mfma(unpack_fp4(x1.z, s11, s11, s11, s11), q.qb[6], acc);
  acc = mfma(unpack_fp4(x1.w, s11, s11, s11, s11), q.qb[7], acc);
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = acc[i];
    if (TAIL && 16 * tau_c + 4 * g + i >= nvalid) v = kNegInf;
    s[i] = v;
  }
  float p[4];
  softmax_step2(st, s, p, 0u, sl2);
  const uint32_t p01 = pk(p[0], p[1]), p23 = pk(p[2], p[3]);
  const half4_t pa0 = sc == 0 ? h4(p01, p23) : h4(0u, 0u), pa1 = sc == 1 ? h4(p01, p23) : h4(0u, 0u);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint2 scb = *(const uint2 *)(vs + 8 * k);      // scales of e = 0..3 (subtile 0), 4..7 (subtile 1)
    const uint32_t f0 = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(vw[k], 1.0f, 0));
    const uint32_t f1 = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(vw[k], 1.0f, 1));
    const uint32_t f2 = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(vw[k], 1.0f, 2));
    const uint32_t f3 = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(vw[k], 1.0f, 3));
    const half4_t b0 = h4(as_u(as_h2(f0) * as_h2(e4m3_pair(scb.x, false))), as_u(as_h2(f1) * as_h2(e4m3_pair(scb.x, true))));
    const half4_t b1 = h4(as_u(as_h2(f2) * as_h2(e4m3_pair(scb.y, false))), as_u(as_h2(f3) * as_h2(e4m3_pair(scb.y, true))));
    st.o[k] = mfma_pv2(b0, b1, pa0, pa1, st.o[k]);
  }
}

template <bool TAIL>
__device__ __forceinline__ void fp8_step2(const uint8_t *blk, int w, int g, int c, const QOp2 &q, float sl2,
                                          int nvalid, State &st) {
  const int lane = 16 * g + c;
  const int qq = g & 1, sa = g >> 1, sc = c >> 3;
  const int tau_a = 2 * w + sa, tau_c = 2 * w + sc;
  uint32_t vw[16];
  {
    const uint8_t *vc = blk + kF8Vc + (w * 4 * 64 + lane) * 16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint4 x = *(const uint4 *)(vc + r * 1024);
      vw[4 * r] = x.x; vw[4 * r + 1] = x.y; vw[4 * r + 2] = x.z; vw[4 * r + 3] = x.w;
    }
  }
  // K: chunk G of (tile, lane') at ((tile * 2 + G) * 64 + lane') * 16, lane quarters 2qq, 2qq+1
  const uint8_t *k0 = blk + ((tau_a * 2) * 64 + 16 * (2 * qq) + c) * 16;
  const uint8_t *k1 = blk + ((tau_a * 2) * 64 + 16 * (2 * qq + 1) + c) * 16;
  const uint4 x0 = *(const uint4 *)k0, y0 = *(const uint4 *)(k0 + 1024);
  const uint4 x1 = *(const uint4 *)k1, y1 = *(const uint4 *)(k1 + 1024);
  float4_t a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = a0;
  a0 = mfma(unpack_fp8(x0.x, x0.y), q.qb[0], a0);
  a0 = mfma(unpack_fp8(x0.z, x0.w), q.qb[1], a0);
  a0 = mfma(unpack_fp8(x1.x, x1.y), q.qb[2], a0);
  a0 = mfma(unpack_fp8(x1.z, x1.w), q.qb[3], a0);
  a1 = mfma(unpack_fp8(y0.x, y0.y), q.qb[4], a1);
  a1 = mfma(unpack_fp8(y0.z, y0.w), q.qb[5], a1);
  a1 = mfma(unpack_fp8(y1.x, y1.y), q.qb[6], a1);
  a1 = mfma(unpack_fp8(y1.z, y1.w), q.qb[7], a1);
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = a0[i] + a1[i];
    if (TAIL && 16 * tau_c + 4 * g + i >= nvalid) v = kNegInf;
    s[i] = v;
  }
  float p[4];
  softmax_step2(st, s, p, 0u, sl2);
  // word 2k + s0 holds slots 4 s0 + (0, 2, 1, 3) of dim 16k + c in byte order
  const uint32_t p02 = pk(p[0], p[2]), p13 = pk(p[1], p[3]);
  const half4_t pa0 = sc == 0 ? h4(p02, p13) : h4(0u, 0u), pa1 = sc == 1 ? h4(p02, p13) : h4(0u, 0u);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    st.o[k] = mfma_pv2(h4(e4m3_pair(vw[2 * k], false), e4m3_pair(vw[2 * k], true)),
                       h4(e4m3_pair(vw[2 * k + 1], false), e4m3_pair(vw[2 * k + 1], true)), pa0, pa1, st.o[k]);
  }
}

template <bool TAIL>
__device__ __forceinline__ void mxfp4_step2(const uint8_t *blk, int w, int g, int c, const QOp2 &q, float sl2,
                                            int nvalid, State &st) {
  const int lane = 16 * g + c;
  const int qq = g & 1, sa = g >> 1, sc = c >> 3;
  const int tau_a = 2 * w + sa, tau_c = 2 * w + sc;
  const int l0 = tau_a * 64 + 16 * (2 * qq) + c, l1 = l0 + 16;
  const uint4 x0 = *(const uint4 *)(blk + l0 * 16), x1 = *(const uint4 *)(blk + l1 * 16);
  const float X0 = e8m0_f32((uint32_t)blk[kMxKs + l0], 0), X1 = e8m0_f32((uint32_t)blk[kMxKs + l1], 0);
  const uint8_t *vc = blk + kMxVc + (w * 2 * 64 + lane) * 16;
  const uint4 vx0 = *(const uint4 *)vc, vx1 = *(const uint4 *)(vc + 1024);
  const uint4 s01 = *(const uint4 *)(blk + kMxVs + (4 * w + g) * 32);
  const uint4 s23 = *(const uint4 *)(blk + kMxVs + (4 * w + g) * 32 + 16);

  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  acc = mfma(unpack_mx(x0.x, X0), q.qb[0], acc);
  acc = mfma(unpack_mx(x0.y, X0), q.qb[1], acc);
  acc = mfma(unpack_mx(x0.z, X0), q.qb[2], acc);
  acc = mfma(unpack_mx(x0.w, X0), q.qb[3], acc);
  acc = mfma(unpack_mx(x1.x, X1), q.qb[4], acc);
  acc = mfma(unpack_mx(x1.y, X1), q.qb[5], acc);
  acc = mfma(unpack_mx(x1.z, X1), q.qb[6], acc);
  acc = mfma(unpack_mx(x1.w, X1), q.qb[7], acc);
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = acc[i];
    if (TAIL && 16 * tau_c + 4 * g + i >= nvalid) v = kNegInf;
    s[i] = v;
  }
  float p[4];
  softmax_step2(st, s, p, 0u, sl2);
  const uint32_t p01 = pk(p[0], p[1]), p23 = pk(p[2], p[3]);
  const half4_t pa0 = sc == 0 ? h4(p01, p23) : h4(0u, 0u), pa1 = sc == 1 ? h4(p01, p23) : h4(0u, 0u);
  const uint32_t xw[8] = {vx0.x, vx0.y, vx0.z, vx0.w, vx1.x, vx1.y, vx1.z, vx1.w};
  const uint32_t sw[8] = {s01.x, s01.y, s01.z, s01.w, s23.x, s23.y, s23.z, s23.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    uint32_t lo[4], hi[4];
    mx_v_tiles(xw[2 * m], xw[2 * m + 1], sw[2 * m], sw[2 * m + 1], lo, hi);
    st.o[2 * m] = mfma_pv2(h4(lo[0], lo[1]), h4(lo[2], lo[3]), pa0, pa1, st.o[2 * m]);
    st.o[2 * m + 1] = mfma_pv2(h4(hi[0], hi[1]), h4(hi[2], hi[3]), pa0, pa1, st.o[2 * m + 1]);
  }
}

template <bool TAIL>
__device__ __forceinline__ void fp16_step2(const uint8_t *blk, int w, int g, int c, const QOp2 &q, float sl2,
                                           int nvalid, State &st) {
  const int lane = 16 * g + c;
  const int qq = g & 1, sa = g >> 1, sc = c >> 3;
  const int tau_a = 2 * w + sa, tau_c = 2 * w + sc;
  // V chunk k of this lane: halves 0..3 are subtile 0's slots, 4..7 subtile 1's
  const uint8_t *vc = blk + kF16Vc + (w * 8 * 64 + lane) * 16;
  uint4 vx[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) vx[k] = *(const uint4 *)(vc + k * 1024);
  // K: the lane strings of quarters 2qq and 2qq+1 (dims 64qq .. 64qq+63) of row c of tile tau_a
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const uint8_t *row = blk + (tau_a * 4 * 64 + 16 * (2 * qq + gi) + c) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = mfma(*(const half8_t *)(row + i * 1024), q.qb[4 * gi + i], acc);
  }
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = acc[i];
    if (TAIL && 16 * tau_c + 4 * g + i >= nvalid) v = kNegInf;
    s[i] = v;
  }
  float p[4];
  softmax_step2(st, s, p, 0u, sl2);
  const uint32_t p01 = pk(p[0], p[1]), p23 = pk(p[2], p[3]);
  const half4_t pa0 = sc == 0 ? h4(p01, p23) : h4(0u, 0u), pa1 = sc == 1 ? h4(p01, p23) : h4(0u, 0u);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    st.o[k] = mfma_pv2(h4(vx[k].x, vx[k].y), h4(vx[k].z, vx[k].w), pa0, pa1, st.o[k]);
  }
}

// fp16 residual, slots 32u .. 32u+31, paired subtiles (direct global loads).  The V loads go
// out with the K loads, before the logits, so that the step waits for memory once.
__device__ __forceinline__ void residual_step2(const uint8_t *res, int R, int r, int u, int g, int c, const QOp2 &q,
                                               float sl2, State &st) {
  const int ntiles = R / 16;
  const int qq = g & 1, sa = g >> 1, sc = c >> 3;
  const int tau_a = 2 * u + sa, tau_c = 2 * u + sc;
  // Rows past r may hold stale bits (even NaN); with the block-diagonal Q a NaN row would reach
  // the other subtile's columns through 0 * NaN, so such rows are fed as zeros.
  const bool arow = tau_a < ntiles && 16 * tau_a + c < r;
  const uint4 *row = (const uint4 *)(res + (arow ? 16 * tau_a + c : 0) * 256 + 128 * qq);   // dims 64qq .. 64qq+63
  uint4 kx[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) kx[j] = row[j];
  const uint8_t *vres = res + (int64_t)R * 256;
  uint2 vx[8][2];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int s0 = 0; s0 < 2; ++s0) {
      const int tau = min(2 * u + s0, ntiles - 1);   // (a tile past the residual is zeroed below)
      vx[k][s0] = *(const uint2 *)(vres + ((tau * kHeadDim + 16 * k + c) * 16 + 4 * g) * 2);
    }
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = mfma(arow ? __builtin_bit_cast(half8_t, kx[j]) : h8(0u, 0u, 0u, 0u), q.qb[j], acc);
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = 16 * tau_c + 4 * g + i;
    s[i] = (tau_c < ntiles && slot < r) ? acc[i] : kNegInf;
  }
  float p[4];
  softmax_step2(st, s, p, 0u, sl2);
  const uint32_t p01 = pk(p[0], p[1]), p23 = pk(p[2], p[3]);
  const half4_t pa0 = sc == 0 ? h4(p01, p23) : h4(0u, 0u), pa1 = sc == 1 ? h4(p01, p23) : h4(0u, 0u);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
#pragma unroll
    for (int s0 = 0; s0 < 2; ++s0) {
      const int tau = 2 * u + s0;
      uint32_t v0 = 0u, v1 = 0u;
      if (tau < ntiles) {
        v0 = vx[k][s0].x;
        v1 = vx[k][s0].y;
        // slots past r may hold stale bits (even NaN): zero them
        const int t0 = 16 * tau + 4 * g;
        if (t0 + 0 >= r) v0 &= 0xFFFF0000u;
        if (t0 + 1 >= r) v0 &= 0x0000FFFFu;
        if (t0 + 2 >= r) v1 &= 0xFFFF0000u;
        if (t0 + 3 >= r) v1 &= 0x0000FFFFu;
      }
      st.o[k] = mfma16(h4(v0, v1), s0 ? pa1 : pa0, st.o[k]);
    }
  }
}

// ---------------------------------------------------------------- call-tagged counters
// A counter in the workspace is a 64-bit word (epoch << kCountBits | count): a 44-bit call
// tag over a 20-bit count (arrivals <= kMaxParts; cursor units <= blocks + items of a tier,
// which the host keeps below 2^20).  A call works only with words tagged with its own
// epoch; a word with any other tag is replaced, by compare-and-swap, with a fresh count of
// this call.  Adds that land on such a word are void (their issuer sees the other tag) and
// are made again.  The last workgroup of a (batch, kv_head) sets its words back to zero once
// every other access of the call has completed, so between calls they hold 0 (tag 0, which
// no call uses); only words the caller wrote since (or a workspace's first use) hold other
// values, and those are replaced unless their top 44 bits equal the call's epoch.  All
// accesses are agent-scope atomics, so workgroups on different XCDs see one order of them.
constexpr int kCountBits = 20;
constexpr uint64_t kCountMask = (1ull << kCountBits) - 1;
__device__ __forceinline__ uint64_t tag_of(uint64_t v) { return v >> kCountBits; }

// Tag the word with this call's epoch and a zero count, unless this call has done so already.
__device__ __forceinline__ void counter_open(uint64_t *w, uint64_t epoch) {
  uint64_t cur = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while (tag_of(cur) != epoch)
    if (__hip_atomic_compare_exchange_strong(w, &cur, epoch << kCountBits, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      break;
}

// The count before this call's add, after an add that came back with another tag: open the
// word with this add counted (count 0 before it), or add again once another opener has.
// Each pass either succeeds or finds the word changed by one of the finitely many other
// accesses of the call.
__device__ __forceinline__ uint32_t counter_add_slow(uint64_t *w, uint64_t epoch) {
  uint64_t cur = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    if (tag_of(cur) == epoch)
      return (uint32_t)(__hip_atomic_fetch_add(w, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kCountMask);
    if (__hip_atomic_compare_exchange_strong(w, &cur, (epoch << kCountBits) | 1u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return 0;
  }
}

// The count before an add whose returned word is `old`.
__device__ __forceinline__ uint32_t counter_result(uint64_t *w, uint64_t epoch, uint64_t old) {
  return tag_of(old) == epoch ? (uint32_t)(old & kCountMask) : counter_add_slow(w, epoch);
}

// ---------------------------------------------------------------- the kernel
struct Item {
  int bh, part, seg;          // seg = -1: residual only
  int j;                      // index of the item among its segment's items
  bool has_res;
  // of the item's sequence (the call's values, or its RagSeq in a ragged batch)
  int items_total, res_ntok, pend_count, pend_slot0;
  int64_t pend_src_tok0;
};

// Part p of every (b, h) comes in the p-th run of B*H workgroups, so that each (b, h) has
// items among the first and among the later residents of the CUs (the older wave has the
// issue priority), and the (b, h) order turns by one per run, so that round-robin dispatch
// puts the items of a (b, h) on different XCDs.  The items of a (b, h) share its chunks and
// so even out these speed differences.
__device__ __forceinline__ Item decode_item(const DecodeArgs &a, int wg) {
  const int nbh = a.B * a.H;
  Item it;
  it.part = wg / nbh;
  it.bh = (wg + it.part) % nbh;
  it.seg = -1;
  it.j = 0;
  for (int s = 0; s < a.nseg; ++s) {
    const DecodeSeg &sg = a.seg[s];
    if (it.part >= sg.part0 && it.part < sg.part0 + sg.items) {
      it.seg = s;
      it.j = it.part - sg.part0;
    }
  }
  it.has_res = a.res_ntok > 0 && it.part == (a.res_item >= 0 ? a.res_item : it.bh % a.items_total);
  it.items_total = a.items_total;
  it.res_ntok = a.res_ntok;
  it.pend_count = a.pend_count;
  it.pend_slot0 = a.pend_slot0;
  it.pend_src_tok0 = a.pend_src_tok0;
  return it;
}

// Ragged batch: the workgroup's (b, h, part) from its table entry, the rest from the
// sequence's RagSeq.  The tables are read through the constant address space (the host writes
// them before the launch; nothing in it writes them), so that, as for the call's own
// arguments, their loads are scalar and can be repeated instead of held in registers.
typedef const __attribute__((address_space(4))) RagSeq ConstRagSeq;
typedef const __attribute__((address_space(4))) uint32_t ConstU32;

__device__ __forceinline__ Item decode_item_ragged(const DecodeArgs &a, int wg) {
  const uint32_t e = ((ConstU32 *)a.rag_wg)[wg];
  const int b = (int)(e & 0xFFFFu), h = (int)((e >> 16) & 0x1FFu);
  ConstRagSeq &r = ((ConstRagSeq *)a.rag)[b];
  Item it;
  it.bh = b * a.H + h;
  it.part = (int)(e >> 25);
  it.seg = -1;
  it.j = 0;
  for (int s = 0; s < a.nseg; ++s) {
    if (it.part >= r.seg[s].part0 && it.part < r.seg[s].part0 + r.seg[s].items) {
      it.seg = s;
      it.j = it.part - r.seg[s].part0;
    }
  }
  it.items_total = r.items_total;
  it.res_ntok = r.res_ntok;
  it.has_res = it.res_ntok > 0 && it.part == it.bh % it.items_total;
  it.pend_count = r.pend_count;
  it.pend_slot0 = r.pend_slot0;
  it.pend_src_tok0 = r.pend_src_tok0;
  return it;
}



// The G query rows of a (b, h) in global memory (consecutive heads).
__device__ __forceinline__ const uint16_t *q_group(const DecodeArgs &a, int bh) {
  const int b = bh / a.H, h = bh % a.H;
  return a.q + ((int64_t)b * a.H * a.G + (int64_t)h * a.G) * kHeadDim;
}

// Row of the head a lane's column belongs to within a group's rows (global or LDS; a valid
// row even for padding columns).
template <int NSUB>
__device__ __forceinline__ const uint16_t *q_row(const uint16_t *group, int c, bool valid_head) {
  const int hc = valid_head ? (NSUB == 2 ? (c & 7) : c) : 0;
  return group + hc * kHeadDim;
}

// The fp16 residual of the item's (b, h), in natural units.
template <int NSUB>
__device__ __forceinline__ void residual_part(const DecodeArgs &a, const Item &it, const uint16_t *qgroup, int w, int g,
                                              int c, bool valid_head, State &st) {
  const uint16_t *qrow = q_row<NSUB>(qgroup, c, valid_head);
  const uint8_t *res = a.res_base + (int64_t)it.bh * a.res_bh_stride;
  const int nsteps = (it.res_ntok + 31) / 32;
  if constexpr (NSUB == 2) {
    QOp2 q;
    load_q2<kFmtFp16, kGroup>(qrow, valid_head, g, c, q);
    set_nm(st, a.scale_log2);
    for (int u = w; u < nsteps; u += kWaves) residual_step2(res, a.res_len, it.res_ntok, u, g, c, q, a.scale_log2, st);
  } else {
    QOp q;
    load_q<kFmtFp16, kGroup>(qrow, valid_head, g, q.qb, q.qs, q.qscale);
    for (int u = w; u < nsteps; u += kWaves) residual_step(res, a.res_len, it.res_ntok, u, g, c, q, a.scale_log2, valid_head, st);
  }
}

template <int FMT, int GS, int NSUB>
__device__ __forceinline__ void stream_segment(const DecodeArgs &a, const DecodeSeg &sg, const Item &it, uint8_t *smem, int *s_chunk, int w,
                               int g, int c, bool valid_head, State &st) {
  const int lane = 16 * g + c;
  constexpr int kBB = (int)block_bytes(FMT, GS);
  const int bb = kBB;
  // 1 KB per wave instruction; a block that ends on a partial KB (per-channel K blocks end on
  // half a KB) gets a last instruction with only the lanes of its remaining bytes active
  constexpr int kTailLanes = (int)(block_bytes(FMT, GS) % 1024) / 16;
  constexpr int kNdma = (kBB + 1023) / 1024;
  // Waves 0..2 load the blocks; wave 3 loads none and hands out the chunks, so that waiting
  // for its cursor atomic never waits for block loads (vmcnt counts both).
  constexpr int kDmaWaves = kWaves - 1;
  const bool dispatcher = w == kDmaWaves;
  // wave w < kDmaWaves loads chunks jj = w, w + kDmaWaves, ... below kNdma: kMineHi of them
  // for the first kNdma % kDmaWaves waves, kMineLo for the others
  constexpr int kMineHi = (kNdma + kDmaWaves - 1) / kDmaWaves, kMineLo = kNdma / kDmaWaves;
  const int mine = dispatcher ? 0 : (kNdma - w + kDmaWaves - 1) / kDmaWaves;
  uint64_t *cursor = sg.cursors + (int64_t)it.bh * kCtrStride;
  const int K = sg.chunk, items = sg.items, F = sg.fixed, nbig = sg.nbig, j = it.j;
  const int nblk = (int)((sg.ntok + kBlock - 1) / kBlock);
  const int fixed_end = min(F * items * K, nblk);            // blocks of the fixed units
  const bool dyn = fixed_end < nblk;                          // a cursor hands out the rest
  // item 0 opens the cursor early, so that the other items' first fetch-adds find it open
  if (dyn && j == 0 && dispatcher && lane == 0) counter_open(cursor, a.epoch);
  const uint8_t *gbh = sg.base + (int64_t)it.bh * sg.bh_stride;   // wave-uniform; lanes add 16 * lane
  const uint32_t lane_off = (uint32_t)lane * 16u;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  constexpr int kNbuf = decode_ring_depth(block_bytes(FMT, GS));
  const int nbuf = kNbuf;
  // INT2 in paired subtiles (the whole ring within 64 KB): the block loop is unrolled over the
  // ring slots (below)
  constexpr bool kUnrollRing = FMT == kFmtInt2 && GS == 64 && NSUB == 2 && kNbuf * kBB <= 65536;
  // Blocks of whole chunks, at most six per wave: a wave's chunk loads are issued in one or two
  // statements and the steady-state wait is a constant
  constexpr bool kBatchIssue = kTailLanes == 0 && kMineHi <= 6;
  const uint16_t *qlds = (const uint16_t *)(smem + a.q_lds_off);   // the group's query rows

  const int tail_valid = (int)(sg.ntok - (int64_t)(nblk - 1) * kBlock);   // slots in the last block
  // The (b, h)'s blocks are visited rotated by a hashed offset: the items of all (b, h) walk
  // their arenas in step, so without it the blocks read at the same time lie one arena stride
  // apart, and for some strides those addresses share HBM channels (32K-token arenas of 257 or
  // 258 blocks decoded in 72-77 us against 65-69 us for nearby strides).  The sum does not
  // depend on the order; the partial last block is recognised by its stored position.
  const int rot = nblk > 1 ? (int)(((uint32_t)it.bh * 2654435761u) % (uint32_t)nblk) : 0;
  // The item's blocks come in units: fixed unit s (s < F) is blocks [(s items + j) K, +K);
  // the cursor's unit u is K blocks at fixed_end + u K for u < nbig, else the single block
  // fixed_end + nbig K + (u - nbig).  A unit starting at or past nblk ends the sequence.
  int u_idx = 0;               // units entered so far - 1
  int u_start = j * K;         // current unit: first block, length, blocks issued from it
  int u_len = min(K, nblk - u_start);
  int u_off = 0;
  int iss_end = 0;             // blocks issued
  bool iss_done = u_start >= nblk;
  uint32_t tailmask = 0;       // ring slots that hold the partial last block
  uint64_t grab = 0;           // dispatcher lane 0: cursor value before its last fetch-add
  auto issue_next = [&]() {
    if (u_off == u_len) {
      ++u_idx;
      if (u_idx < F) {
        u_start = (u_idx * items + j) * K;
      } else if (dyn) {
        const int u = __builtin_amdgcn_readfirstlane(*s_chunk);
        u_start = u < nbig ? fixed_end + u * K : fixed_end + nbig * K + (u - nbig);
      } else {
        u_start = nblk;
      }
      if (u_start >= nblk) {
        iss_done = true;
        return;
      }
      u_len = min(u_idx < F || u_start < fixed_end + nbig * K ? K : 1, nblk - u_start);
      u_off = 0;
      // ask for the unit after this one when the cursor hands it out
      if (dyn && u_idx + 1 >= F && dispatcher && lane == 0)
        grab = __hip_atomic_fetch_add(cursor, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int blk_idx = u_start + u_off;
    const int phys = blk_idx + rot < nblk ? blk_idx + rot : blk_idx + rot - nblk;
    const int slot = (int)((uint32_t)iss_end % (uint32_t)kNbuf);
    if (!dispatcher) {
      const uint8_t *src = gbh + (int64_t)phys * bb;   // uniform
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(slot * bb));   // M0 takes a scalar
      if constexpr (kBatchIssue) {
        // the wave's chunks w, w + kDmaWaves, ...
        if (mine == kMineHi) dma16_runs<kMineHi, kDmaWaves * 1024>(src + w * 1024, lane_off, dst + w * 1024);
        else dma16_runs<kMineLo, kDmaWaves * 1024>(src + w * 1024, lane_off, dst + w * 1024);
      } else {
        for (int jj = w; jj < kNdma; jj += kDmaWaves) {
          if (kTailLanes != 0 && jj == kNdma - 1) {
            if (lane < kTailLanes) dma16(src + jj * 1024, lane_off, dst + jj * 1024);
          } else {
            dma16(src + jj * 1024, lane_off, dst + jj * 1024);
          }
        }
      }
    }
    const bool part = phys == nblk - 1 && tail_valid < kBlock;
    tailmask = (tailmask & ~(1u << slot)) | ((uint32_t)part << slot);
    u_off = __builtin_amdgcn_readfirstlane(u_off + 1);
    iss_end = __builtin_amdgcn_readfirstlane(iss_end + 1);   // uniform: keeps the waits scalar
  };
  for (int t = 0; t < nbuf - 1 && !iss_done; ++t) issue_next();

  // while the first blocks load: the residual (natural units), the operands
  constexpr bool kAff = FMT == kFmtInt2 || FMT == kFmtInt4 || FMT == kFmtInt8;
  // (capped: logits of fp16 operands stay below 2^40 in magnitude, so the cap never binds
  // where it would let p exceed the bound, and m + slack stays finite)
  if constexpr (!kAff) st.slack = fminf(kSlackLog2 / a.scale_log2, 1.0e30f);
  barrier();
  if (it.has_res) residual_part<NSUB>(a, it, qlds, w, g, c, valid_head, st);
  asm volatile("" ::: "memory");   // the operands below are not read before the residual is done
  const uint16_t *qrow = q_row<NSUB>(qlds, c, valid_head);
  QOp q;
  QOp2 q2;
  if constexpr (NSUB == 2) load_q2<FMT, GS>(qrow, valid_head, g, c, q2);
  else load_q<FMT, GS>(qrow, valid_head, g, q.qb, q.qs, q.qscale);
  // affine logits come out in units of 2^-24 (subnormal code operands), times the query row's
  // power-of-two scale
  const float qscale = NSUB == 2 ? q2.qscale : q.qscale;
  const float sl2 = kAff ? a.scale_log2 * (kInvSub / qscale) : a.scale_log2;
  // INT2 in paired subtiles: the columns of subtile 1 accumulate 16 times their PV sums
  // (v_operand2<2>); the factor is exact and taken out with the units below
  constexpr bool kO16 = FMT == kFmtInt2 && NSUB == 2;
  const float ofac = kO16 && (c >> 3) ? 16.0f : 1.0f;
  if constexpr (kAff) {
    if (st.m != kNegInf) st.m *= kSub * qscale;
#pragma unroll
    for (int k = 0; k < 8; ++k) st.o[k] = st.o[k] * (kSub * ofac);
  }
  if constexpr (NSUB == 2) set_nm(st, sl2);
  // One block of the ring: wait for it, issue the next, compute on it.  For INT2 in paired
  // subtiles (the whole ring within 64 KB) the loop is unrolled over the ring, so that each
  // slot's LDS offset is a constant folded into the reads' immediate offsets instead of a vector
  // add per address per block.
  auto one_block = [&](int p, int buf) __attribute__((always_inline)) {
    if (!dispatcher) {
      // blocks issued after this one may stay in flight: with the ring full ahead (the steady
      // state) that count is one of two constants
      const int ahead = iss_end - p - 1;
      if (kBatchIssue && ahead == kNbuf - 2) {
        if (mine == kMineHi) wait_vmcnt_c<kMineHi * (kNbuf - 2)>();
        else wait_vmcnt_c<kMineLo * (kNbuf - 2)>();   // (mine is kMineLo)
      } else {
        wait_vmcnt(__builtin_amdgcn_readfirstlane(mine * ahead));
      }
    } else if (dyn && !iss_done && u_off == u_len && u_idx + 1 >= F) {
      // the issue side enters a cursor unit now: publish the one fetched a unit ago
      if (lane == 0) {
        const uint32_t u = counter_result(cursor, a.epoch, grab);
        *s_chunk = u < (uint32_t)nblk ? (int)u : nblk;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    barrier();
    const bool full = !((tailmask >> buf) & 1u);
    if (!iss_done) issue_next();
    const uint8_t *blk = smem + buf * bb;
    const int nv = full ? kBlock : tail_valid;
    if constexpr (NSUB == 2) {
      if constexpr (FMT == kFmtNvfp4) {
        if (full) nvfp4_step2<false>(blk, w, g, c, q2, sl2, nv, st);
        else nvfp4_step2<true>(blk, w, g, c, q2, sl2, nv, st);
      } else if constexpr (FMT == kFmtFp8) {
        if (full) fp8_step2<false>(blk, w, g, c, q2, sl2, nv, st);
        else fp8_step2<true>(blk, w, g, c, q2, sl2, nv, st);
      } else if constexpr (FMT == kFmtFp16) {
        if (full) fp16_step2<false>(blk, w, g, c, q2, sl2, nv, st);
        else fp16_step2<true>(blk, w, g, c, q2, sl2, nv, st);
      } else if constexpr (FMT == kFmtMxfp4) {
        if (full) mxfp4_step2<false>(blk, w, g, c, q2, sl2, nv, st);
        else mxfp4_step2<true>(blk, w, g, c, q2, sl2, nv, st);
      } else {
        if (full) affine_step2<FMT, GS, false>(blk, w, g, c, q2, sl2, nv, st);
        else affine_step2<FMT, GS, true>(blk, w, g, c, q2, sl2, nv, st);
      }
    } else {
      if constexpr (FMT == kFmtNvfp4) {
        if (full) nvfp4_step<false>(blk, w, g, c, q, sl2, valid_head, nv, st);
        else nvfp4_step<true>(blk, w, g, c, q, sl2, valid_head, nv, st);
      } else if constexpr (FMT == kFmtFp8) {
        if (full) fp8_step<false>(blk, w, g, c, q, sl2, valid_head, nv, st);
        else fp8_step<true>(blk, w, g, c, q, sl2, valid_head, nv, st);
      } else if constexpr (FMT == kFmtFp16) {
        if (full) fp16_step<false>(blk, w, g, c, q, sl2, valid_head, nv, st);
        else fp16_step<true>(blk, w, g, c, q, sl2, valid_head, nv, st);
      } else if constexpr (FMT == kFmtMxfp4) {
        if (full) mxfp4_step<false>(blk, w, g, c, q, sl2, valid_head, nv, st);
        else mxfp4_step<true>(blk, w, g, c, q, sl2, valid_head, nv, st);
      } else {
        if (full) affine_step<FMT, GS, false>(blk, w, g, c, q, sl2, valid_head, nv, st);
        else affine_step<FMT, GS, true>(blk, w, g, c, q, sl2, valid_head, nv, st);
      }
    }
  };
  if constexpr (kUnrollRing) {
    constexpr int kRing = decode_ring_depth(block_bytes(FMT, GS));
    static_assert(kRing == 4, "the unrolled ring has four slots");
    // (iss_end grows as blocks are issued inside one_block: each test sees the current count)
    for (int p = 0; p < iss_end; p += kRing) {
      one_block(p, 0);
      if (p + 1 < iss_end) one_block(p + 1, 1);
      if (p + 2 < iss_end) one_block(p + 2, 2);
      if (p + 3 < iss_end) one_block(p + 3, 3);
    }
  } else {
    int buf = 0;
    for (int p = 0; p < iss_end; ++p) {
      one_block(p, buf);
      buf = buf + 1 == nbuf ? 0 : buf + 1;
    }
  }
  barrier();   // every wave is done with the ring before it is reused
  if constexpr (kAff) {
    // Back to natural units: m * 2^24, and o = 2^24 o - sum P' Z of the group of each dim (for
    // paired subtiles the head's total goes to its subtile-0 column only; the two columns are
    // summed later).
    if (st.m != kNegInf) st.m *= kInvSub / qscale;
    constexpr int NG = kGroups<GS>;
    const bool take = NSUB == 2 ? (c >> 3) == 0 : true;
    float zg[NG];
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      const float zl = st.z[2 * G] + (float)(1 << kSh<FMT>) * st.z[2 * G + 1];
      zg[G] = NSUB == 2 ? head_sum2(zl) : quad_sum(zl);
      if (!take) zg[G] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) st.o[k] = st.o[k] * (kInvSub / ofac) - zg[v_group<GS>(k)];
#pragma unroll
    for (int i = 0; i < 8; ++i) st.z[i] = 0.0f;
  }
}

// The last workgroup's merge of the P partials of a (b, h) (geometry in MergeGeom): the weights
// of the parts per head from their (m, l), then out = sum_p w_p o_p / sum_p w_p l_p with NB
// 16-byte loads in flight per thread.
struct MergeGeom {
  int P, G, GO, S, nout;
  __amdgpu_buffer_rsrc_t prs;
  float *sm_m, *sm_w, *sm_l, *sm_inv;
  float4_t *sm_red;
  int64_t row0;            // output row of head 0 of this (b, h)
  void *out;
  int out_fp32;
};

template <int NB>
__device__ __forceinline__ void merge_tail(const MergeGeom &m, const float *parts) {
  const int P = m.P, G = m.G, GO = m.GO, S = m.S;
  const int w = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
  const int sg0 = S > 1 ? (int)threadIdx.x / GO : 0;
  const int per = sg0 < S ? (P - sg0 + S - 1) / S : 0;       // parts of this thread
  auto o_offset = [&](int pp, int uu) { return ((pp * G + (uu >> 5)) * kPartialStride + 4 + 4 * (uu & 31)) * 4; };
  u32x4 ob[NB];
  {
    const int u0 = S > 1 ? (int)threadIdx.x % GO : (int)threadIdx.x;
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) ob[jb] = __builtin_amdgcn_raw_buffer_load_b128(m.prs, o_offset(sg0 + S * jb, u0), 0, 16);
  }
  for (int idx = threadIdx.x; idx < P * G; idx += kThreads) {
    const float *pp = parts + (int64_t)idx * kPartialStride;       // part idx / G, head idx % G
    m.sm_m[idx] = __hip_atomic_load(pp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    m.sm_l[idx] = __hip_atomic_load(pp + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  // one wave per head, lane l taking parts l and l + 64 (P <= kMaxParts = 128), the max and
  // the weighted sum of l reduced across the wave (a single thread walking the parts of a head
  // one LDS read after another took about a microsecond of the merge for 12 parts)
  {
    for (int hc = w; hc < G; hc += kWaves) {
      const int p0 = lane, p1 = lane + 64;
      const float m0 = p0 < P ? m.sm_m[p0 * G + hc] : kNegInf, m1 = p1 < P ? m.sm_m[p1 * G + hc] : kNegInf;
      const float M = wave_max(fmaxf(m0, m1));
      const float w0 = m0 == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m0 - M);
      const float w1 = m1 == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m1 - M);
      if (p0 < P) m.sm_w[p0 * G + hc] = w0;
      if (p1 < P) m.sm_w[p1 * G + hc] = w1;
      const float L = wave_sum((p0 < P ? w0 * m.sm_l[p0 * G + hc] : 0.0f) + (p1 < P ? w1 * m.sm_l[p1 * G + hc] : 0.0f));
      if (lane == 0) m.sm_inv[hc] = L > 0.0f ? 1.0f / L : 0.0f;
    }
  }
  __syncthreads();
  for (int oi = 0; oi < m.nout; ++oi) {
    const int u = S > 1 ? (int)threadIdx.x % GO : (int)threadIdx.x + oi * kThreads;
    const int hc = u >> 5;
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j0 = 0; j0 < per; j0 += NB) {
      if (j0 > 0 || oi > 0) {
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) ob[jb] = __builtin_amdgcn_raw_buffer_load_b128(m.prs, o_offset(sg0 + S * (j0 + jb), u), 0, 16);
      }
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
        const float wt = j0 + jb < per ? m.sm_w[(sg0 + S * (j0 + jb)) * G + hc] : 0.0f;
        acc += wt * __builtin_bit_cast(float4_t, ob[jb]);
      }
    }
    if (S > 1) {
      if (sg0 < S) m.sm_red[sg0 * GO + u] = acc;
      __syncthreads();
      if (sg0 == 0)
        for (int s2 = 1; s2 < S; ++s2) acc += m.sm_red[s2 * GO + u];
    }
    if (sg0 == 0 && u < GO) {
      const float4_t r = acc * m.sm_inv[hc];
      const int64_t o = (m.row0 + hc) * kHeadDim + 4 * (u & 31);
      if (m.out_fp32) *(float4_t *)((float *)m.out + o) = r;
      else *(uint2 *)((_Float16 *)m.out + o) = make_uint2(pk(r[0], r[1]), pk(r[2], r[3]));
    }
  }
}

// Per-wave state -> LDS rows for the workgroup merge: m[16], l[16] (log2 units) and
// o[16][kWoStride], heads in natural order.  The rows are 128 dims plus 16 floats of padding:
// the 8 (or 16) lanes of one quarter write 16 bytes of 8 different rows at once, which with
// 512-byte rows all fell on the same LDS banks.
constexpr int kWoStride = kHeadDim + 16;
template <int NSUB>
__device__ __forceinline__ void state_to_lds(State &st, int w, int g, int c, float sl2, float *wm, float *wl, float *wo) {
  if constexpr (NSUB == 1) {
    const float l = quad_sum(st.l);
    if (g == 0) {
      wm[w * 16 + c] = st.m * sl2;
      wl[w * 16 + c] = l;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) *(float4_t *)(wo + ((w * 16 + c) * kWoStride + 16 * k + 4 * g)) = st.o[k];
  } else {
    // lane (c, g): column (subtile c >> 3, head c & 7), accumulator rows dims 16k + 4g + i;
    // the subtile-1 column of a head is lane c ^ 8
    const float l = head_sum2(st.l);
    if (g == 0 && c < 8) {
      wm[w * 16 + c] = st.m * sl2;
      wl[w * 16 + c] = l;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float4_t o = st.o[k];
      o[0] += __shfl_xor(o[0], 8);
      o[1] += __shfl_xor(o[1], 8);
      o[2] += __shfl_xor(o[2], 8);
      o[3] += __shfl_xor(o[3], 8);
      if (c < 8) *(float4_t *)(wo + ((w * 16 + c) * kWoStride + 16 * k + 4 * g)) = o;
    }
  }
}

// The call's new token of (b, h), quantized in this launch (the update phase of page "NVFP4
// KV缓存技术详解" §2.1: quantize the new token and append it): for each of its 16-value blocks
// of K and V, s = E4M3_RNE(amax / 6) and E2M1 codes, stored at slot pq_slot of the young arena
// exactly as the append kernel stores them (a slot that opens a block first clears the block:
// the slots past a tier's length hold zero bytes).  The decoded values (code * s, exact in
// fp16) become slot 0 of a one-token fp16 residual (K [16][128], V [1][128][16]) that this
// workgroup attends to.  Streaming workgroups leave the slot out; the words they read may hold
// it or not, and its fields meet zero weights.
__device__ __forceinline__ void nvfp4_append_token(const DecodeArgs &a, int bh) {
  const int s = (int)(a.pq_slot % kBlock);
  uint8_t *blkp = a.pq_arena + (int64_t)bh * a.pq_bh_stride + (a.pq_slot / kBlock) * (int64_t)kNvfp4BlockBytes;
  if (s == 0) {
    for (int i = threadIdx.x; i < (int)(kNvfp4BlockBytes / 16); i += kThreads) ((uint4 *)blkp)[i] = uint4{0u, 0u, 0u, 0u};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
  if (threadIdx.x < 16) {
    const int kv = threadIdx.x >> 3, nb = threadIdx.x & 7;   // tensor, 16-value block
    const uint16_t *src = (kv ? a.pend_v : a.pend_k) + ((int64_t)bh * a.pend_src_ntok + a.pend_src_tok0) * kHeadDim + 16 * nb;
    const uint4 x0 = *(const uint4 *)src, x1 = *(const uint4 *)(src + 8);
    const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t amax = 0;                                   // |x| of finite fp16 orders like its bits
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = max(amax, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    const uint32_t sb = f32_to_e4m3((float)__builtin_bit_cast(_Float16, (uint16_t)amax) / 6.0f);
    const float sc = e4m3_to_f32(sb);
    uint32_t cw[2] = {0u, 0u};                           // the 16 codes, element i at nibble i
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float x = (float)__builtin_bit_cast(_Float16, (uint16_t)(i & 1 ? w[i >> 1] >> 16 : w[i >> 1] & 0xFFFFu));
      cw[i >> 3] |= e2m1_code(x, sc) << (4 * (i & 7));
    }
    // decoded values, as the stream decodes them: the hardware E2M1 -> fp16 conversion times
    // the E4M3 scale in fp16 (exact)
    const uint32_t s2 = e4m3_pair(sb * 0x0101u, false);
    const half8_t d0 = unpack_fp4(cw[0], s2, s2, s2, s2), d1 = unpack_fp4(cw[1], s2, s2, s2, s2);
    const u32x4 d0w = __builtin_bit_cast(u32x4, d0), d1w = __builtin_bit_cast(u32x4, d1);
    const uint32_t dw[8] = {d0w.x, d0w.y, d0w.z, d0w.w, d1w.x, d1w.y, d1w.z, d1w.w};
    uint16_t *rk = (uint16_t *)(a.res_base + (int64_t)bh * a.res_bh_stride);   // K [16][128]
    uint16_t *rv = rk + (int64_t)a.res_len * kHeadDim;                          // V [1][128][16]
    if (kv == 0) {
      // K: the 16 dims are fields 16 (nb & 1) .. +15 of the lane string of quarter nb >> 1
      const int lane = 16 * (nb >> 1) + (s & 15);
      *(uint2 *)(blkp + ((s >> 4) * 64 + lane) * 16 + 8 * (nb & 1)) = make_uint2(cw[0], cw[1]);
      blkp[kNvKs + ((s >> 4) * 64 + lane) * 2 + (nb & 1)] = (uint8_t)sb;
      *(uint4 *)(rk + 16 * nb) = make_uint4(dw[0], dw[1], dw[2], dw[3]);
      *(uint4 *)(rk + 16 * nb + 8) = make_uint4(dw[4], dw[5], dw[6], dw[7]);
    } else {
      // V: dim 16 nb + i is nibble e of word nb % 4 of lane 16 g + i in chunk 2 w + nb / 4
      const int wp = s >> 5, g = (s >> 2) & 3, tt = (s >> 4) & 1, e = 4 * tt + (s & 3);
      uint32_t *vw = (uint32_t *)(blkp + kNvVc + ((2 * wp + (nb >> 2)) * 64 + 16 * g) * 16 + (nb & 3) * 4);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t code = (cw[i >> 3] >> (4 * (i & 7))) & 0xFu;
        vw[4 * i] = (vw[4 * i] & ~(0xFu << (4 * e))) | (code << (4 * e));
      }
      blkp[kNvVs + ((4 * wp + g) * 8 + nb) * 8 + 4 * tt + (s & 3)] = (uint8_t)sb;
#pragma unroll
      for (int i = 0; i < 16; ++i) rv[(16 * nb + i) * 16] = (uint16_t)(i & 1 ? dw[i >> 1] >> 16 : dw[i >> 1] & 0xFFFFu);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// OCC = workgroups per CU the launch is planned for (the bound on VGPRs follows from it).
// OCC = 3 holds only the INT2 (groups of 64, per-token K) step: the host launches it only when
// every tier of the call has that format; its VGPRs then fit three waves per SIMD, which
// hides more of the step's latency (128K INT2 layer 171 -> 156 us, same box).
template <int NSUB, int OCC>
__global__ __launch_bounds__(kThreads, OCC) void decode_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const bool valid_head = (NSUB == 2 ? (c & 7) : c) < a.G;
  const Item it = a.rag ? decode_item_ragged(a, blockIdx.x) : decode_item(a, blockIdx.x);
  __shared__ int s_chunk;
  if (a.pq_nvfp4 && it.has_res) nvfp4_append_token(a, it.bh);
  if (it.pend_count > 0 && it.has_res) {
    // this call's new tokens go to the residual: copied here, before this workgroup (the only
    // reader of the residual in the launch) reads it
    const int64_t src0 = ((int64_t)it.bh * a.pend_src_ntok + it.pend_src_tok0) * kHeadDim;
    residual_store(a.pend_k + src0, a.pend_v + src0, it.pend_count, it.pend_slot0,
                   (uint8_t *)(a.res_base + (int64_t)it.bh * a.res_bh_stride), a.res_len, threadIdx.x, kThreads);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
  State st;
#pragma unroll
  for (int k = 0; k < 8; ++k) st.o[k] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  st.vmask = __builtin_amdgcn_ballot_w64(valid_head);

  // part 0 opens the arrival counter early, so that the arrivals find it open (wave 3 loads no
  // blocks, so its wait here holds up nothing else)
  if (it.part == 0 && w == kWaves - 1 && lane == 0) counter_open(a.counters + (int64_t)it.bh * kCtrStride, a.epoch);
  // residual only (no quantized tier yet)
  if (it.seg < 0 && it.has_res) residual_part<NSUB>(a, it, q_group(a, it.bh), w, g, c, valid_head, st);
  if (it.seg >= 0 && w == kWaves - 1) {
    // wave 3 copies the group's query rows into LDS past the ring: it loads no blocks, so its
    // wait for these loads waits for nothing else, and the other waves read the rows from LDS
    // (after the segment's first barrier) instead of waiting for global loads while their
    // first blocks are in flight
    const int qbytes = a.G * kHeadDim * 2;
    const uint8_t *qsrc = (const uint8_t *)q_group(a, it.bh);
    for (int off = lane * 16; off < qbytes; off += 1024)
      *(uint4 *)(smem + a.q_lds_off + off) = *(const uint4 *)(qsrc + off);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  if (it.seg >= 0) {
    const DecodeSeg &sg = a.rag ? (const DecodeSeg &)((ConstRagSeq *)a.rag)[it.bh / a.H].seg[it.seg] : a.seg[it.seg];
#define KVQ_SEG(F, GS) stream_segment<F, GS, NSUB>(a, sg, it, smem, &s_chunk, w, g, c, valid_head, st)
#define KVQ_AFFINE_SEG(F)                  \
  case F:                                  \
    if (sg.gs == kKc) KVQ_SEG(F, kKc);     \
    else if (sg.gs == 32) KVQ_SEG(F, 32);  \
    else if (sg.gs == 128) KVQ_SEG(F, 128); \
    else KVQ_SEG(F, 64);                   \
    break;
    if constexpr (OCC == 3) {
      KVQ_SEG(kFmtInt2, 64);
    } else {
      switch (sg.fmt) {
        KVQ_AFFINE_SEG(kFmtInt2)
        KVQ_AFFINE_SEG(kFmtInt4)
        KVQ_AFFINE_SEG(kFmtInt8)
        case kFmtFp8: KVQ_SEG(kFmtFp8, kGroup); break;
        case kFmtFp16: KVQ_SEG(kFmtFp16, kGroup); break;
        case kFmtMxfp4: KVQ_SEG(kFmtMxfp4, kGroup); break;
        default: KVQ_SEG(kFmtNvfp4, kGroup); break;
      }
    }
#undef KVQ_AFFINE_SEG
#undef KVQ_SEG
  }
  // ---- merge the four waves in LDS: per wave m[16], l[16], o[16][128] (m in log2 units)
  float *wm = (float *)smem;                       // [4][16]
  float *wl = wm + kWaves * 16;                    // [4][16]
  float *wo = wl + kWaves * 16;                    // [4][16][kWoStride]
  state_to_lds<NSUB>(st, w, g, c, a.scale_log2, wm, wl, wo);
  __syncthreads();

  const int G = a.G;
  float *part = a.partials + ((int64_t)it.bh * a.part_stride + it.part) * G * kPartialStride;
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
      O += wt * wo[(v * 16 + hc) * kWoStride + d];
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
    uint64_t *cnt = a.counters + (int64_t)it.bh * kCtrStride;
    const uint64_t old = __hip_atomic_fetch_add(cnt, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (int)counter_result(cnt, a.epoch, old) + 1 == it.items_total;
  }
  __syncthreads();
  if (!s_last) return;

  const int P = it.items_total;
  const float *parts = a.partials + (int64_t)it.bh * a.part_stride * G * kPartialStride;
  float *sm_m = (float *)smem;            // [P][G]
  float *sm_w = sm_m + P * G;             // [P][G] weights, after the max is known
  float *sm_l = sm_w + P * G;             // [P][G]
  float *sm_inv = sm_l + P * G;           // [G]
  float4_t *sm_red = (float4_t *)(smem + ((3 * P * G + G) * 4 + 15) / 16 * 16);   // [S][G * 32]
  // The weighted sum reads o of every (part, head) as 16-byte loads with the agent-scope cache
  // policy (sc1, as the partials were written: past the writer's XCD L2), through a buffer
  // descriptor bounded by this (b, h)'s partials (a read past them returns zeros).  Thread t
  // takes float4 output u of the G * 32 and the parts sg, sg + S, ...: with more than 16 parts
  // and G < 8, S thread groups share an output (at most 16 parts each where the threads allow),
  // their sums added in a fixed order, so that deterministic splits stay reproducible.  A
  // thread's first batch of loads goes out before the (m, l) reads, so that the two latencies
  // overlap.
  const int GO = G * 32;
  const int S = GO >= kThreads ? 1 : max(1, min(kThreads / GO, (P + 15) / 16));
  const int per = (P + S - 1) / S;                                  // parts per thread, at most
  const __amdgpu_buffer_rsrc_t prs =
      __builtin_amdgcn_make_buffer_rsrc((void *)parts, 0, P * G * kPartialStride * 4, 0x00020000);
  const int b = it.bh / a.H, h = it.bh % a.H;
  const MergeGeom mg{P, G, GO, S, GO > kThreads ? 2 : 1, prs, sm_m, sm_w, sm_l, sm_inv, sm_red,
                     (int64_t)b * a.H * G + (int64_t)h * G, a.out, a.out_fp32};
  if (per <= 1) merge_tail<1>(mg, parts);
  else if (per <= 2) merge_tail<2>(mg, parts);
  else if (per <= 4) merge_tail<4>(mg, parts);
  else if (per <= 8) merge_tail<8>(mg, parts);
  else merge_tail<16>(mg, parts);
  // Every other workgroup of this (b, h) has arrived, each after all its memory operations
  // completed (its cursor fetch-adds included), so no access of this call to the (b, h)'s
  // arrival counter or cursors is left: set them back to zero for the next call.
  if ((int)threadIdx.x < 1 + a.nseg) {
    uint64_t *wd = (threadIdx.x == 0 ? a.counters : a.seg[threadIdx.x - 1].cursors) + (int64_t)it.bh * kCtrStride;
    __hip_atomic_store(wd, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

// LDS of the largest block ring among the call's tiers; the query rows follow it.
static size_t decode_ring_bytes(const DecodeArgs &a) {
  size_t ring = 0;
  for (int s = 0; s < a.nseg; ++s) {
    const int bb = (int)block_bytes(a.seg[s].fmt, a.seg[s].gs);
    ring = std::max(ring, (size_t)decode_ring_depth(bb) * bb);
  }
  return ring;
}

size_t decode_lds_bytes(const DecodeArgs &a) {
  const size_t stream = decode_ring_bytes(a) + (size_t)a.G * kHeadDim * 2;
  const size_t merge = (size_t)kWaves * (16 + 16 + 16 * kWoStride) * sizeof(float);
  return std::max(stream, merge);
}

int decode_occupancy(const int *fmt, const int *gs, int n, int G) {
  if (n == 0 || G > 8) return 2;
  for (int i = 0; i < n; ++i)
    if (fmt[i] != kFmtInt2 || gs[i] != 64) return 2;
  return 3;
}

hipError_t launch_decode(const DecodeArgs &a, int num_wg, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)decode_kernel<1, 2>, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxDecodeLds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void *)decode_kernel<2, 2>, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxDecodeLds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void *)decode_kernel<2, 3>, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxDecodeLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  DecodeArgs b = a;
  b.q_lds_off = (int)decode_ring_bytes(a);
  const size_t lds = decode_lds_bytes(a);
  if (lds > (size_t)kMaxDecodeLds) return hipErrorInvalidValue;
  // two 16-slot subtiles share the MFMA columns when at most 8 query heads share a kv head
  if (a.occ == 3) {
    // only INT2 tiers with groups of 64 (decode_occupancy), G <= 8
    if (a.G > 8 || lds * 3 > 160 * 1024) return hipErrorInvalidValue;
    for (int i = 0; i < a.nseg; ++i)
      if (a.seg[i].fmt != kFmtInt2 || a.seg[i].gs != 64) return hipErrorInvalidValue;
    decode_kernel<2, 3><<<(unsigned)num_wg, kThreads, lds, s>>>(b);
  } else if (a.G <= 8) {
    decode_kernel<2, 2><<<(unsigned)num_wg, kThreads, lds, s>>>(b);
  } else {
    decode_kernel<1, 2><<<(unsigned)num_wg, kThreads, lds, s>>>(b);
  }
  return hipGetLastError();
}

}  // namespace kvq
