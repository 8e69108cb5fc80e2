// Quantize-and-pack kernels of libkvq (gfx950): affine INT2/INT4/INT8 groups of 64 and
// NVFP4 blocks of 16, written into 128-slot cache blocks, plus the fp16 residual copy.
//
// Affine: page "KV缓存量化技术：提升大模型长文本生成效率" §2.1 (S = (max-min)/(2^n-1),
// Z = round(-min/S), groups of 64); codes q = clamp(round(x/S) + Z, 0, 2^n-1).
// NVFP4: page "NVFP4 KV缓存技术详解" §2.1 (16 values share an FP8 scale) and §4.2
// (clip to 6): s = E4M3_RNE(amax/6), code = sign*8 + E2M1_RNE(min(|x|/s, 6)).
//
// Every rounding is decided exactly:
//  * S: fp64 (max - min) is exact for fp16 inputs; the fp64 quotient by 2^n-1 is never
//    closer to an fp16 rounding midpoint than its own error, so one fp64 -> fp16 RNE of
//    it equals the exact rounding.
//  * Z: fp64 -min/S, then round-half-even (same argument with half-integers).
//  * codes: k = rint(x * (1/S)) is within one of round(x/S); the remainder x - k*S is exact
//    in fp32 (one fma), and comparing it with S/2 fixes k, ties to even.
//  * E4M3: fp32 amax/6 (correctly rounded) is never closer to an E4M3 midpoint than its
//    error unless it lies on it exactly; it is then rounded to 3 mantissa bits, ties even.
//  * E2M1: |x| is compared with midpoint*s, both exact in fp32.
#include "kvq_internal.h"
#include "kvq_fp_codes.h"
#include "kvq_rescopy.h"

#include <cmath>
#include <type_traits>

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kRowHalves = 136;  // LDS row stride (halves) of the staged fp16 tokens

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// the 8 fp16 values of a 16-byte LDS read, as floats
__device__ __forceinline__ void unpack8(const uint4 &v, float (&x)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = h2f((uint16_t)(w[i] & 0xFFFFu));
    x[2 * i + 1] = h2f((uint16_t)(w[i] >> 16));
  }
}

// Round a double to the nearest binary16, ties to even; zero becomes +0.
__device__ uint16_t f64_to_f16_rne(double v) {
  if (v == 0.0) return 0;
  uint16_t sign = v < 0 ? 0x8000 : 0;
  double a = fabs(v);
  if (a >= 65520.0) return sign | 0x7C00;
  if (a < 6.103515625e-05) {                        // below 2^-14: multiples of 2^-24
    double k = rint(a * 16777216.0);                // exact scaling, round half even
    return sign | (uint16_t)k;                      // k = 1024 is the smallest normal
  }
  uint64_t bits = (uint64_t)__double_as_longlong(a);
  int e = (int)((bits >> 52) & 0x7FF) - 1023;       // -14..15
  uint64_t m = bits & ((1ull << 52) - 1);
  uint32_t keep = (uint32_t)(m >> 42);
  uint64_t rem = m & ((1ull << 42) - 1), half = 1ull << 41;
  if (rem > half || (rem == half && (keep & 1))) ++keep;
  if (keep == 1024) { keep = 0; ++e; }
  if (e > 15) return sign | 0x7C00;
  return sign | (uint16_t)((e + 15) << 10) | (uint16_t)keep;
}


// round-half-even of x/S for fp16-valued x and S > 0 with |x/S| < 2^20; inv ~ 1/S.  k is
// within one of the answer; the exact remainder r = x - k S decides: |r| > S/2, or |r| = S/2
// with k odd, moves k one step towards r.
__device__ __forceinline__ float div_rne(float x, float S, float inv) {
  const float k = rintf(x * inv);
  const float r = fmaf(-k, S, x);   // exact
  const float h = 0.5f * S;         // exact
  const float ar = fabsf(r);
  const bool odd = ((int)k & 1) != 0;
  return (ar > h || (ar == h && odd)) ? k + copysignf(1.0f, r) : k;
}

__device__ __forceinline__ uint32_t affine_code(float x, float S, float inv, float Z, int qmax) {
  float q = div_rne(x, S, inv) + Z;
  q = fminf(fmaxf(q, 0.0f), (float)qmax);
  return (uint32_t)q;
}

// Bits of S = RN16((mx - mn) / qmax), mx > mn: in fp32 where that provably gives the same
// fp16 value, else in fp64.  The difference is used only when exact (its TwoSum error is 0);
// r = d * RN(1/qmax) is then within 2 fp32 ulps of d / qmax, so rounding r to fp16 (to
// nearest, ties to even) matches unless r lies within a few ulps of a midpoint between fp16
// values (low 13 mantissa bits near 0x1000) or outside the normal fp16 range.
__device__ __forceinline__ uint32_t scale_bits(float mn, float mx, int qmax) {
  const float d = mx - mn;
  const float bb = d - mx;
  const float err = (mx - (d - bb)) + (-mn - bb);
  const float r = d * (1.0f / (float)qmax);
  const uint32_t m13 = __float_as_uint(r) & 0x1FFFu;
  if (err == 0.0f && r >= 0x1p-14f && r < 65504.0f && (m13 < 0x1000u - 8u || m13 > 0x1000u + 8u))
    return __builtin_bit_cast(uint16_t, (_Float16)r);
  return f64_to_f16_rne(((double)mx - (double)mn) / (double)qmax);
}

// Bits of Z = RN16(clamp(RNE(-mn / S), +-65504)) for fp16 values mn and S > 0, a zero always
// +0: by the exact remainder in fp32 (div_rne) where |mn / S| < 2^19, else in fp64.
__device__ __forceinline__ uint32_t zero_bits(float mn, float S) {
  const float inv = 1.0f / S;
  if (fabsf(mn) * inv < 0x1p19f) {
    const float z = fminf(fmaxf(div_rne(-mn, S, inv), -65504.0f), 65504.0f) + 0.0f;   // -0 + 0 = +0
    return __builtin_bit_cast(uint16_t, (_Float16)z);
  }
  double z = rint(-(double)mn / (double)S);
  z = fmin(fmax(z, -65504.0), 65504.0);
  return f64_to_f16_rne(z);
}

// Raise the block's eps (float bits in *eps, non-negative) to the bound of a group whose values
// lie in [mn, mx], whose 1 / S is inv and whose zero point is Z: (max |x / S| + |Z|) 2^-20,
// eight times the largest error of RN(x * inv + Z) against x / S + Z in the group (the
// rounding of inv and that of the fused multiply-add, each within (|x / S| + |Z|) 2^-24).
__device__ __forceinline__ void note_eps(uint32_t *eps, float mn, float mx, float inv, float Z) {
  atomicMax(eps, __float_as_uint((fmaxf(fabsf(mn), fabsf(mx)) * inv + fabsf(Z)) * 0x1p-20f));
}


// Block layout (128 slots, head_dim 128).  K codes: 4 parts w x 2 tiles u x 64 lanes
// (g = lane >> 4, c = lane & 15) x 4n bytes (NVFP4 16) of slot 32w + 16u + c, stored in
// chunks of min(16, 4n) bytes; lane field f holds dim 64(f >> 4) + 16g + (f & 15) (affine)
// or 32g + f (NVFP4, MXFP4).  V codes: 4 parts w x 64 lanes x 8n bytes in 16-byte chunks;
// lane field phi holds dim 16k + c and slot 32w + 16(e >> 2) + 4g + (e & 3), (k, e) per
// format below.
__device__ __forceinline__ int k_lane_dim(int fmt, int g, int f) {
  return (fmt == kFmtNvfp4 || fmt == kFmtMxfp4) ? 32 * g + f : 64 * (f >> 4) + 16 * g + (f & 15);
}
// Affine groups of 32: field f of quarter g holds dim 32j + 8g + e, (j, e) being f's place among
// the decode kernel's MFMA operands (k-step j, element e), so that every step covers one group.
__device__ __forceinline__ int k_lane_dim32(int fmt, int g, int f) {
  int j, e;
  if (fmt == kFmtInt2) {
    const int r = f & 15;
    j = 2 * (f >> 4) + ((f >> 2) & 1);
    e = 2 * (r & 3) + (r >> 3);
  } else if (fmt == kFmtInt4) {
    const int r = f & 7;
    j = f >> 3;
    e = 2 * (r & 3) + (r >> 2);
  } else {
    const int r = f & 7;
    j = f >> 3;
    e = 4 * (r >> 2) + 2 * (r & 1) + ((r >> 1) & 1);
  }
  return 32 * j + 8 * g + e;
}
// Dim fed by element e of MFMA k-step j in lane quarter g of the groups-of-64 K lanes: the field
// f that (j, e) reads, through k_lane_dim.
__device__ __forceinline__ int k_operand_dim(int fmt, int g, int j, int e) {
  int f;
  if (fmt == kFmtInt2) f = 16 * (j >> 1) + 4 * (j & 1) + (e >> 1) + 8 * (e & 1);
  else if (fmt == kFmtInt4) f = 8 * j + (e >> 1) + 4 * (e & 1);
  else f = 8 * j + 4 * (e >> 2) + ((e >> 1) & 1) + 2 * (e & 1);
  return k_lane_dim(fmt, g, f);
}

__device__ __forceinline__ void v_field(int fmt, int phi, int &k, int &e) {
  if (fmt == kFmtInt2) {
    const int u = phi >> 4, m = phi & 15;
    k = 2 * u + ((m >> 2) & 1);
    e = 2 * (m & 3) + (m >> 3);
  } else if (fmt == kFmtInt8 || fmt == kFmtFp8) {   // FP8 codes sit where INT8 codes do
    const int u = phi >> 2, b = phi & 3;
    k = u >> 1;
    e = 4 * (u & 1) + 2 * (b & 1) + (b >> 1);
  } else if (fmt == kFmtMxfp4) {                       // a byte: one slot, dims 16(2m) + c, 16(2m+1) + c
    k = 2 * (phi >> 4) + (phi & 1);
    e = (phi >> 1) & 7;
  } else {
    const int v = phi & 7;
    k = phi >> 3;
    e = fmt == kFmtNvfp4 ? v : 2 * (v & 3) + (v >> 2);
  }
}

// FP16 block: the staged values themselves.  K chunk ((tile*4 + i)*64 + lane) holds dims
// 32g + 8i .. +7 of slot 16 tile + c; V chunk ((w*8 + k)*64 + lane) at kF16Vc holds dim 16k + c
// of slots 32w + 16(e >> 2) + 4g + (e & 3), e = 0..7.  Slots before lo keep their stored
// values; slots [hi, zhi) are cleared.
__device__ void store_fp16_block(const uint16_t *xs, uint8_t *blkp, int kv, int lo, int hi, int zhi, int tid) {
  constexpr int kChunks = kBlock * kHeadDim * 2 / 16;   // 16-byte chunks of K (or V)
  if (kv == 0) {
    for (int id = tid; id < kChunks; id += kThreads) {
      const int lane = id & 63, i = (id >> 6) & 3, tile = id >> 8;
      const int slot = 16 * tile + (lane & 15);
      if (slot < lo || slot >= zhi) continue;
      uint4 v = {0u, 0u, 0u, 0u};
      if (slot < hi) v = *(const uint4 *)&xs[slot * kRowHalves + 32 * (lane >> 4) + 8 * i];
      *(uint4 *)(blkp + (size_t)id * 16) = v;
    }
  } else {
    for (int id = tid; id < kChunks; id += kThreads) {
      const int lane = id & 63, k = (id >> 6) & 7, w = id >> 9;
      const int s0 = 32 * w + 4 * (lane >> 4), d = 16 * k + (lane & 15);
      uint32_t word[4], keep[4];
      bool any = false;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        word[m] = keep[m] = 0u;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int e = 2 * m + hh;
          const int slot = s0 + 16 * (e >> 2) + (e & 3);
          if (slot < lo) {
            keep[m] |= 0xFFFFu << (16 * hh);
          } else if (slot < zhi) {
            any = true;
            if (slot < hi) word[m] |= (uint32_t)xs[slot * kRowHalves + d] << (16 * hh);
          }
        }
      }
      if (!any) continue;
      uint4 *dst = (uint4 *)(blkp + kF16Vc + (size_t)id * 16);
      uint4 out = {word[0], word[1], word[2], word[3]};
      if (keep[0] | keep[1] | keep[2] | keep[3]) {
        const uint4 old = *dst;
        out.x |= old.x & keep[0]; out.y |= old.y & keep[1];
        out.z |= old.z & keep[2]; out.w |= old.w & keep[3];
      }
      *dst = out;
    }
  }
}

// Decoded values S (q - Z) of one full affine block (groups of 64, n-bit codes) into the
// staging rows: block slot s goes to row s - row_off when that row is in [lo, hi).  The
// product is exact in double; it is clamped to +-65504 and rounded to fp16, ties to even.
// The words are walked in storage order, each mapped to its slot and dims as the layout
// above places them (K: a word holds consecutive dims of one slot; V: fields per v_field).
__device__ void stage_affine_decoded(const uint8_t *yb, int n, int kv, int row_off, int lo, int hi, uint16_t *xs,
                                     int tid) {
  const int F = 32 / n, qmax = (1 << n) - 1, nwords = 512 * n;
  auto dec = [&](const uint8_t *sp, const uint8_t *zp, uint32_t q) -> uint16_t {
    const double S = (double)h2f(*(const uint16_t *)sp), Z = (double)h2f(*(const uint16_t *)zp);
    double x = S * ((double)q - Z);
    x = fmin(fmax(x, -65504.0), 65504.0);
    return f64_to_f16_rne(x);
  };
  if (kv == 0) {
    const int cb = min(16, 4 * n), K = 4 * n / cb;
    for (int w = tid; w < nwords; w += kThreads) {
      const int ci = 4 * w / cb, in_chunk = 4 * w % cb;
      const int lane = ci & 63, t2 = ci >> 6;
      const int r = t2 % K, wu = t2 / K;
      const int slot = 16 * wu + (lane & 15), row = slot - row_off;
      if (row < lo || row >= hi) continue;
      const int f0 = (r * cb + in_chunk) / 4 * F;
      const int d0 = 64 * (f0 >> 4) + 16 * (lane >> 4) + (f0 & 15), grp = d0 >> 6;
      const uint8_t *m = yb + aff_km(n) + (slot >> 4) * 128 + 2 * (2 * (slot & 15) + grp);
      const uint32_t word = *(const uint32_t *)(yb + 4 * (size_t)w);
      for (int k = 0; k < F; ++k) xs[row * kRowHalves + d0 + k] = dec(m, m + 64, (word >> (k * n)) & qmax);
    }
  } else {
    const int chunks = n / 2, fmt = n;
    for (int w = tid; w < nwords; w += kThreads) {
      const int lane = (w >> 2) & 63, pc = w >> 8;
      const int part = pc / chunks, omega = 4 * (pc % chunks) + (w & 3);
      const int g = lane >> 4, c = lane & 15;
      const uint32_t word = *(const uint32_t *)(yb + aff_vc(n, 2) + 4 * (size_t)w);
      for (int j = 0; j < F; ++j) {
        int k, e;
        v_field(fmt, omega * F + j, k, e);
        const int slot = 32 * part + 16 * (e >> 2) + 4 * g + (e & 3), row = slot - row_off;
        if (row < lo || row >= hi) continue;
        const int d = 16 * k + c, grp = d >> 6;
        const uint8_t *m = yb + aff_vm(n, 2) + ((slot >> 4) * 4 + ((slot & 15) >> 2)) * 32 + 8 * grp + 2 * (slot & 3);
        xs[row * kRowHalves + d] = dec(m, m + 16, (word >> (j * n)) & qmax);
      }
    }
  }
}

// REFILL: the launch also refills the residual it flushes (cp_count > 0); a separate
// instantiation, so that the other launches (the bulk prefill among them) keep their registers.
template <int FMT, int GS, bool REFILL>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantArgs a, int64_t blk0, int64_t nblk) {
  constexpr bool kMx = FMT == kFmtMxfp4;
  constexpr bool kNv = FMT == kFmtNvfp4 || kMx;          // E2M1 codes (NVFP4 or MXFP4 scales)
  constexpr bool kF8 = FMT == kFmtFp8;                   // fixed scale: codes only
  constexpr bool kF16 = FMT == kFmtFp16;                 // the values themselves
  constexpr bool kAffine = is_affine(FMT);
  constexpr int kBits = kNv ? 4 : kF8 ? 8 : kF16 ? 16 : FMT;
  constexpr int kRowBytes = 16 * kBits;           // bytes per code row (128 fields)
  constexpr int kWordsPerRow = kRowBytes / 4;
  constexpr int kQmax = (1 << kBits) - 1;
  constexpr size_t kBlockBytes = block_bytes(FMT, GS);
  constexpr bool kKcK = GS == kKc;                       // K per channel (V in groups of 64)
  constexpr int NG = kKcK ? 2 : kHeadDim / GS;           // affine groups per token (V's, per channel)
  constexpr int GSV = kKcK ? kGroup : GS;                 // head_dim group width of per-token groups

  // 34.8 KB of staged tokens and 1-3 KB of metadata: four workgroups fit in a CU
  constexpr int kMeta = kMx ? 4 : kNv ? 8 : NG;  // affine: S per group; NVFP4: per 16; MXFP4: per 32
  constexpr int kAffMeta = kNv ? 1 : NG;
  __shared__ __align__(16) uint16_t xs[kBlock * kRowHalves];
  __shared__ float mS[kBlock][kMeta];
  __shared__ float mInv[kBlock][kAffMeta];
  __shared__ float mZ[kBlock][kAffMeta];
  // largest eps_g of the block's affine groups (float bits; see the codes below)
  __shared__ uint32_t s_eps;

  const int tid = threadIdx.x;
  if (tid == 0) s_eps = 0u;
  // a.nsplit workgroups per block, workgroup `sub` taking the slots [ps, pe) of one or more
  // whole 32-slot parts: every code word and every (S, Z) belongs to one part, so the
  // workgroups of a block write disjoint words
  const int nsplit = a.nsplit, sub = (int)(blockIdx.x % (unsigned)nsplit);
  const int64_t blk = blk0 + blockIdx.x / (unsigned)nsplit;
  const int ps = sub * (kBlock / nsplit), pe = ps + kBlock / nsplit;
  const int h = blockIdx.y, b = blockIdx.z >> 1, kv = blockIdx.z & 1;
  const int64_t bstart = blk * kBlock;
  const int lo = max((int)(max(a.dst_slot0, bstart) - bstart), ps);
  const int hi_blk = (int)(min(a.dst_slot0 + a.count, bstart + kBlock) - bstart);
  const int hi = max(lo, min(hi_blk, pe));
  const bool last = blk == blk0 + nblk - 1;
  const int zhi = max(hi, min(last ? kBlock : hi_blk, pe));   // slots [hi, zhi) are cleared
  if (lo >= zhi) return;                          // a part before this append's first slot
  uint8_t *blkp = a.arena + (int64_t)(b * a.H + h) * a.arena_bh_stride + blk * (int64_t)kBlockBytes;
  const int64_t tok_off = a.src_tok0 + bstart - a.dst_slot0;   // source index of slot 0

  // ---- stage the source tokens of slots [lo, hi) in LDS as fp16 rows (none when this
  // workgroup's parts only clear slots past the append)
  if (hi == lo) {
  } else if (a.src_kind == 2) {
    // slots [lo, hi) come from one block of the source arena
    const int64_t s0 = tok_off + lo;
    const uint8_t *yb = a.src_arena + (int64_t)(b * a.H + h) * a.src_bh_stride +
                        (s0 / kBlock) * (int64_t)block_bytes(a.src_fmt, kGroup);
    stage_affine_decoded(yb, a.src_fmt, kv, (int)(tok_off - s0 / kBlock * kBlock), lo, hi, xs, tid);
  } else if (a.src_kind == 0 || kv == 0) {
    const uint8_t *src;
    int64_t row_stride;
    if (a.src_kind == 0) {
      src = (const uint8_t *)(kv ? a.v_src : a.k_src) + (int64_t)(b * a.H + h) * a.src_ntok * 256;
      row_stride = 256;
    } else {
      src = a.res_base + (int64_t)(b * a.H + h) * a.res_bh_stride;   // residual K [R][128]
      row_stride = 256;
    }
    // all of a thread's loads (up to 8 x 16 bytes) are issued before the first LDS write, so
    // that their latencies overlap
    const int nchunks = (hi - lo) * 16;
    constexpr int kPer = kBlock * 16 / kThreads;
    // rows of 256 bytes: chunk c of the staged rows lies c * 16 bytes past the first row
    // (a uniform 64-bit base and a 32-bit per-lane offset)
    const uint8_t *row0 = src + (tok_off + lo) * row_stride;
    uint4 v[kPer];
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      // unconditional (a branch around each load makes the compiler wait for it at the join);
      // past the staged rows the index repeats the last chunk
      const int c = min(tid + t * kThreads, nchunks - 1);
      // (nontemporal: each source row is read once)
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 w = __builtin_nontemporal_load((const u32x4 *)(row0 + (uint32_t)c * 16u));
      v[t] = make_uint4(w.x, w.y, w.z, w.w);
    }
    // the loaded registers pass through empty asm statements: the loads stay here, all issued
    // before the first store, rather than being sunk into the stores' branches (a "memory"
    // clobber would do the same but sends the array through scratch)
#pragma unroll
    for (int t = 0; t < kPer; ++t) asm volatile("" : "+v"(v[t].x), "+v"(v[t].y), "+v"(v[t].z), "+v"(v[t].w));
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      const int c = tid + t * kThreads;
      if (c < nchunks) *(uint4 *)&xs[(lo + c / 16) * kRowHalves + (c % 16) * 8] = v[t];
    }
  } else {
    // residual V: [R/16][128][16] fp16, 16 slots of one dim together.  Runs of 8 residual
    // slots starting at a multiple of 8 come as one 16-byte load per dim (scattered into 8 LDS
    // rows); the slots before the first and after the last such run one value at a time.
    const uint16_t *src = (const uint16_t *)(a.res_base + (int64_t)(b * a.H + h) * a.res_bh_stride + (int64_t)a.res_len * 256);
    const int t_lo = (int)(tok_off + lo), t_hi = (int)(tok_off + hi);   // residual slots of rows [lo, hi)
    const int r0 = (t_lo + 7) & ~7, r1 = t_hi & ~7;
    const int nrun = r1 > r0 ? (r1 - r0) >> 3 : 0;
    const int head = nrun ? r0 - t_lo : t_hi - t_lo;                  // loose slots before the runs
    for (int e = tid; e < nrun * kHeadDim; e += kThreads) {
      const int t0 = r0 + 8 * (e >> 7), d = e & 127;
      const uint4 x = *(const uint4 *)(src + ((t0 >> 4) * kHeadDim + d) * 16 + (t0 & 15));
      uint16_t *dst = &xs[(t0 - (int)tok_off) * kRowHalves + d];
      const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dst[(2 * i) * kRowHalves] = (uint16_t)(w4[i] & 0xFFFFu);
        dst[(2 * i + 1) * kRowHalves] = (uint16_t)(w4[i] >> 16);
      }
    }
    const int nloose = head + (nrun ? t_hi - r1 : 0);
    for (int e = tid; e < nloose * kHeadDim; e += kThreads) {
      const int i = e >> 7, d = e & 127;
      const int t = i < head ? t_lo + i : r1 + (i - head);
      xs[(t - (int)tok_off) * kRowHalves + d] = src[((t >> 4) * kHeadDim + d) * 16 + (t & 15)];
    }
  }
  __syncthreads();
  // A flush followed by the refill of the residual it read: each workgroup refills the residual
  // slots it staged with the caller's last cp_count tokens (the slots of different workgroups are
  // disjoint, and this one's reads completed before the barrier above); the stores go out here,
  // ahead of the codes, so that they complete while the codes are computed.
  if constexpr (REFILL) {
    if (a.cp_count > 0 && hi > lo) {
      const int t_lo = (int)(tok_off + lo), t_hi = min((int)(tok_off + hi), a.cp_count);
      if (t_hi > t_lo) {
        const uint16_t *src = (kv ? a.v_src : a.k_src) + ((int64_t)(b * a.H + h) * a.src_ntok + a.src_ntok - a.cp_count + t_lo) * kHeadDim;
        uint8_t *res = a.res_base + (int64_t)(b * a.H + h) * a.res_bh_stride;
        if (kv == 0) residual_store_k(src, t_hi - t_lo, t_lo, res, tid, kThreads);
        else residual_store_v(src, t_hi - t_lo, t_lo, res, a.res_len, tid, kThreads);
      }
    }
  }
  if constexpr (kF16) {
    store_fp16_block(xs, blkp, kv, lo, hi, zhi, tid);
    return;
  }

  // ---- per-group metadata (none for FP8)
  if constexpr (kF8 || kF16) {
  } else if constexpr (kKcK && !kNv) {
    // per-channel K (this kernel's K half): each dim's 128 values of the block form one group
    // (the block is one whole window; the host quantizes only whole windows)
    if (kv == 0) {
      if (tid < kHeadDim) {
        const int d = tid;
        half2v mn2 = {(_Float16)INFINITY, (_Float16)INFINITY}, mx2 = {-(_Float16)INFINITY, -(_Float16)INFINITY};
#pragma unroll 8
        for (int t = 0; t < kBlock; t += 2) {
          const half2v x2 = {__builtin_bit_cast(_Float16, xs[t * kRowHalves + d]), __builtin_bit_cast(_Float16, xs[(t + 1) * kRowHalves + d])};
          mn2 = __builtin_elementwise_min(mn2, x2);
          mx2 = __builtin_elementwise_max(mx2, x2);
        }
        const float mn = fminf((float)mn2.x, (float)mn2.y), mx = fmaxf((float)mx2.x, (float)mx2.y);
        float S = 0.0f;
        uint32_t Sb = 0;
        if (mx > mn) {
          Sb = scale_bits(mn, mx, kQmax);
          S = h2f((uint16_t)Sb);
        }
        if (!(mx > mn) || S == 0.0f) {
          S = mn != 0.0f ? fabsf(mn) : 1.0f;
          Sb = __builtin_bit_cast(uint16_t, (_Float16)S);
        }
        const uint32_t Zb = zero_bits(mn, S);
        mS[d][0] = S;
        mInv[d][0] = 1.0f / S;
        mZ[d][0] = h2f((uint16_t)Zb);
        note_eps(&s_eps, mn, mx, mInv[d][0], mZ[d][0]);
      }
      __syncthreads();
      // (S, Z) in MFMA operand order: position 32g + 8j + e holds the dim that element feeds
      if (tid < kHeadDim) {
        const int pos = tid, d = k_operand_dim(FMT, pos >> 5, (pos >> 3) & 3, pos & 7);
        uint8_t *m = blkp + aff_km(kBits);
        *(uint16_t *)(m + 2 * pos) = __builtin_bit_cast(uint16_t, (_Float16)mS[d][0]);
        *(uint16_t *)(m + 256 + 2 * pos) = __builtin_bit_cast(uint16_t, (_Float16)mZ[d][0]);
      }
    } else {
      for (int idx = tid; idx < kBlock * 2; idx += kThreads) {
        const int slot = idx >> 1, g = idx & 1;
        if (slot < lo || slot >= hi) continue;
        const uint4 *row = (const uint4 *)&xs[slot * kRowHalves + g * kGroup];
        half2v mn2 = {(_Float16)INFINITY, (_Float16)INFINITY}, mx2 = {-(_Float16)INFINITY, -(_Float16)INFINITY};
#pragma unroll
        for (int i = 0; i < kGroup / 8; ++i) {
          const uint4 v = row[i];
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const half2v x2 = __builtin_bit_cast(half2v, w4[k]);
            mn2 = __builtin_elementwise_min(mn2, x2);
            mx2 = __builtin_elementwise_max(mx2, x2);
          }
        }
        const float mn = fminf((float)mn2.x, (float)mn2.y), mx = fmaxf((float)mx2.x, (float)mx2.y);
        float S = 0.0f;
        uint32_t Sb = 0;
        if (mx > mn) {
          Sb = scale_bits(mn, mx, kQmax);
          S = h2f((uint16_t)Sb);
        }
        if (!(mx > mn) || S == 0.0f) {
          S = mn != 0.0f ? fabsf(mn) : 1.0f;
          Sb = __builtin_bit_cast(uint16_t, (_Float16)S);
        }
        const uint32_t Zb = zero_bits(mn, S);
        mS[slot][g] = S;
        mInv[slot][g] = 1.0f / S;
        mZ[slot][g] = h2f((uint16_t)Zb);
        note_eps(&s_eps, mn, mx, mInv[slot][g], mZ[slot][g]);
        const int tau = slot >> 4, r = slot & 15, q = r >> 2, i = r & 3;
        uint8_t *m = blkp + kc_vm(kBits) + (tau * 4 + q) * 32;
        *(uint16_t *)(m + 8 * g + 2 * i) = (uint16_t)Sb;
        *(uint16_t *)(m + 16 + 8 * g + 2 * i) = (uint16_t)Zb;
      }
    }
  } else if constexpr (!kNv) {
   for (int idx = tid; idx < kBlock * NG; idx += kThreads) {
    const int slot = idx / NG, g = idx % NG;
    uint32_t Sb = 0, Zb = 0;
    bool write = false;
    if (slot >= lo && slot < hi) {
      // min / max of the GS values with packed fp16 compares (exact: they only select)
      const uint4 *row = (const uint4 *)&xs[slot * kRowHalves + g * GS];
      half2v mn2 = {(_Float16)INFINITY, (_Float16)INFINITY}, mx2 = {-(_Float16)INFINITY, -(_Float16)INFINITY};
#pragma unroll
      for (int i = 0; i < GS / 8; ++i) {
        const uint4 v = row[i];
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const half2v x2 = __builtin_bit_cast(half2v, w4[k]);
          mn2 = __builtin_elementwise_min(mn2, x2);
          mx2 = __builtin_elementwise_max(mx2, x2);
        }
      }
      const float mn = fminf((float)mn2.x, (float)mn2.y), mx = fmaxf((float)mx2.x, (float)mx2.y);
      float S = 0.0f;
      if (mx > mn) {
        Sb = scale_bits(mn, mx, kQmax);
        S = h2f((uint16_t)Sb);
      }
      if (!(mx > mn) || S == 0.0f) {          // degenerate group: S = |min|, or 1 when min is 0
        S = mn != 0.0f ? fabsf(mn) : 1.0f;
        Sb = __builtin_bit_cast(uint16_t, (_Float16)S);
      }
      Zb = zero_bits(mn, S);
      mS[slot][g] = S;
      mInv[slot][g] = 1.0f / S;
      mZ[slot][g] = h2f((uint16_t)Zb);
      note_eps(&s_eps, mn, mx, mInv[slot][g], mZ[slot][g]);
      write = true;
    } else if (slot >= hi && slot < zhi) {
      write = true;                            // cleared slot: S = Z = +0
    }
    if (write) {
      // Km: per tile, S of (slot r, group g) at 2(NG r + g), the Z 32 NG bytes later; Vm: per
      // (tile, quarter q), S of group g for slot 4q + i at 8g + 2i, the Z 8 NG bytes later
      const int tau = slot >> 4, r = slot & 15;
      if (kv == 0) {
        uint8_t *m = blkp + aff_km(kBits) + tau * 64 * NG;
        *(uint16_t *)(m + 2 * (NG * r + g)) = (uint16_t)Sb;
        *(uint16_t *)(m + 32 * NG + 2 * (NG * r + g)) = (uint16_t)Zb;
      } else {
        const int q = r >> 2, i = r & 3;
        uint8_t *m = blkp + aff_vm(kBits, NG) + (tau * 4 + q) * 16 * NG;
        *(uint16_t *)(m + 8 * g + 2 * i) = (uint16_t)Sb;
        *(uint16_t *)(m + 8 * NG + 8 * g + 2 * i) = (uint16_t)Zb;
      }
    }
   }
  } else if constexpr (kMx) {
    for (int idx = tid; idx < kBlock * 4; idx += kThreads) {
      const int slot = idx >> 2, m = idx & 3;
      uint32_t sb = 0;
      bool write = false;
      if (slot >= lo && slot < hi) {
        // amax by an integer max of the magnitude bits; X = 2^(floor(log2 amax) - 2) read off
        // the fp16 exponent (or the leading mantissa bit of a subnormal)
        const uint4 *row = (const uint4 *)&xs[slot * kRowHalves + m * kMxBlock];
        u16x2 m2 = {0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = row[i];
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w4[k] & 0x7FFF7FFFu));
        }
        const uint32_t amax = m2.x > m2.y ? m2.x : m2.y;
        float X = 0.0f;
        if (amax != 0) {
          const int ebits = (int)(amax >> 10);
          const int fl = ebits > 0 ? ebits - 15 : (31 - __builtin_clz(amax)) - 24;
          sb = (uint32_t)(fl - 2 + 127);
          X = __uint_as_float(sb << 23);
        }
        mS[slot][m] = X;
        write = true;
      } else if (slot >= hi && slot < zhi) {
        write = true;
      }
      if (write) {
        if (kv == 0) {
          blkp[kMxKs + (slot >> 4) * 64 + 16 * m + (slot & 15)] = (uint8_t)sb;
        } else {
          const int w = slot >> 5, g = (slot >> 2) & 3, e = 4 * ((slot >> 4) & 1) + (slot & 3);
          blkp[kMxVs + ((4 * w + g) * 4 + m) * 8 + e] = (uint8_t)sb;
        }
      }
    }
  } else {
    for (int idx = tid; idx < kBlock * 8; idx += kThreads) {
      const int slot = idx >> 3, nb = idx & 7;
      uint8_t sb = 0;
      bool write = false;
      if (slot >= lo && slot < hi) {
        // |x| of finite fp16 values orders like its bit pattern: integer max of the magnitudes
        const uint4 *row = (const uint4 *)&xs[slot * kRowHalves + nb * kNvBlock];
        u16x2 m2 = {0, 0};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint4 v = row[i];
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w4[k] & 0x7FFF7FFFu));
        }
        const float amax = h2f(m2.x > m2.y ? m2.x : m2.y);
        sb = f32_to_e4m3(amax / 6.0f);
        mS[slot][nb] = e4m3_to_f32(sb);
        write = true;
      } else if (slot >= hi && slot < zhi) {
        write = true;
      }
      if (write) {
        if (kv == 0) {
          const int lane = 16 * (nb >> 1) + (slot & 15);
          blkp[kNvKs + ((slot >> 4) * 64 + lane) * 2 + (nb & 1)] = sb;
        } else {
          const int w = slot >> 5, tt = (slot >> 4) & 1, q = (slot >> 2) & 3, i = slot & 3;
          blkp[kNvVs + ((4 * w + q) * 8 + nb) * 8 + 4 * tt + i] = sb;
        }
      }
    }
  }
  __syncthreads();

  // ---- codes
  constexpr int F = 32 / kBits;                     // fields per word
  // Affine codes, fast: t = RN(x * inv + Z) (one fused multiply-add of the fp16 x, with
  // inv = RN(1 / S)) lies within eps_g of x / S + Z for every x of group g (note_eps), so
  // rint(t) is RNE(x / S) + Z (Z is an integer) unless x / S is within eps_g of a
  // half-integer.  Where |t - rint(t)| reaches 0.5 - eps (eps: the block's largest eps_g) the
  // code is decided by the exact remainder instead (div_rne): a branch that the wave takes
  // only when one of its lanes meets such a value (about 3e-4 of normally distributed inputs,
  // nearly all of them exact ties).
  const float thr = 0.5f - __uint_as_float(s_eps);
  auto fast_code = [&](_Float16 xh, float S_of, float inv, float Z) -> uint32_t {
    const float t = __builtin_fmaf((float)xh, inv, Z);
    float k = rintf(t);
    if (__builtin_expect(fabsf(t - k) >= thr, 0)) k = div_rne((float)xh, S_of, inv) + Z;
    return (uint32_t)__builtin_amdgcn_fmed3f(k, 0.0f, (float)kQmax);
  };
  auto code_of = [&](float x, int slot, int grp) -> uint32_t {
    if constexpr (kF8) return e4m3_cast(x);
    else if constexpr (kNv) return e2m1_code(x, mS[slot][grp]);
    else return affine_code(x, mS[slot][grp], mInv[slot][grp], mZ[slot][grp], kQmax);
  };
  // K code of dim d of a slot (per-channel K: the dim's group; else the slot's group of d)
  auto kcode_of = [&](float x, int slot, int d) -> uint32_t {
    if constexpr (kKcK && !kNv && !kF8) return affine_code(x, mS[d][0], mInv[d][0], mZ[d][0], kQmax);
    else return code_of(x, slot, d / (kMx ? kMxBlock : kNv ? kNvBlock : GSV));
  };
  if (kv == 0) {
    // K: [part w][tile u][chunk r][lane][cb bytes]; a word holds F fields of one slot at F
    // consecutive dims, read from LDS 8 values at a time
    constexpr int kWords = kBlock * kWordsPerRow;
    constexpr int kLaneBytes = 4 * kBits;
    constexpr int kCb = kLaneBytes < 16 ? kLaneBytes : 16;
    constexpr int kK = kLaneBytes / kCb;
    const int wend = (sub + 1) * (kWords / nsplit);   // the words of this workgroup's parts
    for (int w = sub * (kWords / nsplit) + tid; w < wend; w += kThreads) {
      const int ci = (4 * w) / kCb, in_chunk = (4 * w) % kCb;
      const int lane = ci & 63, t2 = ci >> 6;
      const int r = t2 % kK, wu = t2 / kK;
      const int g = lane >> 4, c = lane & 15;
      const int slot = 16 * wu + c;                  // 32 * part + 16 * tile + c
      if (slot < lo || slot >= zhi) continue;
      const int omega = (r * kCb + in_chunk) / 4;    // word of the lane string
      uint32_t word = 0;
      if (kAffine && GS == 32 && slot < hi) {
        // groups of 32: the word's fields are permuted within runs of 8 dims; one at a time
#pragma unroll
        for (int k = 0; k < F; ++k) {
          const int d = k_lane_dim32(FMT, g, omega * F + k);
          word |= fast_code(__builtin_bit_cast(_Float16, xs[slot * kRowHalves + d]), mS[slot][d >> 5], mInv[slot][d >> 5],
                            mZ[slot][d >> 5]) << (k * kBits);
        }
      } else if (kAffine && !kKcK && slot < hi) {
        // one group for the word's F consecutive dims
        const int d0 = k_lane_dim(FMT, g, omega * F);
        const int grp = d0 / GSV;
        const uint16_t *xr = &xs[slot * kRowHalves + d0];
        const float Sg = mS[slot][grp], inv = mInv[slot][grp], Z = mZ[slot][grp];
        _Float16 x[F];
        if constexpr (F >= 8) {
#pragma unroll
          for (int h8 = 0; h8 < F / 8; ++h8) {
            const half8v x8 = __builtin_bit_cast(half8v, *(const uint4 *)(xr + 8 * h8));
#pragma unroll
            for (int k = 0; k < 8; ++k) x[8 * h8 + k] = x8[k];
          }
        } else {
          const half8v x8 = __builtin_bit_cast(half8v, make_uint4((*(const uint2 *)xr).x, (*(const uint2 *)xr).y, 0u, 0u));
#pragma unroll
          for (int k = 0; k < 4; ++k) x[k] = x8[k];
        }
#pragma unroll
        for (int k = 0; k < F; ++k) word |= fast_code(x[k], Sg, inv, Z) << (k * kBits);
      } else if (slot < hi) {
        const int d0 = k_lane_dim(FMT, g, omega * F);   // first of F consecutive dims
        const uint16_t *xr = &xs[slot * kRowHalves + d0];
        if constexpr (F >= 8) {
#pragma unroll
          for (int h8 = 0; h8 < F / 8; ++h8) {
            float x[8];
            unpack8(*(const uint4 *)(xr + 8 * h8), x);
#pragma unroll
            for (int k = 0; k < 8; ++k) word |= kcode_of(x[k], slot, d0 + 8 * h8 + k) << ((8 * h8 + k) * kBits);
          }
        } else {
          const uint2 v = *(const uint2 *)xr;
          const float x[4] = {h2f((uint16_t)(v.x & 0xFFFFu)), h2f((uint16_t)(v.x >> 16)), h2f((uint16_t)(v.y & 0xFFFFu)),
                              h2f((uint16_t)(v.y >> 16))};
#pragma unroll
          for (int k = 0; k < 4; ++k) word |= kcode_of(x[k], slot, d0 + k) << (k * kBits);
        }
      }
      *(uint32_t *)(blkp + (size_t)w * 4) = word;
    }
  } else {
    // V: [part w][chunk r][lane][16 bytes]; lane (g, c) word omega holds fields phi = omega F + j
    // of dim 16 k + c and slot 32 w + 16 (e >> 2) + 4 g + (e & 3).  A task is (part, g, omega,
    // c0): the words of lanes 16 g + c0 .. + NL - 1, whose field j reads the same slot at the NL
    // consecutive dims 16 k + c0 .. (one LDS read and one metadata lookup).  NL = 8, or 4 where
    // 8 would leave threads idle (INT2: 128 tasks of 8 lanes for 256 threads); a workgroup of a
    // split block (one 32-slot part: a quarter of the tasks) gives each task kLaneWords / 4
    // lanes, so that it has one task per thread (INT4: 64 tasks of 8 lanes would leave three
    // waves idle; 2 lanes for INT4, 1 for INT2, 4 for INT8).
    const size_t vc = kMx ? kMxVc : kNv ? kNvVc : kF8 ? kF8Vc : kKcK ? kc_vc(kBits) : aff_vc(kBits, NG);
    constexpr int kChunks = kBits / 2;              // 16-byte chunks per lane
    constexpr int kLaneWords = 4 * kChunks;
    constexpr int kNL = 4 * 4 * kLaneWords * 2 >= kThreads ? 8 : 4 * 4 * kLaneWords * 4 >= kThreads ? 4 : 2;
    auto v_codes = [&](auto nl) __attribute__((always_inline)) {
      constexpr int NL = decltype(nl)::value;
      constexpr int kSplit = 16 / NL;
      constexpr int kTasks = 4 * 4 * kLaneWords * kSplit;
      const int tend = (sub + 1) * (kTasks / nsplit);   // tasks are part-major: this workgroup's parts
      for (int task = sub * (kTasks / nsplit) + tid; task < tend; task += kThreads) {
        const int c0 = NL * (task % kSplit), omega = (task / kSplit) % kLaneWords, g = ((task / kSplit) / kLaneWords) & 3;
        const int part = (task / kSplit) / kLaneWords >> 2;
        uint32_t words[NL] = {};
        uint32_t keep = 0;                            // field bits of slots before lo (kept as stored)
        bool any = false;
  #pragma unroll
        for (int j = 0; j < F; ++j) {
          int k, e;
          v_field(FMT, omega * F + j, k, e);
          const int slot = 32 * part + 16 * (e >> 2) + 4 * g + (e & 3);
          if (slot < lo) {
            keep |= (uint32_t)kQmax << (j * kBits);
            continue;
          }
          if (slot >= zhi) continue;
          any = true;
          if (slot >= hi) continue;                    // cleared: code 0
          const int d0 = 16 * k + c0;
          const int grp = d0 / (kMx ? kMxBlock : kNv ? kNvBlock : GSV);
          uint4 raw = make_uint4(0u, 0u, 0u, 0u);
          if constexpr (NL == 8) {
            raw = *(const uint4 *)&xs[slot * kRowHalves + d0];
          } else if constexpr (NL == 4) {
            const uint2 u = *(const uint2 *)&xs[slot * kRowHalves + d0];
            raw.x = u.x; raw.y = u.y;
          } else if constexpr (NL == 1) {
            raw.x = xs[slot * kRowHalves + d0];
          } else {
            raw.x = *(const uint32_t *)&xs[slot * kRowHalves + d0];
          }
          if constexpr (kAffine) {
            const half8v xh = __builtin_bit_cast(half8v, raw);
            const float Sg = mS[slot][grp], inv = mInv[slot][grp], Z = mZ[slot][grp];
  #pragma unroll
            for (int i = 0; i < NL; ++i) words[i] |= fast_code(xh[i], Sg, inv, Z) << (j * kBits);
          } else {
            float x[8];
            unpack8(raw, x);
  #pragma unroll
            for (int i = 0; i < NL; ++i) words[i] |= code_of(x[i], slot, grp) << (j * kBits);
          }
        }
        if (!any) continue;
  #pragma unroll
        for (int i = 0; i < NL; ++i) {
          const int lane = 16 * g + c0 + i;
          uint32_t *dst = (uint32_t *)(blkp + vc + ((size_t)(part * kChunks + omega / 4) * 64 + lane) * 16 + (omega % 4) * 4);
          *dst = keep ? (*dst & keep) | words[i] : words[i];
        }
      }
    };
    if constexpr (kAffine && !kKcK) {
      if (nsplit > 1) v_codes(std::integral_constant<int, (kLaneWords >= 4 ? kLaneWords / 4 : 1)>{});
      else v_codes(std::integral_constant<int, kNL>{});
    } else {
      v_codes(std::integral_constant<int, kNL>{});
    }
  }
}

// Workgroup (x, h, b) copies tokens [64 x, 64 x + 64) of the copy for (b, h).
constexpr int kCopyTokens = 64;
__global__ __launch_bounds__(256) void residual_copy_kernel(ResCopyArgs a) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t i0 = (int64_t)blockIdx.x * kCopyTokens;
  const int n = (int)min<int64_t>(kCopyTokens, a.count - i0);
  const int64_t src = ((int64_t)(b * a.H + h) * a.src_ntok + a.src_tok0 + i0) * kHeadDim;
  residual_store(a.k_src + src, a.v_src + src, n, (int)(a.dst_slot0 + i0),
                 a.res_base + (int64_t)(b * a.H + h) * a.res_bh_stride, a.res_len, threadIdx.x, 256);
}

}  // namespace

// Compute units of the current device (256 if the query fails), looked up once per device.
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cus[dev];
}

template <int F, int GS>
void launch_quantize_as(const QuantArgs &a, dim3 grid, int64_t blk0, int64_t nblk, hipStream_t s) {
  if (a.cp_count > 0) quantize_kernel<F, GS, true><<<grid, kThreads, 0, s>>>(a, blk0, nblk);
  else quantize_kernel<F, GS, false><<<grid, kThreads, 0, s>>>(a, blk0, nblk);
}

hipError_t launch_quantize(const QuantArgs &in, hipStream_t s) {
  if (in.count <= 0) return hipSuccess;
  const int64_t blk0 = in.dst_slot0 / kBlock;
  const int64_t blk1 = (in.dst_slot0 + in.count - 1) / kBlock;
  const int64_t nblk = blk1 - blk0 + 1;
  // A launch of few blocks (a residual flush: one or two blocks per (b, h)) leaves most CUs
  // idle with one workgroup per block: affine formats with per-token groups then take one
  // workgroup per 32-slot part.
  QuantArgs a = in;
  a.nsplit = is_affine(a.fmt) && a.gs != kKc && nblk * a.H * a.B * 2 < 2 * device_cus() ? 4 : 1;
  dim3 grid((unsigned)(nblk * a.nsplit), (unsigned)a.H, (unsigned)(a.B * 2));
#define KVQ_AFFINE_CASE(F)                                                     \
  case F:                                                                      \
    if (a.gs == kKc) launch_quantize_as<F, kKc>(a, grid, blk0, nblk, s);       \
    else if (a.gs == 32) launch_quantize_as<F, 32>(a, grid, blk0, nblk, s);    \
    else if (a.gs == 128) launch_quantize_as<F, 128>(a, grid, blk0, nblk, s);  \
    else if (a.gs == 64) launch_quantize_as<F, 64>(a, grid, blk0, nblk, s);    \
    else return hipErrorInvalidValue;                                          \
    break;
  switch (a.fmt) {
    KVQ_AFFINE_CASE(kFmtInt2)
    KVQ_AFFINE_CASE(kFmtInt4)
    KVQ_AFFINE_CASE(kFmtInt8)
    case kFmtNvfp4: launch_quantize_as<kFmtNvfp4, 64>(a, grid, blk0, nblk, s); break;
    case kFmtFp8: launch_quantize_as<kFmtFp8, 64>(a, grid, blk0, nblk, s); break;
    case kFmtMxfp4: launch_quantize_as<kFmtMxfp4, 64>(a, grid, blk0, nblk, s); break;
    case kFmtFp16: launch_quantize_as<kFmtFp16, 64>(a, grid, blk0, nblk, s); break;
    default: return hipErrorInvalidValue;
  }
#undef KVQ_AFFINE_CASE
  return hipGetLastError();
}

hipError_t launch_residual_copy(const ResCopyArgs &a, hipStream_t s) {
  if (a.count <= 0) return hipSuccess;
  dim3 grid((unsigned)((a.count + kCopyTokens - 1) / kCopyTokens), (unsigned)a.H, (unsigned)a.B);
  residual_copy_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvq
