// Encoders of the 8-bit and 4-bit float codes shared by the append kernel and the decode
// kernel's in-launch append (page "NVFP4 KV缓存技术详解" §2.1: 16 values share one FP8 scale;
// §4.2: values clipped to the E2M1 maximum 6).  Every rounding is decided exactly:
//  * E4M3: fp32 amax/6 (correctly rounded) is never closer to an E4M3 midpoint than its error
//    unless it lies on it exactly; it is then rounded to 3 mantissa bits, ties to even.
//  * E2M1: |x| is compared with midpoint * s, both exact in fp32.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace kvq {
namespace {

// Non-negative float -> OCP E4M3 byte, round to nearest even, saturating at 448 (0x7E).
__device__ __forceinline__ uint8_t f32_to_e4m3(float v) {
  if (v >= 448.0f) return 0x7E;
  if (v < 0.015625f) return (uint8_t)rintf(v * 512.0f);   // below 2^-6: multiples of 2^-9 (8 -> 0x08)
  uint32_t bits = __float_as_uint(v);
  int e = (int)((bits >> 23) & 0xFF) - 127;                // -6..8
  uint32_t m = bits & 0x7FFFFF;
  uint32_t keep = m >> 20, rem = m & 0xFFFFF, half = 0x80000;
  if (rem > half || (rem == half && (keep & 1))) ++keep;
  if (keep == 8) { keep = 0; ++e; }
  uint32_t code = ((uint32_t)(e + 7) << 3) | keep;
  return (uint8_t)(code > 0x7E ? 0x7E : code);
}

// FP8 cache code of an fp16 value: E4M3 of |x| (round to nearest even, saturating at 448)
// with the sign bit of x.
__device__ __forceinline__ uint32_t e4m3_cast(float x) {
  return (uint32_t)f32_to_e4m3(fabsf(x)) | (signbit(x) ? 0x80u : 0u);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t e = (b >> 3) & 0xF, m = b & 7;
  float mag = e == 0 ? (float)m * 0.001953125f : ldexpf(1.0f + (float)m * 0.125f, (int)e - 7);
  return (b & 0x80) ? -mag : mag;
}

// E2M1 code (sign bit 8, magnitude index 0..7 on {0, 0.5, 1, 1.5, 2, 3, 4, 6}) of x under
// scale s: nearest magnitude of |x| / s clipped to 6, ties to the even index; s = 0 gives a
// signed zero.  The index counts the decision points that |x| has passed: the midpoints m_j s
// between magnitudes j and j + 1, passed when |x| > m_j s for even j and when |x| >= m_j s for
// odd j (a value on a midpoint then lands on the even neighbour).  The points passed form a
// prefix, so three comparisons (a binary search over 1.75, then 0.75 or 3.5, then one of 0.25,
// 1.25, 2.5, 5) find the count; each m_j s is exact in fp32 (3 significant bits times the 4 of
// an E4M3 or power-of-two scale), so every comparison is exact.
__device__ __forceinline__ uint32_t e2m1_code(float x, float s) {
  const float a = fabsf(x);
  const bool c1 = a >= 1.75f * s;
  const bool c2 = a >= (c1 ? 3.5f : 0.75f) * s;
  const bool c3 = a > (c1 ? (c2 ? 5.0f : 2.5f) : (c2 ? 1.25f : 0.25f)) * s;
  const uint32_t idx = s > 0.0f ? 4u * c1 + 2u * c2 + (uint32_t)c3 : 0u;
  return idx | (signbit(x) ? 8u : 0u);
}

// Value of an E2M1 magnitude index (0..7) as a multiple of the scale.
__device__ __forceinline__ float e2m1_value(uint32_t idx) {
  const float t[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  return t[idx & 7];
}

}  // namespace
}  // namespace kvq
