// Device-side helpers shared by the gfx950 kernels of libmxfp8.so.
//
// Number formats (OCP Microscaling v1.0, the MXFP8 of the pages):
//   E4M3 ("E4M3FN") code: sign | 4-bit exponent (bias 7) | 3-bit mantissa,
//     subnormals m/8 * 2^-6, largest finite 448 = 0x7E, 0x7F/0xFF NaN.
//   E8M0 scale byte b: 2^(b - 127), 0xFF NaN.
// Everything here is exact integer/bit arithmetic except the E4M3 rounding,
// which is round-to-nearest-even done on float32 bit patterns.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {

constexpr int kBlock = 32;

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bf16 bits, round to nearest even; NaN -> 0x7FC0 with its sign.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? (((u >> 16) & 0x8000u) | 0x7FC0u) : r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// max |v| over the 8 bf16 values of a 16-byte chunk, as 15-bit magnitude bits
// (non-negative bf16 bit patterns order like their values; NaN > 0x7F80).
__device__ __forceinline__ uint32_t absmax8_bits(uint4 v) {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  us2 a = __builtin_bit_cast(us2, v.x & 0x7FFF7FFFu);
  us2 b = __builtin_bit_cast(us2, v.y & 0x7FFF7FFFu);
  us2 c = __builtin_bit_cast(us2, v.z & 0x7FFF7FFFu);
  us2 d = __builtin_bit_cast(us2, v.w & 0x7FFF7FFFu);
  us2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                    __builtin_elementwise_max(c, d));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// max over the 4 lanes of a quad (lanes 4k..4k+3), via DPP quad permutes.
// Every lane of the quad must be active.
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));  // lanes ^1
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));  // lanes ^2
  return v;
}

// ---------------------------------------------------------------- scales

// E8M0 scale byte (E + 127) of a block whose max magnitude has bf16 bits
// `amax` (sign cleared).
//   FLOOR: E = floor(log2 amax) - 8 = expfield - 135.
//   RCEIL: smallest E with amax <= 448 * 2^E: one more than FLOOR exactly
//          when the significand 1.m exceeds 1.75 (mantissa field > 0x60).
// E is clamped below at -127 (zero and subnormal maxima land there); finite
// bf16 never exceeds E = 120. A NaN or infinite maximum gives 0xFF.
__device__ __forceinline__ uint32_t scale_byte(uint32_t amax, bool rceil) {
  int e = (int)(amax >> 7) - 135 + ((rceil && (amax & 0x7Fu) > 0x60u) ? 1 : 0);
  e = max(e, -127);
  return amax >= 0x7F80u ? 0xFFu : (uint32_t)(e + 127);
}

// 2^-E as a float32 for a finite scale byte b = E + 127 (E in [-127, 120]).
__device__ __forceinline__ float inv_scale(uint32_t b) {
  return __uint_as_float((254u - min(b, 247u)) << 23);
}

// ---------------------------------------------------------------- E4M3

// E4M3 code of y (already divided by the block scale): |y| saturates at 448,
// then rounds to nearest, ties to even; the sign is kept (-0 -> 0x80).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  uint32_t u = __float_as_uint(y);
  float a = fminf(__uint_as_float(u & 0x7FFFFFFFu), 448.0f);
  // below 2^-6 the grid is the subnormal one, spacing 2^-9
  uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);
  // normal: round the float32 mantissa to 3 bits (ties to even), then rebias
  // the exponent from 127 to 7
  uint32_t b = __float_as_uint(a);
  b += 0x7FFFFu + ((b >> 20) & 1u);
  uint32_t nrm = (b >> 20) - (120u << 3);
  return (a < 0.015625f ? sub : nrm) | ((u >> 24) & 0x80u);
}

// Codes of the 8 bf16 values of a chunk, scaled by `mul` = 2^-E, packed
// little-endian into 8 bytes. A block with scale 0xFF encodes 0x7F | sign.
__device__ __forceinline__ uint2 e4m3_chunk(uint4 v, float mul, bool nonfinite) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t out[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t c0 = e4m3_code(bf16_lo(w[2 * i]) * mul);
    uint32_t c1 = e4m3_code(bf16_hi(w[2 * i]) * mul);
    uint32_t c2 = e4m3_code(bf16_lo(w[2 * i + 1]) * mul);
    uint32_t c3 = e4m3_code(bf16_hi(w[2 * i + 1]) * mul);
    out[i] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
  }
  if (nonfinite) {
    // 0x7F with each element's sign (bit 15 of each bf16)
    uint32_t s0 = ((w[0] >> 8) & 0x80u) | ((w[0] >> 16) & 0x8000u) | ((w[1] << 8) & 0x800000u) | (w[1] & 0x80000000u);
    uint32_t s1 = ((w[2] >> 8) & 0x80u) | ((w[2] >> 16) & 0x8000u) | ((w[3] << 8) & 0x800000u) | (w[3] & 0x80000000u);
    out[0] = 0x7F7F7F7Fu | s0;
    out[1] = 0x7F7F7F7Fu | s1;
  }
  return make_uint2(out[0], out[1]);
}

// Value of an E4M3 code as float32 (exact); NaN codes give NaN.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  // normal: (8 + m) * 2^(e - 10) = float with exponent e + 120, mantissa m << 20
  float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  float sub = (float)m * 0.001953125f;   // m * 2^-9
  float v = e ? nrm : sub;
  v = ((c & 0x7Fu) == 0x7Fu) ? __uint_as_float(0x7FC00000u) : v;
  return __uint_as_float(__float_as_uint(v) | ((c & 0x80u) << 24));
}

// ---------------------------------------------------------------- misc

// Quotient by a fixed divisor d >= 1 with a precomputed multiplier
// (Granlund-Montgomery): s = ceil(log2 d), mul = floor(2^32 (2^s - d) / d) + 1,
// q = (mulhi(n, mul) + n) >> s, exact for every 32-bit n.
struct FastDiv {
  uint32_t d, mul, shift;
};

__host__ __device__ inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  uint64_t mul = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
  return FastDiv{d, (uint32_t)mul, s};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
  uint64_t t = (((uint64_t)n * f.mul) >> 32) + n;
  return (uint32_t)(t >> f.shift);
}

}  // namespace mxk
