// Device-side helpers shared by the gfx950 kernels of libmxfp8.so.
//
// Number formats (OCP Microscaling v1.0, the MXFP8 of the pages):
//   E4M3 ("E4M3FN") code: sign | 4-bit exponent (bias 7) | 3-bit mantissa,
//     subnormals m/8 * 2^-6, largest finite 448 = 0x7E, 0x7F/0xFF NaN.
//   E8M0 scale byte b: 2^(b - 127), 0xFF NaN.
// Everything here is exact integer/bit arithmetic except the E4M3 rounding:
// round-to-nearest-even, done by gfx950's scaled conversion instruction on
// the quantization path (e4m3_chunk, cvt4) and on float32 bit patterns in
// e4m3_code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {

constexpr int kBlock = 32;

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bf16 bits with gfx950's v_cvt_pk_bf16_f32: round to nearest
// even (denormals kept), NaN stays a quiet NaN of the same sign.
typedef __bf16 mx_bf16x2 __attribute__((ext_vector_type(2)));
typedef float mx_f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((mx_f32x2{lo, hi}), mx_bf16x2));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.0f) & 0xFFFFu; }

// 16-byte global load marked non-temporal (data streamed through once).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u q = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(q.x, q.y, q.z, q.w);
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

// OR of v over lanes l, l + 4, l + 8, l + 12 of each 16-lane row (DPP
// row_ror:4 then row_ror:8). Every lane of the row must be active.
__device__ __forceinline__ uint32_t or_row_quarters(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false);
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);
  return v;
}

// max of v over the 16 lanes of each DPP row (quad permutes for lanes ^ 1
// and ^ 2, then row_ror:4 and row_ror:8). Every lane of the row must be
// active.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false));
  return v;
}

// OR of v over the lanes l, l ^ 2, 7 - l, (7 - l) ^ 2 of each 8-lane group,
// which include one lane of each pair {2k, 2k + 1} (DPP quad_perm [2,3,0,1]
// then row_half_mirror). Every lane of the group must be active.
__device__ __forceinline__ uint32_t or_octet_pairs(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);
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

// ---------------------------------------------------------------- E4M3 (hardware)
//
// gfx950's v_cvt_scalef32_pk_fp8_bf16 converts two bf16 values x to E4M3
// codes of x / scale, rounded to nearest even, with the sign kept; measured
// on the device, it equals the rounding above for every finite bf16 input
// and every scale 2^E, E in [-127, 127] (including subnormal inputs and the
// subnormal scale 2^-127) whenever |x / scale| <= 448. Above 448 it returns
// NaN, so saturation clamps the magnitudes first (only FLOOR scales can put
// elements above 448). Non-finite inputs give 0x7F | sign.

typedef short mx_v2s __attribute__((ext_vector_type(2)));
typedef __bf16 mx_v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short mx_us2 __attribute__((ext_vector_type(2)));

// 2^E as a float32 for a finite scale byte b = E + 127 (2^-127 is subnormal).
__device__ __forceinline__ float scale_f32(uint32_t b) {
  return __uint_as_float(b ? (b << 23) : 0x00400000u);
}

// bf16 bits of 448 * 2^E (infinity when that overflows bf16, which then
// clamps nothing).
__device__ __forceinline__ uint32_t sat_bits(uint32_t b) {
  return b + 8u >= 255u ? 0x7F80u : (((b + 8u) << 7) | 0x60u);
}

// Clamps the magnitudes of the two bf16 values in w to lim2 (one 16-bit
// limit per half), keeping the signs.
__device__ __forceinline__ uint32_t clamp_pair(uint32_t w, uint32_t lim2) {
  const mx_us2 m = __builtin_elementwise_min(__builtin_bit_cast(mx_us2, w & 0x7FFF7FFFu),
                                             __builtin_bit_cast(mx_us2, lim2));
  return (w & 0x80008000u) | __builtin_bit_cast(uint32_t, m);
}

// Codes of 4 bf16 values (pairs w0 = elements 0, 1 and w1 = 2, 3) divided by
// `scale`, little-endian in one dword.
__device__ __forceinline__ uint32_t cvt4(uint32_t w0, uint32_t w1, float scale) {
  mx_v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(mx_v2s{0, 0}, __builtin_bit_cast(mx_v2bf, w0), scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(mx_v2bf, w1), scale, true);
  return __builtin_bit_cast(uint32_t, r);
}

// Codes of the 8 bf16 values of a chunk under scale byte sb, packed
// little-endian into 8 bytes; `saturate` clamps to 448 * 2^E first (needed
// for FLOOR). A block with scale 0xFF encodes 0x7F | sign.
__device__ __forceinline__ uint2 e4m3_chunk(uint4 v, uint32_t sb, bool saturate) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const bool nonfinite = sb == 0xFFu;
  const float scale = scale_f32(sb);
  if (saturate) {
    const uint32_t lim = sat_bits(sb);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = clamp_pair(w[i], lim | (lim << 16));
  }
  uint32_t out[2] = {cvt4(w[0], w[1], scale), cvt4(w[2], w[3], scale)};
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
