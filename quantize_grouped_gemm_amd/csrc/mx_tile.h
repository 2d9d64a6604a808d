// MX quantization of a 128 x 128 bf16 tile by a 256-thread workgroup, shared
// by the bandwidth-bound kernels (mx_quant.hip) and the grouped GEMM's fused
// SwiGLU epilogue (mx_gemm.hip). Thread t holds 8 chunks of 8 consecutive
// values (16 bytes each): chunk j sits at tile row (t >> 4) + 16 j, columns
// 8 (t & 15) .. 8 (t & 15) + 7, so the 4 lanes of a quad hold one 32-value
// row block. Row-wise quantization works from those registers; column-wise
// quantization from an LDS copy of the tile.
#pragma once

#include "mx_device.h"

namespace mxk {

constexpr int kTR = 128;                 // tile rows
constexpr int kTC = 128;                 // tile columns
constexpr int kTileThreads = 256;
constexpr int kTileChunks = kTR * kTC / 8 / kTileThreads;   // 8 per thread

struct TileOut {
  uint8_t* q;      // codes
  uint8_t* s;      // scales
  int64_t ld;      // codes per output row (plain scale row = ld / 32 bytes)
  int64_t srows;   // output rows (the k128 layout's step stride, in dwords)
  bool k128;       // scales in the k128 layout [ld/128, srows, 4]
};

// Row-wise quantization of the thread's 8 chunks. The tile's (0,0) sits at
// row r0, column c0 of the output. All lanes must reach this function. In the
// k128 layout (c0 % 128 == 0) a row's four block scales form one dword: the
// 16 lanes of the row gather it with two DPP row rotations and one lane
// stores it.
__device__ __forceinline__ void tile_rowq(const uint4 (&v)[kTileChunks], int rows_valid,
                                          int cols_valid, bool rceil, TileOut o, int64_t r0,
                                          int64_t c0) {
  const int t = threadIdx.x;
  const int cc = t & 15;
  const bool colok = cc * 8 < cols_valid;
#pragma unroll
  for (int j = 0; j < kTileChunks; ++j) {
    const int row = (t >> 4) + 16 * j;
    const uint32_t sb = scale_byte(quad_max(absmax8_bits(v[j])), rceil);
    const uint2 codes = e4m3_chunk(v[j], sb, !rceil);
    uint32_t packed = 0;
    if (o.k128) {
      packed = or_row_quarters(sb << (8 * (cc >> 2)));
    }
    if (row < rows_valid && colok) {
      const int64_t orow = r0 + row;
      const int64_t ocol = c0 + cc * 8;
      *reinterpret_cast<uint2*>(o.q + orow * o.ld + ocol) = codes;
      if (o.k128) {
        if (cc == 0) *reinterpret_cast<uint32_t*>(o.s + ((c0 >> 7) * o.srows + orow) * 4) = packed;
      } else if ((cc & 3) == 0) {
        o.s[orow * (o.ld / kBlock) + ocol / kBlock] = (uint8_t)sb;
      }
    }
  }
}

// Loads the thread's chunks of a bf16 tile whose (0,0) is `base` with row
// stride ld elements; chunks outside the valid region read as zero. NT:
// non-temporal loads (see kStreamBytes in mx_quant.hip for when).
template <bool NT = false>
__device__ __forceinline__ void tile_load(uint4 (&v)[kTileChunks], const uint16_t* base,
                                          int64_t ld, int rows_valid, int cols_valid) {
  const int t = threadIdx.x;
  const int cc = t & 15;
#pragma unroll
  for (int j = 0; j < kTileChunks; ++j) {
    const int row = (t >> 4) + 16 * j;
    v[j] = (row < rows_valid && cc * 8 < cols_valid)
               ? (NT ? load_stream16(base + row * ld + cc * 8)
                     : *reinterpret_cast<const uint4*>(base + row * ld + cc * 8))
               : make_uint4(0, 0, 0, 0);
  }
}

// Stage the thread's chunks in LDS: tile row r, 16-byte unit u (columns
// 8 u .. 8 u + 7) at slot r * 16 + (u ^ g(r)), g(r) = 2 ((r >> 4) & 7). A
// ds_write_b128 pass (16 lanes = one row) covers the 64 banks once.
__device__ __forceinline__ int lds_unit(int r, int u) { return r * 16 + (u ^ (((r >> 4) & 7) << 1)); }

__device__ __forceinline__ void tile_to_lds(const uint4 (&v)[kTileChunks], uint4* lds) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kTileChunks; ++j) lds[lds_unit((t >> 4) + 16 * j, t & 15)] = v[j];
}

// Column-wise quantization from the LDS tile. Work item (cp, q): columns
// 2 cp, 2 cp + 1 and tile rows 16 q .. 16 q + 15, i.e. half a 32-row block of
// two output rows. Lane l of wave w takes q = l & 7 and, in pass s, column
// pair cp = 8 (4 s + w) + (l >> 3): the 8 lanes of a column pair cover one
// output row's 128 codes, so each 16-byte store writes 8 whole lines. Block
// maxima pair lanes q, q ^ 1 (one DPP exchange). The LDS reads (one dword =
// two columns, 16 rows) hit 64 distinct banks thanks to the swizzle above.
// Output row = tile column c0 + col, output column = tile row r0 + row.
// col_sb (optional, 128 bytes by tile column): scale bytes given per column
// (one scale for the whole column) in place of the blocks' own.
// All lanes must reach this function.
__device__ __forceinline__ void tile_colq(const uint4* lds4, int rows_valid, int cols_valid,
                                          bool rceil, TileOut o, int64_t r0, int64_t c0,
                                          const uint8_t* col_sb = nullptr) {
  const uint32_t* lds = reinterpret_cast<const uint32_t*>(lds4);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane & 7;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int cp = 8 * (4 * s + w) + (lane >> 3);
    uint32_t v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = lds[lds_unit(16 * q + r, cp >> 2) * 4 + (cp & 3)];
    mx_us2 m = __builtin_bit_cast(mx_us2, v[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int r = 1; r < 16; ++r) m = __builtin_elementwise_max(m, __builtin_bit_cast(mx_us2, v[r] & 0x7FFF7FFFu));
    uint32_t mm = __builtin_bit_cast(uint32_t, m);
    const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)mm, 0xB1, 0xF, 0xF, false);   // lane ^ 1
    m = __builtin_elementwise_max(m, __builtin_bit_cast(mx_us2, other));
    const uint32_t sb0 = col_sb ? (uint32_t)col_sb[2 * cp] : scale_byte(m.x, rceil);
    const uint32_t sb1 = col_sb ? (uint32_t)col_sb[2 * cp + 1] : scale_byte(m.y, rceil);
    if (!rceil) {
      const uint32_t lim2 = sat_bits(sb0) | (sat_bits(sb1) << 16);
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = clamp_pair(v[r], lim2);
    }
    const float sc0 = scale_f32(sb0), sc1 = scale_f32(sb1);
    uint32_t c0w[4], c1w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t* x = &v[4 * k];
      c0w[k] = cvt4(__builtin_amdgcn_perm(x[1], x[0], 0x05040100u), __builtin_amdgcn_perm(x[3], x[2], 0x05040100u), sc0);
      c1w[k] = cvt4(__builtin_amdgcn_perm(x[1], x[0], 0x07060302u), __builtin_amdgcn_perm(x[3], x[2], 0x07060302u), sc1);
      if (sb0 == 0xFFu) {
        uint32_t a = 0x7F7F7F7Fu;
#pragma unroll
        for (int i = 0; i < 4; ++i) a |= ((x[i] >> 15) & 1u) << (8 * i + 7);
        c0w[k] = a;
      }
      if (sb1 == 0xFFu) {
        uint32_t a = 0x7F7F7F7Fu;
#pragma unroll
        for (int i = 0; i < 4; ++i) a |= ((x[i] >> 31) & 1u) << (8 * i + 7);
        c1w[k] = a;
      }
    }
    // scale bytes of the step's four blocks for the two output rows
    uint32_t p0 = 0, p1 = 0;
    if (o.k128) {
      p0 = or_octet_pairs(sb0 << (8 * (q >> 1)));
      p1 = or_octet_pairs(sb1 << (8 * (q >> 1)));
    }
    if (2 * cp < cols_valid && 16 * q < rows_valid) {
      const int64_t orow0 = c0 + 2 * cp;
      const int64_t ocol = r0 + 16 * q;
      *reinterpret_cast<uint4*>(o.q + orow0 * o.ld + ocol) = make_uint4(c0w[0], c0w[1], c0w[2], c0w[3]);
      *reinterpret_cast<uint4*>(o.q + (orow0 + 1) * o.ld + ocol) = make_uint4(c1w[0], c1w[1], c1w[2], c1w[3]);
      if (o.k128) {
        if (q == 0) {
          uint32_t* sd = reinterpret_cast<uint32_t*>(o.s + ((r0 >> 7) * o.srows + orow0) * 4);
          sd[0] = p0;
          sd[1] = p1;
        }
      } else if ((q & 1) == 0) {
        o.s[orow0 * (o.ld / kBlock) + ocol / kBlock] = (uint8_t)sb0;
        o.s[(orow0 + 1) * (o.ld / kBlock) + ocol / kBlock] = (uint8_t)sb1;
      }
    }
  }
}


// e^x for x <= 0 (and for -inf, giving 0, and NaN, giving NaN), within an
// ulp or two: Cody-Waite reduction with log2(e) split into a float32 head and
// tail, x log2(e) = k + f with k = rint(x log2(e)) and |f| <= 1/2, then
// v_exp_f32 (2^f) scaled by 2^k. f = fma(x, head, -k) + x tail: the fused
// product-difference is rounded once (a compensated form would be undone by
// the compiler's floating-point contraction). x <= 0 rules out overflow, so
// the only guard left is underflow: below ln(2^-149) the result is 0.
__device__ __forceinline__ float exp_nonpos(float x) {
  constexpr float kLog2eHi = 1.44269502162933349609375f;   // float32(log2 e)
  constexpr float kLog2eLo = 1.92596303e-08f;              // float32(log2 e - kLog2eHi)
  const float k = __builtin_rintf(x * kLog2eHi);
  const float f = fmaf(x, kLog2eHi, -k) + x * kLog2eLo;
  const float r = ldexpf(__builtin_amdgcn_exp2f(f), (int)k);
  return x < -103.278929903431851f ? 0.0f : r;
}

// 1 / (1 + e^-a) in float32 without a division: t = e^-|a| (exp_nonpos)
// lies in (0, 1], so d = 1 + t lies in (1, 2] and its reciprocal, by
// v_rcp_f32 refined with one Newton step, is normal and within an ulp of
// the quotient; sigma(a) = 1/d for a >= 0 and t/d for a < 0. That is 6
// instructions in place of the 12 of 1 + e^-a and an IEEE division (the
// SwiGLU kernels are bound by their VALU issue rate), at about the same
// accuracy (under 3 ulp), and sigma keeps e^a's subnormal range where
// e^-a would overflow. A NaN stays NaN.
__device__ __forceinline__ float sigmoid_f32(float a) {
  const float t = exp_nonpos(-fabsf(a));
  const float d = 1.0f + t;
  float r = __builtin_amdgcn_rcpf(d);
  r = fmaf(fmaf(-d, r, 1.0f), r, r);
  return a >= 0.0f ? r : t * r;
}

// silu(a) * b in float32.
__device__ __forceinline__ float swiglu_f32(float a, float b) {
  const float s = sigmoid_f32(a);
  return (a * s) * b;
}

__device__ __forceinline__ uint32_t swiglu_pair(uint32_t wa, uint32_t wb) {
  return pack_bf16x2(swiglu_f32(bf16_lo(wa), bf16_lo(wb)), swiglu_f32(bf16_hi(wa), bf16_hi(wb)));
}

}  // namespace mxk
