// Bandwidth-bound kernels of the MXFP8 hot path on gfx950:
//   k_quant_tile      MX block quantization, row-wise and/or column-wise
//   k_swiglu_fwd      fused SwiGLU + dual MX quantization (forward)
//   k_swiglu_bwd      fused SwiGLU backward + dual MX quantization
//   k_dequant         E4M3 x E8M0 -> float32 / bf16
//
// All four share one tile scheme. A 256-thread workgroup owns a 128 x 128
// tile of bf16 values (k_quant_tile: two adjacent ones). Thread t holds 8
// chunks of 8 consecutive values per tile (one 16-byte load each): chunk j
// sits at tile row (t >> 4) + 16 j, columns
// 8 (t & 15) .. 8 (t & 15) + 7, so the 4 lanes of a quad hold one 32-value
// row block and the block maximum is two DPP quad permutes away.
// Row-wise quantization is done straight from registers. For column-wise
// quantization the tile is written to LDS (XOR-swizzled 16-byte units) and
// each lane reads back 16 rows of a column pair (one dword per row); the 8
// lanes of a column pair together hold one 128-code output row, so every
// store instruction writes whole 128-byte lines.
//
// The fused SwiGLU kernels produce their tile in registers from the inputs
// (h = silu(a) * b, or dA / dB), round it to bf16 and run the same two
// quantizations, so the bf16 activation never goes to memory unless asked.

#include "mx_device.h"
#include "mx_kernels.h"
#include "mx_tile.h"

#include <algorithm>

namespace mxk {

// tile_load through a row map: tile row `row` reads input row
// src_row[r0 + row], or zeros where that is negative or past src_rows. The
// tile's 128 map entries are loaded once into LDS (one load by each of 128
// threads) rather than by every thread for each of its 8 rows: the fused
// pad + quantize launches of the MoE Scout step took 16% less time.
// Every thread of the workgroup must call it (it holds a barrier); a second
// call for the same rows rewrites the same entries.
template <bool NT>
__device__ __forceinline__ void tile_load_gather(uint4 (&v)[kTileChunks], const uint16_t* x, int64_t ld,
                                                 const int32_t* src_row, int64_t src_rows, int64_t r0,
                                                 int64_t c0, int rows_valid, int cols_valid) {
  const int t = threadIdx.x;
  const int cc = t & 15;
  __shared__ int32_t smap[kTR];
  if (t < kTR) smap[t] = t < rows_valid ? src_row[r0 + t] : -1;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kTileChunks; ++j) {
    const int row = (t >> 4) + 16 * j;
    const int64_t src = smap[row];
    v[j] = (src >= 0 && src < src_rows && cc * 8 < cols_valid)
               ? (NT ? load_stream16(x + src * ld + c0 + cc * 8)
                     : *reinterpret_cast<const uint4*>(x + src * ld + c0 + cc * 8))
               : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void tile_store_bf16(const uint4 (&v)[kTileChunks], uint16_t* base,
                                                int64_t ld, int rows_valid, int cols_valid) {
  const int t = threadIdx.x;
  const int cc = t & 15;
#pragma unroll
  for (int j = 0; j < kTileChunks; ++j) {
    const int row = (t >> 4) + 16 * j;
    if (row < rows_valid && cc * 8 < cols_valid)
      *reinterpret_cast<uint4*>(base + row * ld + cc * 8) = v[j];
  }
}

// ---------------------------------------------------------------- quantize

// TILES (1 or 2) adjacent 128 x 128 tiles of the same 128 rows per
// workgroup. With two, each row is read as 512 contiguous bytes and its
// row-wise codes written as 256 (at 3 waves per SIMD instead of 5): on
// MI355X the 1.3-2.7 GB expert-weight launches took 3-4% less time and
// column-only quantization of a 448 MiB tensor 11% less, while launches
// through a row map (padding) or with fewer than 48 one-tile workgroups per
// CU took 8-27% more. launch_quant picks per launch. Both tiles are loaded
// before either is quantized; the column-wise pass reuses one LDS tile.
// COL: column-wise output requested (the LDS tile exists only then).
// NT: non-temporal loads.
template <bool COL, bool NT, int TILES>
__global__ __launch_bounds__(kTileThreads) void k_quant_tile(QuantArgs a) {
  const int64_t bz = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * kTR;
  const int rows_valid = (int)min<int64_t>(kTR, a.rows - r0);
  uint4 v[TILES][kTileChunks];
#pragma unroll
  for (int h = 0; h < TILES; ++h) {
    const int64_t c0 = ((int64_t)blockIdx.x * TILES + h) * kTC;
    const int cols_valid = (int)min<int64_t>(kTC, a.cols - c0);
    if (a.src_row)
      tile_load_gather<NT>(v[h], a.x, a.ld, a.src_row, a.src_rows, r0, c0, rows_valid, cols_valid);
    else
      tile_load<NT>(v[h], a.x + (bz * a.rows + r0) * a.ld + c0, a.ld, rows_valid, cols_valid);
  }
#pragma unroll
  for (int h = 0; h < TILES; ++h) {
    const int64_t c0 = ((int64_t)blockIdx.x * TILES + h) * kTC;
    const int cols_valid = (int)min<int64_t>(kTC, a.cols - c0);
    if (a.q_row) {
      TileOut o{a.q_row + bz * a.rows * a.cols, a.s_row + bz * a.rows * (a.cols / kBlock), a.cols, a.rows, a.k128};
      tile_rowq(v[h], rows_valid, cols_valid, a.rceil, o, r0, c0);
    }
  }
  if constexpr (COL) {
    __shared__ uint4 lds[kTR * kTC / 8];
#pragma unroll
    for (int h = 0; h < TILES; ++h) {
      const int64_t c0 = ((int64_t)blockIdx.x * TILES + h) * kTC;
      const int cols_valid = (int)min<int64_t>(kTC, a.cols - c0);
      if (h) __syncthreads();
      tile_to_lds(v[h], lds);
      __syncthreads();
      TileOut o{a.q_col + bz * a.rows * a.cols, a.s_col + bz * a.cols * (a.rows / kBlock), a.rows, a.cols, a.k128};
      tile_colq(lds, rows_valid, cols_valid, a.rceil, o, r0, c0);
    }
  }
}

// ---------------------------------------------------------------- SwiGLU

template <bool NT>
__global__ __launch_bounds__(kTileThreads) void k_swiglu_fwd(SwigluFwdArgs a) {
  __shared__ uint4 lds[kTR * kTC / 8];
  const int64_t r0 = (int64_t)blockIdx.y * kTR;
  const int64_t c0 = (int64_t)blockIdx.x * kTC;
  const int rows_valid = (int)min<int64_t>(kTR, a.rows - r0);
  const int cols_valid = (int)min<int64_t>(kTC, a.hidden - c0);
  uint4 v[kTileChunks], w[kTileChunks];
  tile_load<NT>(v, a.a + r0 * a.ld_ab + c0, a.ld_ab, rows_valid, cols_valid);
  tile_load<NT>(w, a.b + r0 * a.ld_ab + c0, a.ld_ab, rows_valid, cols_valid);
#pragma unroll
  for (int j = 0; j < kTileChunks; ++j)
    v[j] = make_uint4(swiglu_pair(v[j].x, w[j].x), swiglu_pair(v[j].y, w[j].y),
                      swiglu_pair(v[j].z, w[j].z), swiglu_pair(v[j].w, w[j].w));
  if (a.h_out) tile_store_bf16(v, a.h_out + r0 * a.hidden + c0, a.hidden, rows_valid, cols_valid);
  tile_rowq(v, rows_valid, cols_valid, a.rceil, TileOut{a.q_row, a.s_row, a.hidden, a.rows, a.k128}, r0, c0);
  tile_to_lds(v, lds);
  __syncthreads();
  tile_colq(lds, rows_valid, cols_valid, a.rceil, TileOut{a.q_col, a.s_col, a.rows, a.hidden, a.k128}, r0, c0);
}

// dA = dh*b*s*(1 + a*(1-s)), dB = dh*a*s with s = sigmoid(a), float32.
__device__ __forceinline__ void swiglu_grad_f32(float dh, float a, float b, float& da,
                                                float& db) {
  const float s = sigmoid_f32(a);
  da = (dh * b) * (s * (1.0f + a * (1.0f - s)));
  db = dh * (a * s);
}

__device__ __forceinline__ void swiglu_grad_pair(uint32_t wdh, uint32_t wa, uint32_t wb,
                                                 uint32_t& da2, uint32_t& db2) {
  float da0, db0, da1, db1;
  swiglu_grad_f32(bf16_lo(wdh), bf16_lo(wa), bf16_lo(wb), da0, db0);
  swiglu_grad_f32(bf16_hi(wdh), bf16_hi(wa), bf16_hi(wb), da1, db1);
  da2 = pack_bf16x2(da0, da1);
  db2 = pack_bf16x2(db0, db1);
}

template <bool NT>
__global__ __launch_bounds__(kTileThreads) void k_swiglu_bwd(SwigluBwdArgs a) {
  __shared__ uint4 lds[kTR * kTC / 8];
  const int64_t r0 = (int64_t)blockIdx.y * kTR;
  const int64_t c0 = (int64_t)blockIdx.x * kTC;
  const int rows_valid = (int)min<int64_t>(kTR, a.rows - r0);
  const int cols_valid = (int)min<int64_t>(kTC, a.hidden - c0);
  const int64_t H2 = 2 * a.hidden;
  uint4 da[kTileChunks], db[kTileChunks];
  {
    uint4 vdh[kTileChunks], va[kTileChunks];
    tile_load<NT>(vdh, a.dh + r0 * a.ld_dh + c0, a.ld_dh, rows_valid, cols_valid);
    tile_load<NT>(va, a.a + r0 * a.ld_ab + c0, a.ld_ab, rows_valid, cols_valid);
    tile_load<NT>(db, a.b + r0 * a.ld_ab + c0, a.ld_ab, rows_valid, cols_valid);
#pragma unroll
    for (int j = 0; j < kTileChunks; ++j) {
      uint4 x, y;
      swiglu_grad_pair(vdh[j].x, va[j].x, db[j].x, x.x, y.x);
      swiglu_grad_pair(vdh[j].y, va[j].y, db[j].y, x.y, y.y);
      swiglu_grad_pair(vdh[j].z, va[j].z, db[j].z, x.z, y.z);
      swiglu_grad_pair(vdh[j].w, va[j].w, db[j].w, x.w, y.w);
      da[j] = x;
      db[j] = y;
    }
  }
  if (a.dab_out) {
    tile_store_bf16(da, a.dab_out + r0 * H2 + c0, H2, rows_valid, cols_valid);
    tile_store_bf16(db, a.dab_out + r0 * H2 + a.hidden + c0, H2, rows_valid, cols_valid);
  }
  const TileOut orow{a.q_row, a.s_row, H2, a.rows, a.k128};
  tile_rowq(da, rows_valid, cols_valid, a.rceil, orow, r0, c0);
  tile_rowq(db, rows_valid, cols_valid, a.rceil, orow, r0, a.hidden + c0);
  const TileOut ocol{a.q_col, a.s_col, a.rows, H2, a.k128};
  tile_to_lds(da, lds);
  __syncthreads();
  tile_colq(lds, rows_valid, cols_valid, a.rceil, ocol, r0, c0);
  __syncthreads();
  tile_to_lds(db, lds);
  __syncthreads();
  tile_colq(lds, rows_valid, cols_valid, a.rceil, ocol, r0, a.hidden + c0);
}

// ---------------------------------------------------------------- dequantize

// Each thread converts the codes behind one 16-byte output store (8 codes to
// bf16, 4 to float32), so the lanes of a store instruction write 1 KB of
// consecutive bytes; it loads those codes (8 or 4 bytes, also consecutive
// across lanes) and their block's scale byte. Chunk i (kCodes codes) is row
// i / (cols / kCodes); the quotient comes from a precomputed multiplier
// (FastDiv, 32-bit) when the chunk count fits 32 bits, from 64-bit
// division otherwise (IDX64). The grid-stride loop takes kUnroll chunks per
// pass and issues all their loads before converting any, so that several
// loads per wave are in flight.
template <bool F32, bool IDX64>
__device__ __forceinline__ void dequant_load(const DequantArgs& a, FastDiv per_row, int64_t per, int64_t i,
                                             uint32_t (&w)[F32 ? 1 : 2], uint32_t& sb) {
  constexpr int kCodes = F32 ? 4 : 8;
  if constexpr (F32) {
    w[0] = *reinterpret_cast<const uint32_t*>(a.q + 4 * i);
  } else {
    const uint2 c = *reinterpret_cast<const uint2*>(a.q + 8 * i);
    w[0] = c.x;
    w[1] = c.y;
  }
  int64_t r, cc;
  if constexpr (IDX64) {
    r = i / per;
    cc = i - r * per;
  } else {
    const uint32_t rr = fdiv((uint32_t)i, per_row);
    r = rr;
    cc = (int64_t)((uint32_t)i - rr * per_row.d);
  }
  const int64_t blk = (cc * kCodes) >> 5;
  sb = a.k128 ? a.s[((blk >> 2) * a.rows + r) * 4 + (blk & 3)] : a.s[r * (a.cols / 32) + blk];
}

template <bool F32>
__device__ __forceinline__ void dequant_store(const DequantArgs& a, int64_t i, const uint32_t (&w)[F32 ? 1 : 2],
                                              uint32_t sb) {
  constexpr int kCodes = F32 ? 4 : 8;
  float f[kCodes];
#pragma unroll
  for (int k = 0; k < kCodes; ++k) {
    const float v = e4m3_value((w[k >> 2] >> (8 * (k & 3))) & 0xFFu);
    // v has at most 4 significant bits and |v| >= 2^-9, so v * 2^(sb-127)
    // is exact in float32 down to 2^-136 (a float32 subnormal); only
    // E = 127 with |v| > 1 overflows, to infinity
    f[k] = sb == 0xFFu ? __uint_as_float(0x7FC00000u) : ldexpf(v, (int)sb - 127);
  }
  if constexpr (F32)
    reinterpret_cast<float4*>(a.out)[i] = make_float4(f[0], f[1], f[2], f[3]);
  else
    reinterpret_cast<uint4*>(a.out)[i] = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                                   pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}

template <bool F32, bool IDX64>
__global__ __launch_bounds__(256) void k_dequant(DequantArgs a, FastDiv per_row) {
  constexpr int kCodes = F32 ? 4 : 8;
  constexpr int kUnroll = 4;
  const int64_t per = a.cols / kCodes;
  const int64_t n = a.rows * per;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    uint32_t w[kUnroll][F32 ? 1 : 2], sb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) dequant_load<F32, IDX64>(a, per_row, per, i + u * stride, w[u], sb[u]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) dequant_store<F32>(a, i + u * stride, w[u], sb[u]);
  }
  for (; i < n; i += stride) {
    uint32_t w[F32 ? 1 : 2], sb;
    dequant_load<F32, IDX64>(a, per_row, per, i, w, sb);
    dequant_store<F32>(a, i, w, sb);
  }
}

}  // namespace mxk

// ---------------------------------------------------------------- launch

namespace mxk {

// Launches whose bf16 inputs total less than this read them with
// non-temporal loads. Measured on MI355X in the routed-experts MLP step and
// on a [32768, 7168] tensor: below it the non-temporal reads were 5-16%
// faster (188 MB activations, the 448 MiB tensor, the 0.9 GB SwiGLU
// backward inputs); on the 1.3 and 2.7 GB expert weights they were 2-7%
// slower, so those keep plain loads.
constexpr int64_t kStreamBytes = (int64_t)1 << 30;

template <int TILES>
static void launch_quant_t(const QuantArgs& a, int64_t batch, bool nt, hipStream_t s) {
  dim3 grid((unsigned)((a.cols + TILES * kTC - 1) / (TILES * kTC)), (unsigned)((a.rows + kTR - 1) / kTR),
            (unsigned)batch);
  if (a.q_col) {
    if (nt) hipLaunchKernelGGL((k_quant_tile<true, true, TILES>), grid, dim3(kTileThreads), 0, s, a);
    else hipLaunchKernelGGL((k_quant_tile<true, false, TILES>), grid, dim3(kTileThreads), 0, s, a);
  } else {
    if (nt) hipLaunchKernelGGL((k_quant_tile<false, true, TILES>), grid, dim3(kTileThreads), 0, s, a);
    else hipLaunchKernelGGL((k_quant_tile<false, false, TILES>), grid, dim3(kTileThreads), 0, s, a);
  }
}

// Two tiles per workgroup without a row map once the one-tile grid has at
// least 48 workgroups per CU (see k_quant_tile).
constexpr int64_t kPairMinTiles = 48 * 256;

hipError_t launch_quant(const QuantArgs& a, int64_t batch, hipStream_t s) {
  const bool nt = batch * a.rows * a.cols * 2 < kStreamBytes;
  const int64_t tiles = ((a.cols + kTC - 1) / kTC) * ((a.rows + kTR - 1) / kTR) * batch;
  if (!a.src_row && tiles >= kPairMinTiles)
    launch_quant_t<2>(a, batch, nt, s);
  else
    launch_quant_t<1>(a, batch, nt, s);
  return hipGetLastError();
}

hipError_t launch_swiglu_fwd(const SwigluFwdArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.hidden + kTC - 1) / kTC), (unsigned)((a.rows + kTR - 1) / kTR));
  if (2 * a.rows * a.hidden * 2 < kStreamBytes)
    hipLaunchKernelGGL(k_swiglu_fwd<true>, grid, dim3(kTileThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_swiglu_fwd<false>, grid, dim3(kTileThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const SwigluBwdArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.hidden + kTC - 1) / kTC), (unsigned)((a.rows + kTR - 1) / kTR));
  if (3 * a.rows * a.hidden * 2 < kStreamBytes)
    hipLaunchKernelGGL(k_swiglu_bwd<true>, grid, dim3(kTileThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_swiglu_bwd<false>, grid, dim3(kTileThreads), 0, s, a);
  return hipGetLastError();
}

template <bool F32>
static hipError_t launch_dequant_t(const DequantArgs& a, hipStream_t s) {
  constexpr int kCodes = F32 ? 4 : 8;
  const int64_t n = a.rows * a.cols / kCodes;
  if (n == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 256 * 64);
  // the grid-stride index stays below n + 4 x grid size (the unrolled pass
  // reads up to three strides ahead, all below n); 32-bit quotients need
  // that below 2^32
  if (n + 4 * blocks * 256 < ((int64_t)1 << 32))
    hipLaunchKernelGGL((k_dequant<F32, false>), dim3((unsigned)blocks), dim3(256), 0, s, a,
                       make_fastdiv((uint32_t)(a.cols / kCodes)));
  else
    hipLaunchKernelGGL((k_dequant<F32, true>), dim3((unsigned)blocks), dim3(256), 0, s, a, FastDiv{});
  return hipGetLastError();
}

hipError_t launch_dequant(const DequantArgs& a, hipStream_t s) {
  return a.out_f32 ? launch_dequant_t<true>(a, s) : launch_dequant_t<false>(a, s);
}

}  // namespace mxk
