// FP8 E4M3 with one power-of-two scale per row, gfx950: the non-MX FP8
// grouped-mm training variant. Its scaling is not on the pages that define
// the method (they name FP8GroupedMMConfig and its ~10% tokens/s for FP8 MoE
// training, and say its support was set aside in favour of MXFP8); here each
// row of the quantized axis gets the scale the RCEIL rule picks for the whole
// row, and the weight gradient's operands get one scale per (column, group).
// The scale byte is written once per 32-block, in the k128 layout, so the
// operands are MX operands whose block scales along a row are equal and the
// MXFP8 GEMMs compute the row-scaled GEMM unchanged.
//
//   k_fp8_rowscale   16 whole rows per workgroup (16 lanes per row): a pass
//                    for the row maximum, a second pass for the codes
//   k_fp8_col_amax   per 128 x 128 tile, column maxima folded into the
//                    caller's int32 workspace [batch, segments, cols] with
//                    atomic max (segments: the groups of the row offsets,
//                    plus the rows after the last)
//   k_fp8_col_quant  per tile, column-wise codes with the column's scale
//                    (the shared column tile routine with given scales)
//   k_fp8_amax_rc    both directions at once: per tile, row maxima and
//                    column maxima folded into the workspace (one read)
//   k_fp8_dual_quant per tile, row-wise and column-wise codes from one read
//                    with the scales the maxima give

#include "mx_device.h"
#include "mx_kernels.h"
#include "mx_tile.h"

#include <algorithm>
#include <mutex>

namespace mxk {

// Work area of the allocation-free dual quantizer
// (mx_quantize_fp8_dual_scratch): a file-scope device array, so the call
// needs no allocation of its own. Each GPU the library runs on holds its own
// copy until the process ends. In host code the name is only a stand-in:
// kernels get the device address that hipGetSymbolAddress returns for the
// current device (fp8_scratch).
static __device__ __align__(256) int32_t scratch[kFp8ScratchInts];

namespace {
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[64];   // device address of `scratch`, per device
}  // namespace

hipError_t fp8_scratch(int32_t** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

constexpr int kRowsPerGroup = 16;   // rows of one k_fp8_rowscale workgroup

__global__ __launch_bounds__(256) void k_fp8_rowscale(Fp8Args a) {
  const int t = threadIdx.x, cc = t & 15;
  const int64_t b = blockIdx.y;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerGroup + (t >> 4);
  const bool ok = row < a.rows;
  const uint16_t* x = a.x + (b * a.rows + (ok ? row : 0)) * a.ld;
  const int steps = (int)(a.cols / 128);
  uint32_t m = 0;
  if (ok)
    for (int it = 0; it < steps; ++it)
      m = max(m, absmax8_bits(*reinterpret_cast<const uint4*>(x + it * 128 + cc * 8)));
  m = row16_max(m);
  const uint32_t sb = scale_byte(m, true);
  if (!ok) return;
  uint8_t* q = a.q + (b * a.rows + row) * a.cols;
  uint32_t* s = reinterpret_cast<uint32_t*>(a.s) + b * steps * a.rows;
  for (int it = 0; it < steps; ++it) {
    const uint4 v = *reinterpret_cast<const uint4*>(x + it * 128 + cc * 8);
    *reinterpret_cast<uint2*>(q + it * 128 + cc * 8) = e4m3_chunk(v, sb, false);
    if (cc == 0) s[it * a.rows + row] = sb * 0x01010101u;
  }
}

// Segment of row r: the first group whose end lies past r (E for the rows
// after the last end, or 0 without offsets).
__device__ __forceinline__ int row_segment(const Fp8Args& a, int64_t r) {
  if (!a.offs) return 0;
  int lo = 0, hi = a.E;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)a.offs[mid] > r) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// Zeroes the column maxima, and the row maxima that follow them when
// both directions are asked for. Wave 0 of workgroup 0 also checks the
// segment offsets: non-decreasing multiples of 128 no larger than rows (the
// grouped GEMMs' rule); otherwise bit 0 of *dev_err is set. Bad offsets only
// change which segment a tile's scales come from: row_segment's search
// always returns a segment in [0, E].
__global__ __launch_bounds__(256) void k_fp8_clear(Fp8Args a) {
  const int64_t n = a.batch * a.segments * a.cols + (a.row_max ? a.batch * a.rows : 0);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    a.work[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x < 64 && a.offs && a.dev_err) {
    const int lane = threadIdx.x;
    bool bad = false;
    int32_t prev_last = 0;
    for (int g0 = 0; g0 < a.E; g0 += 64) {
      const int g = g0 + lane;
      const int32_t v = g < a.E ? a.offs[g] : INT32_MAX;
      int32_t prev = __shfl_up(v, 1);
      if (lane == 0) prev = prev_last;
      if (g < a.E) bad |= (v & 127) != 0 || v < prev || (int64_t)v > a.rows;
      prev_last = __shfl(v, 63);
    }
    if (__any(bad) && lane == 0) atomicOr(a.dev_err, 1);
  }
}

// Column maxima of the tile held in v (tile_load layout, (0,0) at row r0,
// column c0 of batch entry b), folded into the column workspace with atomic
// max. part: 4 x kTC dwords of LDS. All threads must reach this function.
__device__ __forceinline__ void fold_col_max(const uint4 (&v)[kTileChunks], uint32_t (*part)[kTC], const Fp8Args& a,
                                             int64_t b, int64_t r0, int64_t c0) {
  const int t = threadIdx.x, cc = t & 15, lane = t & 63, w = t >> 6;
  // magnitudes of the thread's 8 columns, maximum over its 8 rows
  uint32_t m[4] = {0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < kTileChunks; ++j) {
    const uint32_t w4[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      m[k] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(mx_us2, m[k]),
                                                                    __builtin_bit_cast(mx_us2, w4[k] & 0x7FFF7FFFu)));
  }
  // the other rows of the wave with the same columns: lanes ^ 16, ^ 32
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int d = 16; d < 64; d <<= 1)
      m[k] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(mx_us2, m[k]),
                                                                    __builtin_bit_cast(mx_us2, (uint32_t)__shfl_xor((int)m[k], d))));
  }
  if (lane < 16)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      part[w][cc * 8 + 2 * k] = m[k] & 0xFFFFu;
      part[w][cc * 8 + 2 * k + 1] = m[k] >> 16;
    }
  __syncthreads();
  if (t < kTC) {
    const uint32_t mm = max(max(part[0][t], part[1][t]), max(part[2][t], part[3][t]));
    const int seg = row_segment(a, r0);
    atomicMax(reinterpret_cast<unsigned int*>(a.work) + (b * a.segments + seg) * a.cols + c0 + t, mm);
  }
}

__global__ __launch_bounds__(256) void k_fp8_col_amax(Fp8Args a) {
  __shared__ uint32_t part[4][kTC];
  const int64_t b = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * kTR, c0 = (int64_t)blockIdx.x * kTC;
  uint4 v[kTileChunks];
  tile_load(v, a.x + (b * a.rows + r0) * a.ld + c0, a.ld, kTR, kTC);
  fold_col_max(v, part, a, b, r0, c0);
}

// Both directions: the row maxima of the tile (the 16 lanes of a row reduce
// their chunks, as k_fp8_rowscale does over a whole row) and its column
// maxima, each folded into its workspace with atomic max.
__global__ __launch_bounds__(256) void k_fp8_amax_rc(Fp8Args a) {
  __shared__ uint32_t part[4][kTC];
  const int t = threadIdx.x;
  const int64_t b = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * kTR, c0 = (int64_t)blockIdx.x * kTC;
  uint4 v[kTileChunks];
  tile_load(v, a.x + (b * a.rows + r0) * a.ld + c0, a.ld, kTR, kTC);
#pragma unroll
  for (int j = 0; j < kTileChunks; ++j) {
    const uint32_t m = row16_max(absmax8_bits(v[j]));
    if ((t & 15) == 0)
      atomicMax(reinterpret_cast<unsigned int*>(a.row_max) + b * a.rows + r0 + (t >> 4) + 16 * j, m);
  }
  fold_col_max(v, part, a, b, r0, c0);
}

__global__ __launch_bounds__(256) void k_fp8_col_quant(Fp8Args a) {
  __shared__ uint4 lds[kTR * kTC / 8];
  __shared__ uint8_t sb[kTC];
  const int t = threadIdx.x;
  const int64_t b = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * kTR, c0 = (int64_t)blockIdx.x * kTC;
  if (t < kTC) {
    const int seg = row_segment(a, r0);
    const uint32_t mm = reinterpret_cast<const uint32_t*>(a.work)[(b * a.segments + seg) * a.cols + c0 + t];
    sb[t] = (uint8_t)scale_byte(mm, true);
  }
  uint4 v[kTileChunks];
  tile_load(v, a.x + (b * a.rows + r0) * a.ld + c0, a.ld, kTR, kTC);
  tile_to_lds(v, lds);
  __syncthreads();
  tile_colq(lds, kTR, kTC, true, TileOut{a.q + b * a.rows * a.cols, a.s + b * a.rows * (a.cols / kBlock), a.rows, a.cols, true},
            r0, c0, sb);
}

// Both directions from one read of the tile: row-wise codes with the scale
// of the row's maximum (as k_fp8_rowscale writes them) and column-wise codes
// with the scale of the column's (as k_fp8_col_quant writes them).
__global__ __launch_bounds__(256) void k_fp8_dual_quant(Fp8Args a) {
  __shared__ uint4 lds[kTR * kTC / 8];
  __shared__ uint8_t csb[kTC];
  __shared__ uint8_t rsb[kTR];
  const int t = threadIdx.x, cc = t & 15;
  const int64_t b = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * kTR, c0 = (int64_t)blockIdx.x * kTC;
  if (t < kTC) {
    const int seg = row_segment(a, r0);
    csb[t] = (uint8_t)scale_byte(reinterpret_cast<const uint32_t*>(a.work)[(b * a.segments + seg) * a.cols + c0 + t],
                                 true);
  } else {
    rsb[t - kTC] = (uint8_t)scale_byte(reinterpret_cast<const uint32_t*>(a.row_max)[b * a.rows + r0 + (t - kTC)],
                                       true);
  }
  uint4 v[kTileChunks];
  tile_load(v, a.x + (b * a.rows + r0) * a.ld + c0, a.ld, kTR, kTC);
  tile_to_lds(v, lds);
  __syncthreads();
  uint8_t* q = a.q + (b * a.rows + r0) * a.cols + c0 + cc * 8;
  uint32_t* s = reinterpret_cast<uint32_t*>(a.s) + (b * (a.cols / kTC) + c0 / kTC) * a.rows + r0;
#pragma unroll
  for (int j = 0; j < kTileChunks; ++j) {
    const int row = (t >> 4) + 16 * j;
    const uint32_t sb = rsb[row];
    *reinterpret_cast<uint2*>(q + row * a.cols) = e4m3_chunk(v[j], sb, false);
    if (cc == 0) s[row] = sb * 0x01010101u;
  }
  tile_colq(lds, kTR, kTC, true,
            TileOut{a.q_col + b * a.rows * a.cols, a.s_col + b * a.rows * (a.cols / kBlock), a.rows, a.cols, true},
            r0, c0, csb);
}

hipError_t launch_fp8_rowscale(const Fp8Args& a, hipStream_t s) {
  dim3 grid((unsigned)((a.rows + kRowsPerGroup - 1) / kRowsPerGroup), (unsigned)a.batch);
  hipLaunchKernelGGL(k_fp8_rowscale, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fp8_colscale(const Fp8Args& a, hipStream_t s) {
  const int64_t n = a.batch * a.segments * a.cols;
  hipLaunchKernelGGL(k_fp8_clear, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 4096)), dim3(256), 0, s, a);
  dim3 grid((unsigned)(a.cols / kTC), (unsigned)(a.rows / kTR), (unsigned)a.batch);
  hipLaunchKernelGGL(k_fp8_col_amax, grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_fp8_col_quant, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fp8_dual(const Fp8Args& a, hipStream_t s) {
  const int64_t n = a.batch * a.segments * a.cols + a.batch * a.rows;
  hipLaunchKernelGGL(k_fp8_clear, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 4096)), dim3(256), 0, s, a);
  dim3 grid((unsigned)(a.cols / kTC), (unsigned)(a.rows / kTR), (unsigned)a.batch);
  hipLaunchKernelGGL(k_fp8_amax_rc, grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_fp8_dual_quant, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mxk
