// Per-group token padding / unpadding and the bf16 grouped weight gradient
// of the wgrad_with_hp recipe, gfx950.
//
// k_pad / k_unpad are row copies: one wave per row, 16 bytes per lane per
// step. Every workgroup of k_pad first rebuilds the group table (per-group
// source starts and padded slot ends, a prefix sum over E <= 1024 groups done
// by wave 0 with shuffles), then maps each of its padded rows to its source
// row by binary search over the slot ends.
//
// k_hp_wgrad computes dW[g] = G[s:e]^T X[s:e] for bf16 G [Tcap, N] and
// X [Tcap, K] with v_mfma_f32_32x32x16_bf16. Tokens (the contraction) are the
// strided axis of both operands, so tiles of 32 tokens are staged in LDS as
// loaded (row = token) and each lane gathers its 8 consecutive tokens of one
// column with 16-bit LDS reads.

#include "mx_device.h"
#include "mx_kernels.h"

#include <algorithm>

namespace mxk {

constexpr int kPadMaxGroups = 1024;

// Inclusive prefix sum over one wave.
__device__ __forceinline__ int32_t wave_scan(int32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int32_t o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

__global__ __launch_bounds__(256) void k_pad(PadArgs a) {
  __shared__ int32_t src_start[kPadMaxGroups];
  __shared__ int32_t slot_end[kPadMaxGroups];
  __shared__ int32_t sizes_s[kPadMaxGroups];
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int32_t carry_src = 0, carry_slot = 0;
    bool bad = false;
    for (int g0 = 0; g0 < a.E; g0 += 64) {
      const int g = g0 + lane;
      int32_t n = g < a.E ? a.sizes[g] : 0;
      bad |= n < 0;
      n = max(n, 0);
      const int32_t slot = (n + a.multiple - 1) / a.multiple * a.multiple;
      const int32_t inc_src = wave_scan(n) + carry_src;
      const int32_t inc_slot = wave_scan(slot) + carry_slot;
      if (g < a.E) {
        sizes_s[g] = n;
        src_start[g] = inc_src - n;
        slot_end[g] = inc_slot;
      }
      carry_src = __shfl(inc_src, 63);
      carry_slot = __shfl(inc_slot, 63);
    }
    bad = __any(bad) || (int64_t)carry_src != a.T || (int64_t)carry_slot > a.Tcap;
    if (blockIdx.x == 0 && lane == 0 && bad && a.dev_err) atomicOr(a.dev_err, 2);
  }
  __syncthreads();
  if (blockIdx.x == 0)
    for (int g = threadIdx.x; g < a.E; g += blockDim.x) a.offs_pad[g] = slot_end[g];

  const int lane = threadIdx.x & 63;
  const int64_t rows_per_block = blockDim.x / 64;
  const int64_t r = (int64_t)blockIdx.x * rows_per_block + (threadIdx.x >> 6);
  if (r >= a.Tcap) return;
  // first group whose slot ends past r
  int lo = 0, hi = a.E;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (slot_end[mid] > r) hi = mid; else lo = mid + 1;
  }
  int64_t src = -1;
  if (lo < a.E) {
    const int64_t i = r - (lo == 0 ? 0 : slot_end[lo - 1]);
    if (i < sizes_s[lo]) src = src_start[lo] + i;
    if (src >= a.T) src = -1;
  }
  if (lane == 0) a.src_row[r] = (int32_t)src;
  uint4* dst = reinterpret_cast<uint4*>(a.x_pad + r * a.row_bytes);
  const int64_t n16 = a.row_bytes / 16;
  if (src >= 0) {
    const uint4* s = reinterpret_cast<const uint4*>(a.x + src * a.row_bytes);
    for (int64_t c = lane; c < n16; c += 64) dst[c] = s[c];
  } else {
    for (int64_t c = lane; c < n16; c += 64) dst[c] = make_uint4(0, 0, 0, 0);
  }
}

__global__ __launch_bounds__(256) void k_unpad(UnpadArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (r >= a.Tcap) return;
  const int64_t src = a.src_row[r];
  if (src < 0 || src >= a.T) return;
  const uint4* s = reinterpret_cast<const uint4*>(a.y_pad + r * a.row_bytes);
  uint4* d = reinterpret_cast<uint4*>(a.y + src * a.row_bytes);
  const int64_t n16 = a.row_bytes / 16;
  for (int64_t c = lane; c < n16; c += 64) d[c] = s[c];
}

hipError_t launch_pad(const PadArgs& a, hipStream_t s) {
  // at least one workgroup: it also writes offs_pad
  hipLaunchKernelGGL(k_pad, dim3((unsigned)std::max<int64_t>(1, (a.Tcap + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_unpad(const UnpadArgs& a, hipStream_t s) {
  if (a.Tcap == 0) return hipSuccess;
  hipLaunchKernelGGL(k_unpad, dim3((unsigned)((a.Tcap + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- hp wgrad

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kHpBM = 128, kHpBN = 128, kHpBK = 32;   // dW rows (N), cols (K), tokens

__global__ __launch_bounds__(256) void k_hp_wgrad(HpWgradArgs a) {
  __shared__ uint16_t sg[kHpBK][kHpBM];   // G tile: [token][n]
  __shared__ uint16_t sx[kHpBK][kHpBN];   // X tile: [token][k]
  __shared__ int32_t ends[kPadMaxGroups];
  // cleaned group ends (see the MXFP8 grouped GEMMs): clamp, align, monotone
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int32_t carry = 0, prev_raw = 0;
    bool bad = false;
    for (int g0 = 0; g0 < a.E; g0 += 64) {
      const int g = g0 + lane;
      const int32_t raw = g < a.E ? a.offs[g] : INT32_MAX;
      int32_t c = (int32_t)min<int64_t>(max(raw, 0), a.Tcap) & ~127;
      bad |= g < a.E && c != raw;
      int32_t prev = __shfl_up(raw, 1);
      if (lane == 0) prev = prev_raw;
      bad |= g < a.E && raw < prev;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        int32_t o = __shfl_up(c, d);
        if (lane >= d) c = max(c, o);
      }
      c = max(c, carry);
      if (g < a.E) ends[g] = c;
      carry = __shfl(c, 63);
      prev_raw = __shfl(raw, 63);
    }
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && lane == 0 && __any(bad) &&
        a.dev_err)
      atomicOr(a.dev_err, 1);
  }
  __syncthreads();
  const int g = blockIdx.z;
  const int64_t t0 = g == 0 ? 0 : ends[g - 1];
  const int64_t t1 = ends[g];
  const int64_t n0 = (int64_t)blockIdx.y * kHpBM;
  const int64_t k0 = (int64_t)blockIdx.x * kHpBN;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int wm = w >> 1, wn = w & 1;   // wave owns a 64 x 64 sub-tile
  const int vn = (int)min<int64_t>(kHpBM, a.N - n0);
  const int vk = (int)min<int64_t>(kHpBN, a.K - k0);

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  // loader: 32 tokens x 128 columns x 2 B = 8 KB per operand = 512 chunks of
  // 16 B; thread t loads chunk t and t + 256 of each (row = id / 16)
  for (int64_t tk = t0; tk < t1; tk += kHpBK) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int id = t + 256 * h;
      const int row = id >> 4, c8 = (id & 15) * 8;
      const uint4 zero = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(&sg[row][c8]) =
          c8 < vn ? *reinterpret_cast<const uint4*>(a.g + (tk + row) * a.N + n0 + c8) : zero;
      *reinterpret_cast<uint4*>(&sx[row][c8]) =
          c8 < vk ? *reinterpret_cast<const uint4*>(a.x + (tk + row) * a.K + k0 + c8) : zero;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {   // two 16-token MFMA steps
      v8bf av[2], bv[2];
      const int kk = 16 * s + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int col_a = wm * 64 + 32 * i + (lane & 31);
        const int col_b = wn * 64 + 32 * i + (lane & 31);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          av[i][e] = __builtin_bit_cast(__bf16, sg[kk + e][col_a]);
          bv[i][e] = __builtin_bit_cast(__bf16, sx[kk + e][col_b]);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  uint16_t* out = a.out + g * a.N * a.K;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = wn * 64 + 32 * j + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < vn && col < vk)
          out[(n0 + row) * a.K + k0 + col] = (uint16_t)f32_to_bf16(acc[i][j][r]);
      }
    }
}

hipError_t launch_hp_wgrad(const HpWgradArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.K + kHpBN - 1) / kHpBN), (unsigned)((a.N + kHpBM - 1) / kHpBM),
            (unsigned)a.E);
  hipLaunchKernelGGL(k_hp_wgrad, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mxk
