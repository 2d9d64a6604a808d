// Per-group token padding / unpadding, gfx950.
//
// k_pad / k_unpad are row copies: one wave per row, 16 bytes per lane per
// step. Every workgroup of k_pad first rebuilds the group table (per-group
// source starts and padded slot ends, a prefix sum over E <= 1024 groups done
// by wave 0 with shuffles), then maps each of its padded rows to its source
// row by binary search over the slot ends. k_pad_map writes that row map
// (and the padded offsets) without copying any row.
//

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

struct GroupTable {
  int32_t src_start[kPadMaxGroups];   // first source row of each group
  int32_t slot_end[kPadMaxGroups];    // exclusive end of each group's padded slot
  int32_t sizes[kPadMaxGroups];
};

// Builds the group table in LDS (wave 0, prefix sums with shuffles); ends
// with a workgroup barrier. Workgroup 0 also writes offs_pad and reports
// negative sizes, sizes that do not add up to T, or slots past Tcap.
__device__ void build_group_table(const PadArgs& a, GroupTable& gt) {
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
        gt.sizes[g] = n;
        gt.src_start[g] = inc_src - n;
        gt.slot_end[g] = inc_slot;
      }
      carry_src = __shfl(inc_src, 63);
      carry_slot = __shfl(inc_slot, 63);
    }
    bad = __any(bad) || (int64_t)carry_src != a.T || (int64_t)carry_slot > a.Tcap;
    if (blockIdx.x == 0 && lane == 0 && bad && a.dev_err) atomicOr(a.dev_err, 2);
  }
  __syncthreads();
  if (blockIdx.x == 0)
    for (int g = threadIdx.x; g < a.E; g += blockDim.x) a.offs_pad[g] = gt.slot_end[g];
}

// Source row of padded row r, or -1 for pad rows and the tail.
__device__ __forceinline__ int64_t padded_source(const PadArgs& a, const GroupTable& gt, int64_t r) {
  // first group whose slot ends past r
  int lo = 0, hi = a.E;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (gt.slot_end[mid] > r) hi = mid; else lo = mid + 1;
  }
  int64_t src = -1;
  if (lo < a.E) {
    const int64_t i = r - (lo == 0 ? 0 : gt.slot_end[lo - 1]);
    if (i < gt.sizes[lo]) src = gt.src_start[lo] + i;
    if (src >= a.T) src = -1;
  }
  return src;
}

__global__ __launch_bounds__(256) void k_pad(PadArgs a) {
  __shared__ GroupTable gt;
  build_group_table(a, gt);
  const int lane = threadIdx.x & 63;
  const int64_t rows_per_block = blockDim.x / 64;
  const int64_t r = (int64_t)blockIdx.x * rows_per_block + (threadIdx.x >> 6);
  if (r >= a.Tcap) return;
  const int64_t src = padded_source(a, gt, r);
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

// The row map alone (for consumers that gather rows themselves, such as the
// fused pad + quantize): one padded row per thread.
__global__ __launch_bounds__(256) void k_pad_map(PadArgs a) {
  __shared__ GroupTable gt;
  build_group_table(a, gt);
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r < a.Tcap) a.src_row[r] = (int32_t)padded_source(a, gt, r);
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

hipError_t launch_pad_map(const PadArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_pad_map, dim3((unsigned)std::max<int64_t>(1, (a.Tcap + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_unpad(const UnpadArgs& a, hipStream_t s) {
  if (a.Tcap == 0) return hipSuccess;
  hipLaunchKernelGGL(k_unpad, dim3((unsigned)((a.Tcap + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mxk
