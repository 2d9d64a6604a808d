// MXFP8 scaled GEMMs on gfx950 block-scaled FP8 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4: E4M3 x E4M3 with one E8M0 scale per
// 32-element K block of each operand row, float32 accumulation).
//
// Every GEMM here is C[m, n] = sum_k A[m, k] B[n, k], both operands row-major
// with K contiguous, scales [rows, K/32]. Three kernels share one tile
// routine:
//   k_gemm_dense    one matrix pair (the linear layer's fwd / dgrad / wgrad)
//   k_gemm_grouped  2-D x 3-D: row tiles of A belong to one expert group and
//                   multiply that expert's B (grouped fwd and dgrad)
//   k_gemm_wgrad    2-D x 2-D: per expert, the contraction runs over the
//                   group's own token range (grouped weight gradient)
//
// Tile routine: a 256-thread workgroup computes a 256 x 256 output tile in
// K steps of 128 (four scale blocks). Waves form a 2 x 2 grid, each owning a
// 128 x 128 sub-tile = 4 x 4 MFMA blocks of 32 x 32 (256 float accumulators
// per lane). Per K step the workgroup stages A and B (32 KB each) and their
// scale dwords in LDS, double-buffered: the global loads of step k+1 are in
// flight while step k's MFMAs run. LDS rows are 128 bytes with the 16-byte
// pieces XOR-swizzled by (row & 7), so the 8 lanes that read one piece
// column of 8 consecutive rows hit 8 different bank groups.
//
// MFMA operand layout (32x32x64, 8-bit elements, measured on the device):
// lane l holds row (l & 31) of its 32-row block; with h = l >> 5 its bytes
// 0..15 are K = 16 h .. 16 h + 15 and its bytes 16..31 are K = 32 + 16 h ..
// 32 + 16 h + 15. Its scale byte covers row (l & 31) and K block h (K = 32 h
// .. 32 h + 31), i.e. scale lanes 0..31 serve the low K half and 32..63 the
// high half. Output register i of lane l is
// C[8 (i >> 2) + 4 (l >> 5) + (i & 3)][l & 31].

#include "mx_device.h"
#include "mx_kernels.h"

namespace mxk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kGemmThreads = 256;
constexpr int kStageA = kBM * kBK;                     // bytes of codes per stage
constexpr int kStageB = kBN * kBK;
constexpr int kLdsCodes = 2 * (kStageA + kStageB);     // 128 KB
constexpr int kLdsBytes = kLdsCodes + 2 * (kBM + kBN) * 4;
constexpr int kMaxGroups = 1024;                       // group table lives in LDS

struct TileSpec {
  const uint8_t* a;   // codes of A row 0 of the tile (K index 0)
  const uint8_t* sa;  // scales of A row 0
  const uint8_t* b;
  const uint8_t* sb;
  int64_t lda, ldb, ldsa, ldsb;
  int valid_m, valid_n;  // A rows / B rows that exist in this tile (1..256)
  int64_t k_begin;       // first contraction index, multiple of 128
  int nk;                // number of 128-wide K steps (0 => C = 0)
  void* out;             // C(0, 0) of the tile
  int64_t ldo;
  bool out_f32;
};

template <int OPSEL>
__device__ __forceinline__ v16f mfma_mx(const v8i& a, const v8i& b, const v16f& c, uint32_t sa,
                                        uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPSEL, (int)sa, OPSEL,
                                                         (int)sb);
}

__device__ __forceinline__ v8i cat8(uint4 x, uint4 y) {
  return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}

__device__ __forceinline__ void store_tile(const v16f (&acc)[4][4], const TileSpec& ts) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = wn * 128 + 32 * j + (lane & 31);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int row = wm * 128 + 32 * i + 8 * (k >> 2) + 4 * (lane >> 5) + (k & 3);
        if (row < ts.valid_m && col < ts.valid_n) {
          if (ts.out_f32)
            reinterpret_cast<float*>(ts.out)[row * ts.ldo + col] = acc[i][j][k];
          else
            reinterpret_cast<uint16_t*>(ts.out)[row * ts.ldo + col] =
                (uint16_t)f32_to_bf16(acc[i][j][k]);
        }
      }
    }
  }
}

// Writes zeros over a valid_m x valid_n tile (tail rows, empty groups).
__device__ __forceinline__ void zero_tile(const TileSpec& ts) {
  const int esz = ts.out_f32 ? 4 : 2;
  const int row_bytes = ts.valid_n * esz;
  uint8_t* base = reinterpret_cast<uint8_t*>(ts.out);
  for (int r = threadIdx.x >> 4; r < ts.valid_m; r += kGemmThreads / 16) {
    uint8_t* row = base + (int64_t)r * ts.ldo * esz;
    for (int c = (threadIdx.x & 15) * 4; c < row_bytes; c += 64)
      *reinterpret_cast<uint32_t*>(row + c) = 0u;
  }
}

__device__ __forceinline__ void gemm_tile(const TileSpec& ts, uint8_t* lds) {
  if (ts.nk <= 0) {
    zero_tile(ts);
    return;
  }
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int wm = w >> 1, wn = w & 1;

  uint4* ldsA = reinterpret_cast<uint4*>(lds);                       // [2][256 rows][8]
  uint4* ldsB = reinterpret_cast<uint4*>(lds + 2 * kStageA);         // [2][256][8]
  uint32_t* ldsSA = reinterpret_cast<uint32_t*>(lds + kLdsCodes);    // [2][256]
  uint32_t* ldsSB = ldsSA + 2 * kBM;                                 // [2][256]

  // global -> register staging: thread t loads 16-byte piece p of rows
  // r0 + 32 j (j < 8) of both operands, plus one scale dword of row t
  const int p = t & 7;
  const int r0 = t >> 3;
  uint4 ra[8], rb[8];
  uint32_t rsa, rsb;
  const int sra = min(t, ts.valid_m - 1);
  const int srb = min(t, ts.valid_n - 1);

  auto gload = [&](int ks) {
    const int64_t kb = ts.k_begin + (int64_t)ks * kBK;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int rowa = min(r0 + 32 * j, ts.valid_m - 1);
      const int rowb = min(r0 + 32 * j, ts.valid_n - 1);
      ra[j] = *reinterpret_cast<const uint4*>(ts.a + rowa * ts.lda + kb + 16 * p);
      rb[j] = *reinterpret_cast<const uint4*>(ts.b + rowb * ts.ldb + kb + 16 * p);
    }
    rsa = *reinterpret_cast<const uint32_t*>(ts.sa + sra * ts.ldsa + kb / 32);
    rsb = *reinterpret_cast<const uint32_t*>(ts.sb + srb * ts.ldsb + kb / 32);
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = r0 + 32 * j;
      const int slot = row * 8 + (p ^ (row & 7));
      ldsA[st * (kStageA / 16) + slot] = ra[j];
      ldsB[st * (kStageB / 16) + slot] = rb[j];
    }
    ldsSA[st * kBM + t] = rsa;
    ldsSB[st * kBN + t] = rsb;
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

  gload(0);
  sstore(0);
  __syncthreads();

  const int lrow = lane & 31;   // operand row within a 32-row block
  const int khalf = lane >> 5;  // h: which 16-byte piece of each 32-wide K half
  for (int ks = 0; ks < ts.nk; ++ks) {
    const int st = ks & 1;
    if (ks + 1 < ts.nk) gload(ks + 1);

    const uint4* A = ldsA + st * (kStageA / 16);
    const uint4* B = ldsB + st * (kStageB / 16);
    uint32_t sva[4], svb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sva[i] = ldsSA[st * kBM + wm * 128 + 32 * i + lrow] >> (8 * khalf);
      svb[i] = ldsSB[st * kBN + wn * 128 + 32 * i + lrow] >> (8 * khalf);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // 16-byte pieces of this 64-wide sub-step held by the lane (see the
      // layout note at the top): K 16h.. and K 32+16h..
      const int p0 = (4 * s + khalf) ^ (lrow & 7);
      const int p1 = (4 * s + 2 + khalf) ^ (lrow & 7);
      v8i av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra_ = wm * 128 + 32 * i + lrow;
        av[i] = cat8(A[ra_ * 8 + p0], A[ra_ * 8 + p1]);
        const int rb_ = wn * 128 + 32 * i + lrow;
        bv[i] = cat8(B[rb_ * 8 + p0], B[rb_ * 8 + p1]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = s == 0 ? mfma_mx<0>(av[i], bv[j], acc[i][j], sva[i], svb[j])
                             : mfma_mx<2>(av[i], bv[j], acc[i][j], sva[i], svb[j]);
    }
    if (ks + 1 < ts.nk) sstore(st ^ 1);
    __syncthreads();
  }
  store_tile(acc, ts);
}

// ---------------------------------------------------------------- groups

// Group table in LDS: cleaned exclusive ends of the E groups. Offsets are
// clamped into [0, cap], rounded down to a multiple of 128 and made
// non-decreasing; any change means the caller's offsets were invalid and
// bit 0 of *dev_err is raised (by workgroup 0 only). Returns via LDS.
__device__ void load_group_ends(const int32_t* offs, int E, int64_t cap, int32_t* ends,
                                int32_t* dev_err, bool reporter) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int32_t carry = 0;       // running max of cleaned ends
    int32_t prev_raw = 0;
    bool bad = false;
    for (int g0 = 0; g0 < E; g0 += 64) {
      const int g = g0 + lane;
      int32_t raw = g < E ? offs[g] : INT32_MAX;
      int32_t c = (int32_t)min<int64_t>(max(raw, 0), cap) & ~127;
      bad |= g < E && c != raw;
      int32_t prev = __shfl_up(raw, 1);
      if (lane == 0) prev = prev_raw;
      bad |= g < E && raw < prev;
      // inclusive running max
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        int32_t o = __shfl_up(c, d);
        if (lane >= d) c = max(c, o);
      }
      c = max(c, carry);
      if (g < E) ends[g] = c;
      carry = __shfl(c, 63);
      prev_raw = __shfl(raw, 63);
    }
    const bool any_bad = __any(bad);
    if (reporter && lane == 0 && any_bad && dev_err) atomicOr(dev_err, 1);
  }
  __syncthreads();
}

__device__ __forceinline__ int64_t group_start(const int32_t* ends, int g) {
  return g == 0 ? 0 : ends[g - 1];
}

// ---------------------------------------------------------------- kernels

__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_dense(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int64_t n0 = (int64_t)blockIdx.x * kBN;
  TileSpec ts;
  ts.a = a.qa + m0 * a.lda;
  ts.sa = a.sa + m0 * a.ldsa;
  ts.b = a.qb + n0 * a.ldb;
  ts.sb = a.sb + n0 * a.ldsb;
  ts.lda = a.lda;
  ts.ldb = a.ldb;
  ts.ldsa = a.ldsa;
  ts.ldsb = a.ldsb;
  ts.valid_m = (int)min<int64_t>(kBM, a.M - m0);
  ts.valid_n = (int)min<int64_t>(kBN, a.N - n0);
  ts.k_begin = 0;
  ts.nk = (int)(a.K / kBK);
  const int esz = a.out_f32 ? 4 : 2;
  ts.out = reinterpret_cast<uint8_t*>(a.out) + (m0 * a.ldo + n0) * esz;
  ts.ldo = a.ldo;
  ts.out_f32 = a.out_f32;
  gemm_tile(ts, lds);
}

// blockIdx.y enumerates 256-row tiles of the groups in order (a group of r
// rows has ceil(r / 256) tiles; the last may hold only 128 rows), followed by
// the tiles of the tail [ends[E-1], Tcap), which are written as zeros.
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_grouped(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int32_t ends[kMaxGroups + 1];
  __shared__ int32_t tile_end[kMaxGroups + 1];   // inclusive prefix of tile counts
  const bool reporter = blockIdx.x == 0 && blockIdx.y == 0;
  load_group_ends(a.offs, a.E, a.M, ends, a.dev_err, reporter);
  if (threadIdx.x < 64) {
    // tile counts of groups 0..E (E = the tail), inclusive prefix sum
    const int lane = threadIdx.x;
    int32_t carry = 0;
    for (int g0 = 0; g0 <= a.E; g0 += 64) {
      const int g = g0 + lane;
      const int32_t end = g < a.E ? ends[g] : (int32_t)a.M;
      const int32_t start = g == 0 ? 0 : ends[g - 1];
      int32_t v = g <= a.E ? (end - start + kBM - 1) / kBM : 0;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        int32_t o = __shfl_up(v, d);
        if (lane >= d) v += o;
      }
      v += carry;
      if (g <= a.E) tile_end[g] = v;
      carry = __shfl(v, 63);
    }
    if (lane == 0) ends[a.E] = (int32_t)a.M;
  }
  __syncthreads();
  const int tile = blockIdx.y;
  if (tile >= tile_end[a.E]) return;
  // first group whose tile range ends past `tile`
  int lo = 0, hi = a.E;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (tile_end[mid] > tile) hi = mid; else lo = mid + 1;
  }
  const int g = lo;
  const int first = g == 0 ? 0 : tile_end[g - 1];
  const int64_t gs = group_start(ends, g);
  const int64_t m0 = gs + (int64_t)(tile - first) * kBM;
  const int64_t n0 = (int64_t)blockIdx.x * kBN;
  TileSpec ts;
  const int gb = min(g, a.E - 1);
  ts.a = a.qa + m0 * a.lda;
  ts.sa = a.sa + m0 * a.ldsa;
  ts.b = a.qb + gb * a.b_group_stride + n0 * a.ldb;
  ts.sb = a.sb + gb * a.sb_group_stride + n0 * a.ldsb;
  ts.lda = a.lda;
  ts.ldb = a.ldb;
  ts.ldsa = a.ldsa;
  ts.ldsb = a.ldsb;
  ts.valid_m = (int)min<int64_t>(kBM, ends[g] - m0);
  ts.valid_n = (int)min<int64_t>(kBN, a.N - n0);
  ts.k_begin = 0;
  ts.nk = g < a.E ? (int)(a.K / kBK) : 0;
  const int esz = a.out_f32 ? 4 : 2;
  ts.out = reinterpret_cast<uint8_t*>(a.out) + (m0 * a.ldo + n0) * esz;
  ts.ldo = a.ldo;
  ts.out_f32 = a.out_f32;
  gemm_tile(ts, lds);
}

// blockIdx.z ranks the groups by token count (largest first, so the longest
// tiles are dispatched first); blockIdx.y / x tile dW[g] = [N, K].
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_wgrad(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int32_t ends[kMaxGroups + 1];
  __shared__ int32_t pick;
  const bool reporter = blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0;
  if (threadIdx.x == 0) pick = min((int)blockIdx.z, a.E - 1);
  load_group_ends(a.offs, a.E, a.M, ends, a.dev_err, reporter);   // ends with a barrier
  // group whose rank (descending size, ties by index) equals blockIdx.z
  for (int g = threadIdx.x; g < a.E; g += blockDim.x) {
    const int32_t sg = ends[g] - (int32_t)group_start(ends, g);
    int rank = 0;
    for (int h = 0; h < a.E; ++h) {
      const int32_t sh = ends[h] - (int32_t)group_start(ends, h);
      rank += (sh > sg) || (sh == sg && h < g);
    }
    if (rank == (int)blockIdx.z) pick = g;
  }
  __syncthreads();
  const int g = pick;
  const int64_t ts0 = group_start(ends, g);
  const int64_t n0 = (int64_t)blockIdx.y * kBM;   // rows of dW = rows of A (= N)
  const int64_t k0 = (int64_t)blockIdx.x * kBN;   // cols of dW = rows of B (= K)
  TileSpec ts;
  ts.a = a.qa + n0 * a.lda;
  ts.sa = a.sa + n0 * a.ldsa;
  ts.b = a.qb + k0 * a.ldb;
  ts.sb = a.sb + k0 * a.ldsb;
  ts.lda = a.lda;
  ts.ldb = a.ldb;
  ts.ldsa = a.ldsa;
  ts.ldsb = a.ldsb;
  ts.valid_m = (int)min<int64_t>(kBM, a.N - n0);
  ts.valid_n = (int)min<int64_t>(kBN, a.K - k0);
  ts.k_begin = ts0;
  ts.nk = (int)((ends[g] - ts0) / kBK);
  const int esz = a.out_f32 ? 4 : 2;
  ts.out = reinterpret_cast<uint8_t*>(a.out) + (g * a.out_group_stride + n0 * a.ldo + k0) * esz;
  ts.ldo = a.ldo;
  ts.out_f32 = a.out_f32;
  gemm_tile(ts, lds);
}

// ---------------------------------------------------------------- launch

static hipError_t set_lds(const void* fn) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
}

hipError_t launch_gemm_dense(const GemmArgs& a, hipStream_t s) {
  hipError_t e = set_lds((const void*)k_gemm_dense);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((a.N + kBN - 1) / kBN), (unsigned)((a.M + kBM - 1) / kBM));
  hipLaunchKernelGGL(k_gemm_dense, grid, dim3(kGemmThreads), kLdsBytes, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_grouped(const GemmArgs& a, hipStream_t s) {
  hipError_t e = set_lds((const void*)k_gemm_grouped);
  if (e != hipSuccess) return e;
  // sum over E groups + tail of ceil(rows / 256) with rows multiples of 128
  const int64_t mtiles = a.M / kBM + (a.E + 2) / 2 + 1;
  dim3 grid((unsigned)((a.N + kBN - 1) / kBN), (unsigned)mtiles);
  hipLaunchKernelGGL(k_gemm_grouped, grid, dim3(kGemmThreads), kLdsBytes, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_wgrad(const GemmArgs& a, hipStream_t s) {
  hipError_t e = set_lds((const void*)k_gemm_wgrad);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((a.K + kBN - 1) / kBN), (unsigned)((a.N + kBM - 1) / kBM), (unsigned)a.E);
  hipLaunchKernelGGL(k_gemm_wgrad, grid, dim3(kGemmThreads), kLdsBytes, s, a);
  return hipGetLastError();
}

}  // namespace mxk
