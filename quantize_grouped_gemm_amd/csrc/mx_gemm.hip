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

// Epilogue: each wave stages its 128 x 128 float sub-tile through LDS in two
// halves of 64 rows (32 KB per wave per half) and writes whole 16-byte
// chunks of output rows; only a chunk that crosses valid_n falls back to
// element stores. The K loop's last barrier has released the LDS.
__device__ __forceinline__ void store_tile(const v16f (&acc)[4][4], const TileSpec& ts, uint8_t* lds) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  float* buf = reinterpret_cast<float*>(lds) + w * (64 * 132);   // [64][128 + 4 pad]
  const int esz = ts.out_f32 ? 4 : 2;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * half + ii;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int r = 32 * ii + 8 * (k >> 2) + 4 * (lane >> 5) + (k & 3);
          buf[r * 132 + 32 * j + (lane & 31)] = acc[i][j][k];
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    // 64 rows x 128 columns; a lane handles 4 consecutive columns per step
    const int row0 = wm * 128 + 64 * half;
    const int col0 = wn * 128;
#pragma unroll 4
    for (int e = lane; e < 64 * 32; e += 64) {
      const int r = e >> 5, c = (e & 31) * 4;
      const int row = row0 + r, col = col0 + c;
      if (row >= ts.valid_m || col >= ts.valid_n) continue;
      const float4 v = *reinterpret_cast<const float4*>(&buf[r * 132 + c]);
      uint8_t* dst = reinterpret_cast<uint8_t*>(ts.out) + ((int64_t)row * ts.ldo + col) * esz;
      if (col + 4 <= ts.valid_n) {
        if (ts.out_f32)
          *reinterpret_cast<float4*>(dst) = v;
        else
          *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
      } else {
        const float f[4] = {v.x, v.y, v.z, v.w};
        for (int q = 0; q < ts.valid_n - col; ++q) {
          if (ts.out_f32)
            reinterpret_cast<float*>(dst)[q] = f[q];
          else
            reinterpret_cast<uint16_t*>(dst)[q] = (uint16_t)f32_to_bf16(f[q]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
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

// Operands of one 64-wide K sub-step S (0 or 1) of a 128-wide K step. The
// lane's two 16-byte pieces are K 16 h.. and K 32 + 16 h.. of the sub-step
// (h = lane >> 5), XOR-swizzled by the row.
template <int S>
__device__ __forceinline__ void load_ops(const uint4* A, const uint4* B, v8i (&av)[4], v8i (&bv)[4],
                                         int wm, int wn, int lrow, int khalf) {
  const int p0 = (4 * S + khalf) ^ (lrow & 7);
  const int p1 = (4 * S + 2 + khalf) ^ (lrow & 7);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm * 128 + 32 * i + lrow;
    av[i] = cat8(A[ra * 8 + p0], A[ra * 8 + p1]);
    const int rb = wn * 128 + 32 * i + lrow;
    bv[i] = cat8(B[rb * 8 + p0], B[rb * 8 + p1]);
  }
}

// 4 x 4 MFMAs of sub-step S; its scales are byte 2 S of the shifted scale
// dwords (see the layout note at the top).
template <int S>
__device__ __forceinline__ void mfmas(const v8i (&av)[4], const v8i (&bv)[4], const uint32_t (&sva)[4],
                                      const uint32_t (&svb)[4], v16f (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mfma_mx<2 * S>(av[i], bv[j], acc[i][j], sva[i], svb[j]);
}

__device__ __forceinline__ void gemm_tile(const TileSpec& ts, uint8_t* lds) {
  if (ts.nk <= 0) {
    zero_tile(ts);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;

  const uint4* ldsA = reinterpret_cast<const uint4*>(lds);                  // [2][256 rows][8]
  const uint4* ldsB = reinterpret_cast<const uint4*>(lds + 2 * kStageA);    // [2][256][8]
  uint32_t* ldsSA = reinterpret_cast<uint32_t*>(lds + kLdsCodes);           // [2][256]
  uint32_t* ldsSB = ldsSA + 2 * kBM;                                        // [2][256]

  // Global -> LDS with direct DMA loads (buffer_load_dwordx4 ... lds): each
  // instruction writes 64 lanes x 16 bytes to consecutive LDS, so one
  // instruction fills 8 tile rows; wave w fills rows 64 w .. 64 w + 63 of A
  // and of B. LDS slot (row, s) must hold global piece s ^ (row & 7), so lane
  // l (row 8 i + (l >> 3), slot l & 7) fetches piece (l & 7) ^ (l >> 3).
  // The per-lane byte offset is the same for every instruction; the row
  // block and K step go in the scalar offset. Each operand's buffer resource
  // ends after its last valid row, so rows past it read as zero.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      (void*)ts.a, (short)0, (int)(ts.valid_m * ts.lda), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)ts.b, (short)0, (int)(ts.valid_n * ts.ldb), 0x00020000);
  const __amdgpu_buffer_rsrc_t rssa = __builtin_amdgcn_make_buffer_rsrc(
      (void*)ts.sa, (short)0, (int)(ts.valid_m * ts.ldsa), 0x00020000);
  const __amdgpu_buffer_rsrc_t rssb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)ts.sb, (short)0, (int)(ts.valid_n * ts.ldsb), 0x00020000);
  const uint32_t voff_a = (lane >> 3) * (uint32_t)ts.lda + 16 * ((lane & 7) ^ (lane >> 3));
  const uint32_t voff_b = (lane >> 3) * (uint32_t)ts.ldb + 16 * ((lane & 7) ^ (lane >> 3));
  const uint32_t voff_sa = lane * (uint32_t)ts.ldsa;
  const uint32_t voff_sb = lane * (uint32_t)ts.ldsb;
  auto issue = [&](int ks, int st) {
    const uint32_t kb = (uint32_t)ts.k_begin + (uint32_t)ks * kBK;
    uint8_t* la = lds + st * kStageA + (64 * wu) * kBK;
    uint8_t* lb = lds + 2 * kStageA + st * kStageB + (64 * wu) * kBK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t row0 = 64 * wu + 8 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsa, (__attribute__((address_space(3))) void*)(la + i * 1024), 16, voff_a,
          row0 * (uint32_t)ts.lda + kb, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsb, (__attribute__((address_space(3))) void*)(lb + i * 1024), 16, voff_b,
          row0 * (uint32_t)ts.ldb + kb, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rssa, (__attribute__((address_space(3))) void*)(ldsSA + st * kBM + 64 * wu), 4, voff_sa,
        64 * wu * (uint32_t)ts.ldsa + kb / 32, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rssb, (__attribute__((address_space(3))) void*)(ldsSB + st * kBN + 64 * wu), 4, voff_sb,
        64 * wu * (uint32_t)ts.ldsb + kb / 32, 0, 0);
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

  const int lrow = lane & 31;   // operand row within a 32-row block
  const int khalf = lane >> 5;  // h: which 16-byte piece of each 32-wide K half
  v8i a0[4], b0[4], a1[4], b1[4];
  uint32_t sva[4], svb[4];

  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int ks = 0; ks < ts.nk; ++ks) {
    const int st = ks & 1;
    const uint4* A = ldsA + st * (kStageA / 16);
    const uint4* B = ldsB + st * (kStageB / 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sva[i] = ldsSA[st * kBM + wm * 128 + 32 * i + lrow] >> (8 * khalf);
      svb[i] = ldsSB[st * kBN + wn * 128 + 32 * i + lrow] >> (8 * khalf);
    }
    load_ops<0>(A, B, a0, b0, wm, wn, lrow, khalf);
    load_ops<1>(A, B, a1, b1, wm, wn, lrow, khalf);
    __builtin_amdgcn_sched_barrier(0);
    mfmas<0>(a0, b0, sva, svb, acc);
    __builtin_amdgcn_sched_barrier(0);
    if (ks + 1 < ts.nk) issue(ks + 1, st ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas<1>(a1, b1, sva, svb, acc);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's DMA into the other stage
    __syncthreads();
  }
  store_tile(acc, ts, lds);
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
