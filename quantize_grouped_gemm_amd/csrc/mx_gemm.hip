// MXFP8 scaled GEMMs on gfx950 block-scaled FP8 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4: E4M3 x E4M3 with one E8M0 scale per
// 32-element K block of each operand row, float32 accumulation).
//
// Every GEMM here is C[m, n] = sum_k A[m, k] B[n, k], both operands row-major
// with K contiguous, block scales in the K128 layout [K/128, rows, 4] (the
// four block scales of a row's 128-wide K step form one dword, rows
// contiguous). Three kernels share one tile routine:
//   k_gemm_dense    one matrix pair (the linear layer's fwd / dgrad / wgrad)
//   k_gemm_grouped  2-D x 3-D: row tiles of A belong to one expert group and
//                   multiply that expert's B (grouped fwd and dgrad)
//   k_gemm_wgrad    2-D x 2-D: per expert, the contraction runs over the
//                   group's own token range (grouped weight gradient); its
//                   bf16 instance is the wgrad_with_hp GEMM (see "bf16
//                   wgrad" below)
//
// Tile routine: a 256-thread workgroup computes a 256 x 256 output tile in
// K steps of 128 (four scale blocks, two MFMA K sub-steps). Waves form a
// 2 x 2 grid, each owning a 128 x 128 sub-tile = 4 x 4 MFMA blocks of
// 32 x 32 (256 float accumulators per lane, in AGPRs). Operands reach LDS
// in two stage buffers (66 KB each), with a barrier in the middle of every
// step: A's rows and the scales by direct DMA (buffer_load ... lds), issued
// after the barrier that frees their buffer, so they have a step to land;
// B's rows through registers, loaded a step before the waves write them to
// LDS (see step_full). The two buffers are separate LDS objects and the loop
// is unrolled twice, so the compiler can tell each DMA from the reads it
// overlaps. LDS rows are 128 bytes; row r's 16-byte piece p sits in
// slot p ^ f(r) with f(r) = (r & 7) ^ ((r >> 3) & 1). A ds_read_b128 serves
// 16 lanes (16 consecutive rows, one piece) per pass over the 64 banks
// (256 bytes): rows of one parity share 128-byte halves, and f takes 8
// distinct values on the 8 even and on the 8 odd rows of any aligned group
// of 16, so the pass is free of bank conflicts (and so are 8-lane groups).
//
// Tile order: workgroups are dispatched round-robin over the 8 XCDs, each
// with its own L2. Tiles are numbered in bands of a few row tiles (column
// tiles walked within a band), and the dense and grouped kernels deal chunks
// of 16 consecutive tiles to the XCDs round-robin, so the workgroups
// resident on one XCD share A and B tiles while every XCD gets a spread of
// the tile order. The weight-gradient kernel gives each XCD an equal
// contiguous share of every group instead (its groups run one after
// another). Band heights and chunk sizes are per kernel (kOrderDense ...).
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
#include "mx_tile.h"

namespace mxk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kGemmThreads = 256;
constexpr int kStageA = kBM * kBK;                       // 32 KB of A codes per stage
constexpr int kStageB = kBN * kBK;                       // 32 KB of B codes
constexpr int kStageS = (kBM + kBN) * 4;                 // scale dwords of A and B (2 KB)
constexpr int kStageBytes = kStageA + kStageB + kStageS;
// Tile order per kernel: row tiles per band, tiles per XCD chunk (dense and
// grouped) and column tiles sharing an A row tile's L2 prefetch. Chosen by
// paired runs on MI355X over band heights 1-16 and chunks 8-64: against one
// order for all (bands of 8, chunks of 32), the MoE Scout step took about
// 2.5% less time, the dense and DeepSeek-V3-like steps 0.4-1%. The weight
// gradient does best with bands of 3 or 6 rather than 4 or 5 (about 3% on
// MoE Scout, 1% on the DeepSeek-V3-like shapes, both recipes).
struct TileOrder {
  int band, chunk, a_share;
};
constexpr TileOrder kOrderDense{4, 16, 4};
constexpr TileOrder kOrderGrouped{2, 16, 8};
constexpr TileOrder kOrderWgrad{3, 0, 4};
constexpr int kMaxGroups = 1024;                         // from 64 groups on, the table lives in LDS
// vector-memory ops per wave and K step of the MXFP8 loop:
constexpr int kDmaOpsA = 10;   // A and the scales by DMA
constexpr int kBLoads = 8;     // B's rows by plain loads (see load_b_regs)
constexpr int kPfOps = 2;      // the L2 prefetch

struct TileSpec {
  const uint8_t* a;   // codes of A row 0 of the tile (K index 0)
  const uint8_t* sa;  // k128 scale dword of A row 0, K step 0
  const uint8_t* b;
  const uint8_t* sb;
  int64_t lda, ldb;
  int64_t sstep_a, sstep_b;   // scale bytes per K step (4 x scale rows)
  int64_t sbytes_a, sbytes_b; // scale bytes from sa / sb to the end of the scale matrix
  int valid_m, valid_n;  // A rows / B rows that exist in this tile (1..256)
  int64_t k_begin;       // first contraction index, multiple of 128
  int nk;                // number of 128-wide K steps (0 => C = 0)
  int pf_a0, pf_an;      // rows [pf_a0, pf_a0 + pf_an) of A and
  int pf_b0, pf_bn;      // rows [pf_b0, pf_b0 + pf_bn) of B are this tile's L2 prefetch share
  void* out;             // C(0, 0) of the tile
  int64_t ldo;
  bool out_f32;
  // B rows 128..255 of the tile sit b_hi rows further down B, and the
  // output columns of its second column half out_hi columns further right
  // (the fused SwiGLU tile: gate and up halves of one block of h)
  int64_t b_hi = 0, out_hi = 0;
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

// Epilogue: each wave stages its 128 x 128 float sub-tile through its own
// LDS area in four passes of one MFMA block row (32 rows), row pitch 136
// floats (rows 4 apart, written by the two lane halves of a ds_write_b32,
// then start 32 banks apart). It reads back 16-byte chunks: lane l takes
// row 2 m + (l >> 5), columns 4 (l & 31) .. + 3, so a store instruction
// writes two whole 128-column rows. Full tiles take a path without bounds
// checks; edge tiles check rows and columns.
constexpr int kEpiPitch = 136;
constexpr int kEpiWaveBytes = 32 * kEpiPitch * 4;   // one wave's staging area

template <bool F32>
__device__ __forceinline__ void store_chunk(uint8_t* dst, const float4& v) {
  if constexpr (F32)
    *reinterpret_cast<float4*>(dst) = v;
  else
    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

template <bool F32>
__device__ __forceinline__ void store_tile_t(const v16f (&acc)[4][4], const TileSpec& ts, float* buf) {
  constexpr int esz = F32 ? 4 : 2;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const bool full = ts.valid_m == kBM && ts.valid_n == kBN;
  const int64_t rs = ts.ldo * esz;   // bytes per output row
  const int lrow = lane >> 5, col = 4 * (lane & 31);
  uint8_t* base =
      reinterpret_cast<uint8_t*>(ts.out) + (int64_t)(wm * 128 + lrow) * rs + (wn * (128 + ts.out_hi) + col) * esz;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 16; ++k)
        buf[(8 * (k >> 2) + 4 * (lane >> 5) + (k & 3)) * kEpiPitch + 32 * j + (lane & 31)] = acc[i][j][k];
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    uint8_t* rowp = base + (int64_t)(32 * i) * rs;
    if (full) {
#pragma unroll
      for (int m = 0; m < 16; ++m)
        store_chunk<F32>(rowp + (int64_t)(2 * m) * rs,
                         *reinterpret_cast<const float4*>(&buf[(2 * m + lrow) * kEpiPitch + col]));
    } else {
      const int grow0 = wm * 128 + 32 * i + lrow, gcol = wn * 128 + col;
      for (int m = 0; m < 16; ++m) {
        if (grow0 + 2 * m >= ts.valid_m || gcol >= ts.valid_n) continue;
        const float4 v = *reinterpret_cast<const float4*>(&buf[(2 * m + lrow) * kEpiPitch + col]);
        uint8_t* dst = rowp + (int64_t)(2 * m) * rs;
        if (gcol + 4 <= ts.valid_n) {
          store_chunk<F32>(dst, v);
        } else {
          const float f[4] = {v.x, v.y, v.z, v.w};
          for (int q = 0; q < ts.valid_n - gcol; ++q) {
            if constexpr (F32)
              reinterpret_cast<float*>(dst)[q] = f[q];
            else
              reinterpret_cast<uint16_t*>(dst)[q] = (uint16_t)f32_to_bf16(f[q]);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // the reads are done before the next pass writes
    __builtin_amdgcn_wave_barrier();
  }
}

// The tile's pointers are uniform over the workgroup but may be derived from
// LDS values (group tables); reading them from lane 0 keeps buffer resources
// in scalar registers.
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int uniform_i32(int v) { return (int)__builtin_amdgcn_readfirstlane((uint32_t)v); }

// Every field of a tile is the same in all lanes of the workgroup, but the
// grouped kernels derive them from group tables in LDS, which the compiler
// treats as per-lane values: buffer resources built from them would then be
// wrapped in a loop over distinct lane values at every DMA. Reading each
// field from lane 0 keeps them in scalar registers.
__device__ __forceinline__ TileSpec uniform_spec(const TileSpec& t) {
  TileSpec u;
  u.a = (const uint8_t*)uniform_ptr(t.a);
  u.sa = (const uint8_t*)uniform_ptr(t.sa);
  u.b = (const uint8_t*)uniform_ptr(t.b);
  u.sb = (const uint8_t*)uniform_ptr(t.sb);
  u.lda = uniform_i64(t.lda);
  u.ldb = uniform_i64(t.ldb);
  u.sstep_a = uniform_i64(t.sstep_a);
  u.sstep_b = uniform_i64(t.sstep_b);
  u.sbytes_a = uniform_i64(t.sbytes_a);
  u.sbytes_b = uniform_i64(t.sbytes_b);
  u.valid_m = uniform_i32(t.valid_m);
  u.valid_n = uniform_i32(t.valid_n);
  u.k_begin = uniform_i64(t.k_begin);
  u.nk = uniform_i32(t.nk);
  u.pf_a0 = uniform_i32(t.pf_a0);
  u.pf_an = uniform_i32(t.pf_an);
  u.pf_b0 = uniform_i32(t.pf_b0);
  u.pf_bn = uniform_i32(t.pf_bn);
  u.out = uniform_ptr(t.out);
  u.ldo = uniform_i64(t.ldo);
  u.out_f32 = uniform_i32(t.out_f32) != 0;
  u.b_hi = uniform_i64(t.b_hi);
  u.out_hi = uniform_i64(t.out_hi);
  return u;
}

// Epilogue of a full tile straight from the accumulators (no LDS). Lane l's
// element (i, j, k) is row 32 i + 8 (k >> 2) + 4 h + (k & 3), column
// 32 j + (l & 31) of its wave's sub-tile (h = l >> 5). The row part of each
// store's offset is uniform (scalar offset), the lane part a vector offset.
//   fp32: one dword store per element register: lanes 0..31 and 32..63 each
//         write one whole 128-byte row segment.
//   bf16: neighbouring lanes swap one value so that an even lane holds
//         columns c, c + 1 of row r(k) and an odd lane columns c - 1, c of
//         row r(k + 1); one dword store per register pair writes four
//         64-byte row segments.
// The caller guarantees 256 x 256 valid elements and 256 rows < 2^31 bytes.
// STREAM marks the stores non-temporal: the weight gradients' dW, which no
// kernel of the step reads back, then evicts less of the operand rows that
// the workgroups running beside it share in L2 (on the routed-experts
// shapes: 15% fewer bytes fetched and 2% less time per launch).
template <bool F32, bool STREAM = false>
__device__ __forceinline__ void store_tile_direct(const v16f (&acc)[4][4], const TileSpec& ts) {
  constexpr int kAux = STREAM ? 2 : 0;   // cache policy bits: nt
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int h = lane >> 5, c = lane & 31;
  const uint32_t rs = (uint32_t)ts.ldo * (F32 ? 4u : 2u);   // row pitch in bytes
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(ts.out), (short)0, 0x7FFFFFFF, 0x00020000);
  if constexpr (F32) {
    const uint32_t voff = (uint32_t)(wm * 128 + 4 * h) * rs + (uint32_t)(wn * (128 + ts.out_hi) + c) * 4u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint32_t soff = (uint32_t)(32 * i + 8 * (k >> 2) + (k & 3)) * rs;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][k]), r, voff + 128u * j, soff, kAux);
      }
  } else {
    // selections by mask arithmetic: the registers are indexed statically
    const uint32_t om = 0u - (uint32_t)(lane & 1);   // all ones on odd lanes
    const uint32_t voff =
        (uint32_t)(wm * 128 + 4 * h + (lane & 1)) * rs + (uint32_t)(wn * (128 + ts.out_hi) + (c & ~1)) * 2u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t soff = (uint32_t)(32 * i + 8 * (q >> 1) + 2 * (q & 1)) * rs;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t u0 = __float_as_uint(acc[i][j][2 * q]), u1 = __float_as_uint(acc[i][j][2 * q + 1]);
          const uint32_t send = u1 ^ ((u0 ^ u1) & om);   // even lanes send row k + 1, odd lanes row k
          const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, true);
          const uint32_t lo = u0 ^ ((u0 ^ got) & om);
          const uint32_t hi = got ^ ((got ^ u1) & om);
          __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(__uint_as_float(lo), __uint_as_float(hi)), r,
                                                voff + 64u * j, soff, kAux);
        }
      }
  }
}

__device__ __forceinline__ bool direct_epilogue(const TileSpec& ts) {
  return ts.valid_m == kBM && ts.valid_n == kBN && ts.ldo * (ts.out_f32 ? 4 : 2) * kBM < ((int64_t)1 << 31);
}

__device__ __forceinline__ void store_tile(const v16f (&acc)[4][4], const TileSpec& ts, uint8_t* lds) {
  float* buf = reinterpret_cast<float*>(lds);
  if (ts.out_f32)
    store_tile_t<true>(acc, ts, buf);
  else
    store_tile_t<false>(acc, ts, buf);
}

// Writes zeros over a valid_m x valid_n tile (tail rows, empty groups).
__device__ __forceinline__ void zero_tile(const TileSpec& ts) {
  const int esz = ts.out_f32 ? 4 : 2;
  const int row_bytes = ts.valid_n * esz;
  uint8_t* base = reinterpret_cast<uint8_t*>(ts.out);
  const int64_t pitch = ts.ldo * esz;
  if (ts.valid_n == kBN && ((reinterpret_cast<uintptr_t>(base) | (uintptr_t)pitch) & 15) == 0) {
    // whole rows of 16-byte stores: 64 (fp32) or 32 (bf16) lanes per row
    const int lanes_per_row = row_bytes >> 4;
    const int rows_per_pass = kGemmThreads / lanes_per_row;
    const int c = threadIdx.x % lanes_per_row;
    for (int r = threadIdx.x / lanes_per_row; r < ts.valid_m; r += rows_per_pass)
      reinterpret_cast<uint4*>(base + r * pitch)[c] = make_uint4(0, 0, 0, 0);
    return;
  }
  for (int r = threadIdx.x >> 4; r < ts.valid_m; r += kGemmThreads / 16) {
    uint8_t* row = base + (int64_t)r * ts.ldo * esz;
    for (int c = (threadIdx.x & 15) * 4; c < row_bytes; c += 64)
      *reinterpret_cast<uint32_t*>(row + c) = 0u;
  }
}

// s_waitcnt immediate waiting until at most n vector-memory operations of
// this wave are outstanding and all LDS operations are done (gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
#define MX_WAIT_VM_LDS(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (0x7 << 4))

// Operands of one 64-wide K sub-step S (0 or 1) of a 128-wide K step, read
// from stage buffer `st`. The lane's two 16-byte pieces are K 16 h.. and
// K 32 + 16 h.. of the sub-step (h = lane >> 5); row r's piece p sits in slot
// p ^ f(r) (see the note at the top).
template <int S>
__device__ __forceinline__ void load_ops(const uint8_t* st, v8i (&av)[4], v8i (&bv)[4], int wm, int wn,
                                         int lane) {
  const uint4* A = reinterpret_cast<const uint4*>(st);
  const uint4* B = reinterpret_cast<const uint4*>(st + kStageA);
  const int lrow = lane & 31, h = lane >> 5;
  const int f = (lrow & 7) ^ ((lrow >> 3) & 1);   // rows differ by multiples of 32
  const int p0 = (4 * S + h) ^ f;
  const int p1 = (4 * S + 2 + h) ^ f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm * 128 + 32 * i + lrow;
    av[i] = cat8(A[ra * 8 + p0], A[ra * 8 + p1]);
    const int rb = wn * 128 + 32 * i + lrow;
    bv[i] = cat8(B[rb * 8 + p0], B[rb * 8 + p1]);
  }
}

// 4 x 4 MFMAs of sub-step S; its scales are byte 2 S of the scale dwords
// shifted right by hs = 8 h (see the layout note at the top). The dwords are
// kept as read and shifted here, so no wait for the scale reads lands in the
// middle of the phase that issues them.
template <int S>
__device__ __forceinline__ void mfmas(const v8i (&av)[4], const v8i (&bv)[4], const uint32_t (&sva)[4],
                                      const uint32_t (&svb)[4], uint32_t hs, v16f (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mfma_mx<2 * S>(av[i], bv[j], acc[i][j], sva[i] >> hs, svb[j] >> hs);
}

// Barrier between the waves of the workgroup that neither waits for nor
// orders outstanding DMA (the caller waits with s_waitcnt first); the empty
// asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct TileDma {
  __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
  uint32_t voff_a[2], voff_b[2];
  uint32_t voff_pa, voff_pb;   // prefetch: this lane's row of the tile's A / B prefetch share
  uint32_t lda, ldb, sstep_a, sstep_b;
  uint32_t k_begin;
  uint32_t brow_add;   // rows added to this wave's B rows (b_hi for the tile's second half)
  uint32_t voff_rl;    // register B loads: lane offset in a B row block
  uint32_t lds_wb[2];  // register B writes: lane offset in an 8-row block of the stage (even / odd block)
  int wu;
};

// DMA of K step ks into stage buffer `st`: each instruction writes 64 lanes x
// 16 bytes to consecutive LDS, i.e. 8 tile rows; wave w fills rows 64 w ..
// 64 w + 63 of A and of B (8 instructions each) and the scale dwords of those
// rows. Lane l (row 8 i + (l >> 3), slot l & 7) fetches piece
// (l & 7) ^ f(row) = (l & 7) ^ (l >> 3) ^ (i & 1). The per-lane offset takes
// one of two values (even / odd i); the row block and K step go in the
// scalar offset. The scales of a K step are 256 consecutive dwords per
// operand (k128 layout): wave w copies dwords 64 w .. 64 w + 63 of each, two
// 128-byte lines per instruction.
__device__ __forceinline__ void issue_step(const TileDma& d, int ks, uint8_t* st) {
  const uint32_t kb = d.k_begin + (uint32_t)ks * kBK;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t row0 = 64 * d.wu + 8 * i;
    uint8_t* rows = st + row0 * kBK;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ra, (__attribute__((address_space(3))) void*)rows, 16,
                                             d.voff_a[i & 1], row0 * d.lda + kb, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rb, (__attribute__((address_space(3))) void*)(rows + kStageA), 16,
                                             d.voff_b[i & 1], (row0 + d.brow_add) * d.ldb + kb, 0, 0);
  }
  uint8_t* sdst = st + kStageA + kStageB + 64 * d.wu * 4;
  const uint32_t lane4 = (threadIdx.x & 63) * 4;
  const uint32_t kstep = kb / kBK;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rsa, (__attribute__((address_space(3))) void*)sdst, 4, lane4,
                                           kstep * d.sstep_a + 256 * d.wu, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rsb, (__attribute__((address_space(3))) void*)(sdst + kBM * 4), 4,
                                           lane4, kstep * d.sstep_b + 4 * (64 * d.wu + d.brow_add), 0, 0);
}

// The same without the B rows (they come through registers): A's 8
// instructions and the scale dwords.
__device__ __forceinline__ void issue_step_a(const TileDma& d, int ks, uint8_t* st) {
  const uint32_t kb = d.k_begin + (uint32_t)ks * kBK;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t row0 = 64 * d.wu + 8 * i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ra, (__attribute__((address_space(3))) void*)(st + row0 * kBK), 16,
                                             d.voff_a[i & 1], row0 * d.lda + kb, 0, 0);
  }
  uint8_t* sdst = st + kStageA + kStageB + 64 * d.wu * 4;
  const uint32_t lane4 = (threadIdx.x & 63) * 4;
  const uint32_t kstep = kb / kBK;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rsa, (__attribute__((address_space(3))) void*)sdst, 4, lane4,
                                           kstep * d.sstep_a + 256 * d.wu, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rsb, (__attribute__((address_space(3))) void*)(sdst + kBM * 4), 4,
                                           lane4, kstep * d.sstep_b + 4 * (64 * d.wu + d.brow_add), 0, 0);
}

// B rows of K step ks through registers. A stage can be refilled only after
// the barrier that frees it, and its DMA must have landed by the next
// barrier; the DMA path takes about 24 clocks per instruction, so with both
// operands on it a step's 64 instructions per CU filled most of that window.
// Plain 16-byte loads into registers need no free stage: B's rows are loaded
// a whole step before they are written to LDS (see step_full), and only A's
// rows and the scales stay on the DMA. Lane l loads piece l & 7 of row
// l >> 3 of each of the wave's 8-row blocks (8 lanes read one row's 128
// bytes) and writes it to slot (l & 7) ^ f(row) = (l & 7) ^ (l >> 3) ^ (i & 1),
// the layout the DMA produces.
struct RegB {
  uint4 v[8];
};

__device__ __forceinline__ void load_b_regs(const TileDma& d, int ks, RegB& b) {
  const uint32_t kb = d.k_begin + (uint32_t)ks * kBK;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t row0 = 64 * d.wu + 8 * i;
    b.v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(d.rb, d.voff_rl,
                                                                             (row0 + d.brow_add) * d.ldb + kb, 0));
  }
}

__device__ __forceinline__ void store_b_regs(const TileDma& d, const RegB& b, uint8_t* st) {
  uint8_t* B = st + kStageA;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint4*>(B + (64 * d.wu + 8 * i) * kBK + d.lds_wb[i & 1]) = b.v[i];
}

// L2 prefetch of K step ks: one 4-byte load per lane per operand touches
// the 128-byte line that holds a row's K chunk of the step, so that the
// step's DMA, issued two steps later, finds its lines in L2. Workgroups that
// run at the same time on one XCD share A and B tiles (see band_order); each
// prefetches only its share of the rows, so a line is fetched about once per
// XCD and the texture path (about 2 clocks per line touched) stays free for
// the DMA. The loads go to a scratch LDS area that is never read: they need
// no register and are not removed as dead.
__device__ __forceinline__ void prefetch_step(const TileDma& d, int ks, uint8_t* sink) {
  const uint32_t kb = d.k_begin + (uint32_t)ks * kBK;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ra, (__attribute__((address_space(3))) void*)sink, 4, d.voff_pa, kb, 0,
                                           0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rb, (__attribute__((address_space(3))) void*)sink, 4, d.voff_pb, kb, 0,
                                           0);
}

// Scale dwords of the lane's A and B row blocks in stage buffer `st`: byte
// 2 S + h of each serves sub-step S (mfmas shifts by 8 h).
__device__ __forceinline__ void load_scales(const uint8_t* st, uint32_t (&sva)[4], uint32_t (&svb)[4], int wm,
                                            int wn, int lane) {
  const uint32_t* SA = reinterpret_cast<const uint32_t*>(st + kStageA + kStageB);
  const uint32_t* SB = SA + kBM;
  const int lrow = lane & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sva[i] = SA[wm * 128 + 32 * i + lrow];
    svb[i] = SB[wn * 128 + 32 * i + lrow];
  }
}

struct Regs {
  v8i a0[4], b0[4], a1[4], b1[4];   // operands of sub-steps 0 and 1
  uint32_t sva[4], svb[4];          // scales of the step being multiplied
  uint32_t nsa[4], nsb[4];          // scales of the next step
};

// Interleaving hints: within the next scheduling region, follow each of the
// 16 MFMAs with `ds` LDS reads and `vm` vector-memory instructions.
template <int DS, int VM>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (DS > 0) __builtin_amdgcn_sched_group_barrier(0x100, DS, 0);
    if constexpr (VM > 0) __builtin_amdgcn_sched_group_barrier(0x010, VM, 0);
  }
}

// Interleaving of the first half with register B: each of the 16 MFMAs is
// followed by one LDS read, and by one LDS write (the first 8) or one load
// (the last 8).
__device__ __forceinline__ void interleave_rw() {
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (t < 8)
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    else
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
  }
}

// One K step ks held in stage buffer `cur`; sub-step 0's operands and the
// step's scales are in registers, step ks+1's B rows are in `rb`, and its A
// rows and scales are in flight to `nxt` (that DMA is followed by exactly
// two prefetch loads).
//   1. sub-step 0's MFMAs run while sub-step 1's operands are read from
//      `cur`, step ks+1's B rows are written from `rb` to `nxt` (no wave
//      reads `nxt` before the barrier below, and its DMA fills other rows),
//      and then step ks+2's B rows are loaded into `rb`, a step ahead of
//      their LDS writes;
//   2. wait until this wave's DMA of step ks+1 has landed (only the B loads
//      just issued and the last prefetch may be outstanding) and its LDS
//      accesses are done, then barrier: `cur` is free and `nxt` is complete
//      for all waves;
//   3. the DMA of step ks+2's A rows and scales into `cur` (the last step,
//      once past the end: it is never read) and the L2 prefetch of step ks+3
//      are issued while sub-step 1's MFMAs run and step ks+1's sub-step 0
//      operands and scales are read from `nxt`. The DMA goes out one
//      instruction per MFMA: issued in a burst, the four waves' DMA fills
//      the texture path's queue and the next MFMA waits behind a stalled
//      load.
// The MFMA unit thus sees no gap for LDS latency or DMA issue; only the
// barrier itself lies between the two halves. The last step runs the same
// code: its writes and DMA fill a free buffer and its reads of `nxt` go
// unused, which keeps a single register assignment for the accumulators.
__device__ __forceinline__ void step_full(const TileDma& d, int ks, int nk, uint8_t* cur, uint8_t* nxt, Regs& r,
                                          v16f (&acc)[4][4], int wm, int wn, int lane, uint8_t* sink, RegB& rb) {
  __builtin_amdgcn_sched_barrier(0);
  mfmas<0>(r.a0, r.b0, r.sva, r.svb, 8 * (lane >> 5), acc);
  load_ops<1>(cur, r.a1, r.b1, wm, wn, lane);
  store_b_regs(d, rb, nxt);
  load_b_regs(d, ks + 2 < nk ? ks + 2 : nk - 1, rb);
  interleave_rw();
  __builtin_amdgcn_sched_barrier(0);
  MX_WAIT_VM_LDS(kPfOps + kBLoads);
  wg_barrier();
  __builtin_amdgcn_sched_barrier(0);
  issue_step_a(d, ks + 2 < nk ? ks + 2 : nk - 1, cur);
  prefetch_step(d, ks + 3 < nk ? ks + 3 : nk - 1, sink);
  mfmas<1>(r.a1, r.b1, r.sva, r.svb, 8 * (lane >> 5), acc);
  load_ops<0>(nxt, r.a0, r.b0, wm, wn, lane);
  load_scales(nxt, r.nsa, r.nsb, wm, wn, lane);
  interleave<2, 1>();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.sva[i] = r.nsa[i];
    r.svb[i] = r.nsb[i];
  }
}

// LDS writes of this wave are done, then a workgroup barrier (without the
// wait for outstanding global stores that a full __syncthreads implies).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  wg_barrier();
}

// Outputs of the fused SwiGLU epilogue (the w13 forward of the grouped MLP).
struct SwigluOut {
  uint8_t *q_row, *s_row, *q_col, *s_col;   // h quantized both ways, k128 scales
  uint16_t* h;                              // bf16 h, or null
  int64_t rows, hidden;                     // h is [rows, hidden]
  bool rceil;
};

// Fused SwiGLU + dual MX quantization of one tile of the w13 forward. The
// tile's first 128 columns are the gate a = z[:, c0 .. c0 + 127] and its last
// 128 the matching up columns b = z[:, H + c0 ..] (z itself is stored by the
// caller). Every h element is formed exactly as the standalone SwiGLU kernel
// forms it: from the bf16-rounded a and b, in float32, rounded to bf16; and
// it is quantized by the same tile routines, so the codes are the same bytes.
//   1. The up waves (wn = 1) pass their bf16 values to the gate waves of the
//      same rows through LDS, in register order (both hold the MFMA layout).
//   2. The gate waves form h and write it to LDS as a [256][128] bf16 tile;
//      neighbouring lanes swap one value so each write is a whole dword.
//   3. All 256 threads quantize the two 128 x 128 halves of that tile.
// Rows past valid_m belong to the next group and are left alone.
__device__ __forceinline__ void swiglu_epilogue(const v16f (&acc)[4][4], const SwigluOut& o, int valid_m,
                                                int64_t r0, int64_t c0, uint8_t* lds_x, uint8_t* lds_y) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  uint32_t* X = reinterpret_cast<uint32_t*>(lds_x);   // [2][128 pairs][64 lanes] bf16 pairs of b
  uint32_t* Y = reinterpret_cast<uint32_t*>(lds_y);   // [256][64] dwords: h rows of 128 bf16
  lds_barrier();   // every wave is done with the stage buffers
  if (wn == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          X[(wm * 128 + (i * 4 + j) * 8 + q) * 64 + lane] = pack_bf16x2(acc[i][j][2 * q], acc[i][j][2 * q + 1]);
      }
  }
  lds_barrier();
  if (wn == 0) {
    const uint32_t om = 0u - (uint32_t)(lane & 1);   // all ones on odd lanes
    const int h = lane >> 5, c = lane & 31;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t bp = X[(wm * 128 + (i * 4 + j) * 8 + q) * 64 + lane];
          const uint32_t ap = pack_bf16x2(acc[i][j][2 * q], acc[i][j][2 * q + 1]);
          const uint32_t h0 = f32_to_bf16(swiglu_f32(bf16_lo(ap), bf16_lo(bp)));   // row k = 2q
          const uint32_t h1 = f32_to_bf16(swiglu_f32(bf16_hi(ap), bf16_hi(bp)));   // row k + 1
          // even lanes: columns c, c + 1 of row k; odd lanes: c - 1, c of row k + 1
          const uint32_t send = h1 ^ ((h0 ^ h1) & om);
          const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, true) & 0xFFFFu;
          const uint32_t lo = h0 ^ ((h0 ^ got) & om);
          const uint32_t hi = got ^ ((got ^ h1) & om);
          const int row = wm * 128 + 32 * i + 8 * (q >> 1) + 4 * h + 2 * (q & 1) + (lane & 1);
          Y[row * 64 + ((32 * j + c) >> 1)] = lo | (hi << 16);
        }
  }
  lds_barrier();
  uint4* Q = reinterpret_cast<uint4*>(lds_x);   // the quantizer's LDS tile; b is no longer needed
  const int t = threadIdx.x, cc = t & 15;
  for (int s = 0; s < 2; ++s) {
    const int rv = min(kTR, valid_m - kTR * s);
    if (rv <= 0) break;
    uint4 v[kTileChunks];
#pragma unroll
    for (int jj = 0; jj < kTileChunks; ++jj) {
      const int row = (t >> 4) + 16 * jj;
      v[jj] = *reinterpret_cast<const uint4*>(&Y[(kTR * s + row) * 64 + 4 * cc]);
    }
    const int64_t rs0 = r0 + kTR * s;
    if (o.h) {
#pragma unroll
      for (int jj = 0; jj < kTileChunks; ++jj) {
        const int row = (t >> 4) + 16 * jj;
        if (row < rv) *reinterpret_cast<uint4*>(o.h + (rs0 + row) * o.hidden + c0 + 8 * cc) = v[jj];
      }
    }
    if (o.q_row) tile_rowq(v, rv, kTC, o.rceil, TileOut{o.q_row, o.s_row, o.hidden, o.rows, true}, rs0, c0);
    if (o.q_col) {
      tile_to_lds(v, Q);
      lds_barrier();
      tile_colq(Q, rv, kTC, o.rceil, TileOut{o.q_col, o.s_col, o.rows, o.hidden, true}, rs0, c0);
      lds_barrier();   // before the next half overwrites Q
    }
  }
}

// Stores a finished tile (and, FUSED, runs the SwiGLU epilogue on it).
template <bool FUSED, bool STREAM = false>
__device__ __forceinline__ void finish_tile(const v16f (&acc)[4][4], const TileSpec& ts, uint8_t* st0, uint8_t* st1,
                                            const SwigluOut* so, int64_t h_r0, int64_t h_c0) {
  const int w = threadIdx.x >> 6;
  if (direct_epilogue(ts)) {
    if (ts.out_f32)
      store_tile_direct<true, STREAM>(acc, ts);
    else
      store_tile_direct<false, STREAM>(acc, ts);
  } else {
    wg_barrier();   // every wave is done with the stage buffers
    uint8_t* mine = (w & 1 ? st1 : st0) + (w >> 1) * kEpiWaveBytes;
    store_tile(acc, ts, mine);
  }
  if constexpr (FUSED) swiglu_epilogue(acc, *so, ts.valid_m, h_r0, h_c0, st1, st0);
}

// FUSED: the tile is a fused SwiGLU tile (see swiglu_epilogue); a tile
// without K steps (the tail) then still runs the epilogue, on zeros. That
// case returns on its own path, so the K loop's accumulators never merge
// with constant zeros (the merge made the register allocator spill).
// STREAM: non-temporal output stores (see store_tile_direct).
template <bool FUSED = false, bool STREAM = false>
__device__ __forceinline__ void gemm_tile(const TileSpec& tile, const SwigluOut* so = nullptr, int64_t h_r0 = 0,
                                          int64_t h_c0 = 0) {
  const TileSpec ts = uniform_spec(tile);
  __shared__ __align__(16) uint8_t st0[kStageBytes];
  __shared__ __align__(16) uint8_t st1[kStageBytes];
  __shared__ __align__(16) uint8_t sink[256];
  if (ts.nk <= 0) {
    if constexpr (FUSED) {
      v16f zero[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) zero[i][j] = v16f{};
      finish_tile<true>(zero, ts, st0, st1, so, h_r0, h_c0);
    } else {
      zero_tile(ts);
    }
    return;
  }
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;

  TileDma d;
  d.wu = __builtin_amdgcn_readfirstlane(w);
  d.brow_add = d.wu >= 2 ? (uint32_t)ts.b_hi : 0u;
  // each buffer resource ends after the last valid row: rows past it read 0
  d.ra = __builtin_amdgcn_make_buffer_rsrc((void*)ts.a, (short)0, (int)(ts.valid_m * ts.lda), 0x00020000);
  d.rb = __builtin_amdgcn_make_buffer_rsrc((void*)ts.b, (short)0, (int)((ts.valid_n + ts.b_hi) * ts.ldb),
                                           0x00020000);
  // scale rows past the valid ones hold other rows' scales (or read 0 past
  // the end of the matrix): they only meet zero operand rows, whose
  // outputs are not stored
  d.rsa = __builtin_amdgcn_make_buffer_rsrc((void*)ts.sa, (short)0, (int)ts.sbytes_a, 0x00020000);
  d.rsb = __builtin_amdgcn_make_buffer_rsrc((void*)ts.sb, (short)0, (int)ts.sbytes_b, 0x00020000);
  d.lda = (uint32_t)ts.lda;
  d.ldb = (uint32_t)ts.ldb;
  d.sstep_a = (uint32_t)ts.sstep_a;
  d.sstep_b = (uint32_t)ts.sstep_b;
  d.k_begin = (uint32_t)ts.k_begin;
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const uint32_t piece = (lane & 7) ^ (lane >> 3) ^ par;
    d.voff_a[par] = (lane >> 3) * d.lda + 16 * piece;
    d.voff_b[par] = (lane >> 3) * d.ldb + 16 * piece;
  }
  d.voff_rl = (lane >> 3) * d.ldb + 16 * (lane & 7);
#pragma unroll
  for (int par = 0; par < 2; ++par) d.lds_wb[par] = (lane >> 3) * kBK + 16 * ((lane & 7) ^ (lane >> 3) ^ par);
  // the 256 lanes of the workgroup spread over the share's rows
  const uint32_t t = threadIdx.x;
  d.voff_pa = (uint32_t)(ts.pf_a0 + ((t * (uint32_t)ts.pf_an) >> 8)) * d.lda;
  {
    const uint32_t prow = (uint32_t)(ts.pf_b0 + ((t * (uint32_t)ts.pf_bn) >> 8));
    d.voff_pb = (prow + (prow >= 128 ? (uint32_t)ts.b_hi : 0u)) * d.ldb;
  }

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

  const int nk = ts.nk;
  const int last = nk - 1;
  // prologue: steps 0 and 1 to LDS, each DMA followed by two prefetch loads
  // (steps 2 and 3; past the end, the last step stands in). The first loop
  // step prefetches step 3 again: the waits count on one prefetch pair
  // after every DMA. (Prefetching one step ahead of the DMA rather than two
  // made the grouped GEMM 3% faster on MoE Scout shapes.)
  // Step 0 comes whole by DMA; step 1's B rows are loaded into registers
  // (the first loop step writes them) and its A rows and scales by DMA.
  RegB rb;
  issue_step(d, 0, st0);
  prefetch_step(d, 2 < nk ? 2 : last, sink);
  load_b_regs(d, 1 < nk ? 1 : last, rb);
  issue_step_a(d, 1 < nk ? 1 : last, st1);
  prefetch_step(d, 3 < nk ? 3 : last, sink);
  // step 0 has landed (step 1's loads and DMA and the prefetches may not)
  MX_WAIT_VM_LDS(2 * kPfOps + kBLoads + kDmaOpsA);
  wg_barrier();
  Regs r;
  load_ops<0>(st0, r.a0, r.b0, wm, wn, lane);
  load_scales(st0, r.sva, r.svb, wm, wn, lane);
  // pairs of steps, then an odd last step: every path into a step on st0
  // has waited for st0's DMA at the barrier before
  int ks = 0;
  for (; ks + 1 < nk; ks += 2) {
    step_full(d, ks, nk, st0, st1, r, acc, wm, wn, lane, sink, rb);
    step_full(d, ks + 1, nk, st1, st0, r, acc, wm, wn, lane, sink, rb);
  }
  if (ks < nk) step_full(d, ks, nk, st0, st1, r, acc, wm, wn, lane, sink, rb);
  MX_WAIT_VM_LDS(0);
  finish_tile<FUSED, STREAM>(acc, ts, st0, st1, so, h_r0, h_c0);
}

// ---------------------------------------------------------------- bf16 wgrad
//
// The wgrad_with_hp GEMM dW[g] = G[s:e]^T X[s:e] on the unquantized bf16
// operands, whose contraction axis (tokens) is the strided one: G [Tcap, N]
// and X [Tcap, K] row-major. Same 256 x 256 tiles, waves, tile order and
// two-stage DMA as above, with v_mfma_f32_32x32x16_bf16 and K steps of 64
// tokens. A stage holds each operand as loaded: 64 token rows x 256 columns
// x 2 bytes (32 units of 16 bytes per row). The MFMA wants each lane to hold
// 8 consecutive tokens of one column. gfx950's transposing LDS read
// (ds_read_b64_tr_b16) delivers them: within each group of 16 lanes, lane j
// receives element j % 4 of the 8-byte chunks that lanes 4 e + j / 4
// (e = 0..3) address (measured on the device). Lane 4 e + q of a group thus
// addresses columns 4 q .. 4 q + 3 of the group's 16 in token row e, and
// lane j gets 4 tokens of column j; two reads give the 8. Unit u of token
// row t sits at slot u ^ (4 (t % 4)), so the 4 token rows and 4 units that a
// 32-lane pass touches cover the 64 banks once.
constexpr int kHpT = 64;                  // tokens per K step
constexpr int kHpRowB = 512;              // LDS bytes per token row (256 columns)
constexpr int kHpPart = kHpT * kHpRowB;   // 32 KB per operand and stage
static_assert(2 * kHpPart <= kStageBytes, "an hp stage fits a stage buffer");
static_assert(2 * kEpiWaveBytes <= kStageBytes, "two waves' epilogue areas fit a stage buffer");

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

struct HpDma {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t voff_a[2], voff_b[2];   // lane offsets for even / odd instructions
  uint32_t lda, ldb;               // bytes per token row of G / of X
  uint32_t t_begin;
  int wu;
};

// One 16-byte-per-lane LDS DMA (64 lanes x 16 bytes to lds_dst onwards),
// written as inline assembly: the compiler does not track it, so it inserts
// no wait for it before the transposing LDS reads (whose memory operands
// carry no alias information and would otherwise wait for every DMA in
// flight). The step loop orders DMA and reads itself: explicit s_waitcnt
// vmcnt before each workgroup barrier. The statement sets M0, so it names M0
// as clobbered and the compiler keeps no value of its own there across it.
__device__ __forceinline__ void dma16(const __amdgpu_buffer_rsrc_t& r, const uint8_t* lds_dst, uint32_t voff,
                                      uint32_t soff) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(const_cast<uint8_t*>(lds_dst));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(m0), "v"(voff), "s"(r),
               "s"(soff)
               : "m0");
}

// DMA of K step ks (64 tokens) of both operands into stage `st` (G part,
// then X part). Instruction i of wave w covers token rows 16 w + 2 i and
// 16 w + 2 i + 1; lane l writes slot l & 31 of row + (l >> 5), i.e. global
// unit (l & 31) ^ (4 ((2 i + (l >> 5)) % 4)).
__device__ __forceinline__ void issue_hp(const HpDma& d, int ks, uint8_t* st) {
  const uint32_t t0 = d.t_begin + (uint32_t)ks * kHpT;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t row = 16 * d.wu + 2 * i;
    dma16(d.ra, st + row * kHpRowB, d.voff_a[i & 1], (t0 + row) * d.lda);
    dma16(d.rb, st + kHpPart + row * kHpRowB, d.voff_b[i & 1], (t0 + row) * d.ldb);
  }
}

__device__ __forceinline__ v4s tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(const_cast<uint8_t*>(p)));
}

// MFMA operands of 16-token sub-step S (0..3) of a part for the wave's 128
// columns (half `whalf` of the 256): block i = columns 32 i .. 32 i + 31.
template <int S>
__device__ __forceinline__ void read_hp(const uint8_t* part, v8bf (&o)[4], int whalf, int lane) {
  const int g = lane >> 4, j = lane & 15, e = j >> 2;
  const int trow = 16 * S + 8 * (g >> 1) + e;   // t % 4 == e
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = 16 * whalf + 4 * i + 2 * (g & 1) + ((j & 3) >> 1);
    const uint8_t* p = part + trow * kHpRowB + ((u ^ (4 * e)) << 4) + 8 * (j & 1);
    const v4s lo = tr16(p), hi = tr16(p + 4 * kHpRowB);
    o[i] = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

template <int S>
__device__ __forceinline__ void mfmas_hp(const v8bf (&a)[4], const v8bf (&b)[4], v16f (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

struct HpRegs {
  v8bf a[4][4], b[4][4];   // [sub-step][block]
};

// One K step ks from stage `cur` (sub-steps 0, 1 already in registers);
// `nxt` receives step ks+1's DMA after the barrier at the start of the step.
// Phase A: sub-steps 0, 1 multiply while 2, 3 are read from `cur`; barrier;
// phase B: sub-steps 2, 3 multiply while step ks+1's 0, 1 are read from
// `nxt`. Mirrors step_full of the MXFP8 tile.
__device__ __forceinline__ void step_hp(const HpDma& d, int ks, int nk, uint8_t* cur, uint8_t* nxt, HpRegs& r,
                                        v16f (&acc)[4][4], int wm, int wn, int lane) {
  __builtin_amdgcn_sched_barrier(0);
  mfmas_hp<0>(r.a[0], r.b[0], acc);
  mfmas_hp<1>(r.a[1], r.b[1], acc);
  read_hp<2>(cur, r.a[2], wm, lane);
  read_hp<2>(cur + kHpPart, r.b[2], wn, lane);
  read_hp<3>(cur, r.a[3], wm, lane);
  read_hp<3>(cur + kHpPart, r.b[3], wn, lane);
  __builtin_amdgcn_sched_barrier(0);
  MX_WAIT_VM_LDS(0);   // step ks+1 has landed (this wave) and the reads are done
  wg_barrier();
  __builtin_amdgcn_sched_barrier(0);
  issue_hp(d, ks + 2 < nk ? ks + 2 : nk - 1, cur);
  mfmas_hp<2>(r.a[2], r.b[2], acc);
  mfmas_hp<3>(r.a[3], r.b[3], acc);
  read_hp<0>(nxt, r.a[0], wm, lane);
  read_hp<0>(nxt + kHpPart, r.b[0], wn, lane);
  read_hp<1>(nxt, r.a[1], wm, lane);
  read_hp<1>(nxt + kHpPart, r.b[1], wn, lane);
  __builtin_amdgcn_sched_barrier(0);
}

// ts.a / ts.b: column n0 of G / k0 of X (token row 0); ts.lda / ts.ldb: bytes
// per token row; ts.sbytes_a / sbytes_b: bytes from ts.a / ts.b to the end
// of the operand; ts.k_begin: first token; ts.nk: 64-token steps (even).
__device__ __forceinline__ void gemm_tile_hp(const TileSpec& tile) {
  const TileSpec ts = uniform_spec(tile);
  __shared__ __align__(16) uint8_t hs0[kStageBytes];
  __shared__ __align__(16) uint8_t hs1[kStageBytes];
  if (ts.nk <= 0) {
    zero_tile(ts);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  HpDma d;
  d.wu = __builtin_amdgcn_readfirstlane(w);
  // columns past N (K) read other rows' values or 0 past the end: they only
  // reach dW rows (columns) that are not stored
  d.ra = __builtin_amdgcn_make_buffer_rsrc((void*)ts.a, (short)0, (int)ts.sbytes_a, 0x00020000);
  d.rb = __builtin_amdgcn_make_buffer_rsrc((void*)ts.b, (short)0, (int)ts.sbytes_b, 0x00020000);
  d.lda = (uint32_t)ts.lda;
  d.ldb = (uint32_t)ts.ldb;
  d.t_begin = (uint32_t)ts.k_begin;
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const uint32_t unit = (lane & 31) ^ (4 * ((2 * par + (lane >> 5)) & 3));
    d.voff_a[par] = (lane >> 5) * d.lda + 16 * unit;
    d.voff_b[par] = (lane >> 5) * d.ldb + 16 * unit;
  }
  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
  const int nk = ts.nk;
  issue_hp(d, 0, hs0);
  issue_hp(d, 1 < nk ? 1 : nk - 1, hs1);
  MX_WAIT_VM_LDS(16);   // step 0 has landed
  wg_barrier();
  HpRegs r;
  read_hp<0>(hs0, r.a[0], wm, lane);
  read_hp<0>(hs0 + kHpPart, r.b[0], wn, lane);
  read_hp<1>(hs0, r.a[1], wm, lane);
  read_hp<1>(hs0 + kHpPart, r.b[1], wn, lane);
  int ks = 0;
  for (; ks + 1 < nk; ks += 2) {
    step_hp(d, ks, nk, hs0, hs1, r, acc, wm, wn, lane);
    step_hp(d, ks + 1, nk, hs1, hs0, r, acc, wm, wn, lane);
  }
  if (ks < nk) step_hp(d, ks, nk, hs0, hs1, r, acc, wm, wn, lane);
  MX_WAIT_VM_LDS(0);
  if (direct_epilogue(ts)) {   // dW: non-temporal, as in the MXFP8 weight gradient
    if (ts.out_f32)
      store_tile_direct<true, true>(acc, ts);
    else
      store_tile_direct<false, true>(acc, ts);
    return;
  }
  wg_barrier();
  uint8_t* mine = (w & 1 ? hs1 : hs0) + (w >> 1) * kEpiWaveBytes;
  store_tile(acc, ts, mine);
}

// Maps the linear index of a workgroup (dispatched round-robin over the 8
// XCDs) to a tile index so that each XCD gets a contiguous run of tiles.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int xcd = b & 7, j = b >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd * per + min(xcd, rem) + j;
}

// Deals tiles [0, total) to the 8 XCDs in chunks of CHUNK consecutive
// tiles, round-robin: chunk k is XCD (k % 8)'s (k / 8)-th chunk. Workgroup b
// (dispatched to XCD b % 8 as that XCD's (b >> 3)-th) gets its XCD's
// (b >> 3)-th tile, or -1 past the end. Used where tile costs vary across
// the tile order (grouped GEMMs: a band holding several small groups loads
// more distinct B tiles), so that no XCD's share is all slow tiles. The
// XCD's 32 CUs run two chunks at a time, so tiles running together still
// share A and B tiles in that XCD's L2.
template <int CHUNK>
__device__ __forceinline__ int xcd_chunked(int b, int total) {
  const int x = b & 7, j = b >> 3;
  const int t = ((j / CHUNK) * 8 + x) * CHUNK + j % CHUNK;
  return t < total ? t : -1;
}

// Workgroup indices the chunked deal of `total` tiles spans.
template <int CHUNK>
__host__ __device__ constexpr int64_t xcd_chunked_span(int64_t total) {
  return (total + 8 * CHUNK - 1) / (8 * CHUNK) * (8 * CHUNK);
}

// Tile index -> (row tile, column tile) in bands of BAND row tiles, column
// tiles walked within a band. `first` and `rows` return the band.
template <int BAND>
__device__ __forceinline__ void band_order(int t, int mt, int nt, int& m, int& n, int& first, int& rows) {
  const int band = t / (BAND * nt);
  first = band * BAND;
  rows = min(BAND, mt - first);
  const int r = t - band * BAND * nt;
  m = first + r % rows;
  n = r / rows;
}

// Prefetch shares. Workgroups running together on an XCD hold consecutive
// tile indices: the row tiles of one band times a few column tiles. An A
// row tile is thus shared by about ASHARE column tiles: column tile n takes
// rows (256 / ASHARE) (n % ASHARE) onwards, 256 / ASHARE of them. A B column
// tile is shared by the `cnt` row tiles of the band that use the same B
// (all of the band, or in a grouped GEMM the band's tiles of one group); the
// row tile at position `idx` among them takes the idx-th of cnt equal
// slices of its rows.
template <int ASHARE>
__device__ __forceinline__ void set_prefetch_shares(TileSpec& ts, int n, int idx, int cnt) {
  ts.pf_a0 = (kBM / ASHARE) * (n % ASHARE);
  ts.pf_an = kBM / ASHARE;
  const int part = (kBM + cnt - 1) / cnt;
  ts.pf_b0 = idx * part;
  ts.pf_bn = part;
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

// Fewer than 64 groups: every wave holds the group table in registers,
// lane g for group g and lane E for the tail. The prefix sums run on DPP
// moves instead of LDS permutes, and a tile finds its group with one
// ballot, so no LDS table and no workgroup barrier stand between a
// workgroup's start and its first DMA.
constexpr int kWaveGroups = 63;

// Inclusive prefix maximum (MAX) or sum over the wave's 64 lanes of
// non-negative values: shifts by 1, 2, 4 and 8 within each row of 16
// lanes, then row 0's last lane into row 1 and row 2's into row 3, then
// lane 31 into rows 2 and 3. A lane whose source lies outside its row, or
// that a row mask leaves out, takes 0, which changes neither a maximum nor a
// sum of non-negative values.
template <bool MAX>
__device__ __forceinline__ int32_t wave_scan(int32_t x) {
  auto step = [&](int32_t y) { x = MAX ? max(x, y) : x + y; };
  step(__builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false));   // row_shr:1
  step(__builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false));   // row_shr:2
  step(__builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false));   // row_shr:4
  step(__builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false));   // row_shr:8
  step(__builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false));   // row_bcast:15
  step(__builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false));   // row_bcast:31
  return x;
}

// The value of the lane below (0 for lane 0): DPP wave_shr:1.
__device__ __forceinline__ int32_t lane_below(int32_t x) {
  return __builtin_amdgcn_update_dpp(0, x, 0x138, 0xF, 0xF, false);
}

struct WaveGroups {
  int32_t end, start;   // lane g < E: group g's rows [start, end); lane E: the tail [ends[E-1], cap)
};

// The offsets cleaned as load_group_ends cleans them (clamped to [0, cap],
// rounded down to 128 rows, made non-decreasing), with the same report.
__device__ __forceinline__ WaveGroups wave_group_ends(const int32_t* offs, int E, int64_t cap, int32_t* dev_err,
                                                     bool reporter) {
  const int lane = threadIdx.x & 63;
  const int32_t raw = lane < E ? offs[lane] : 0;
  const int32_t c = (int32_t)min<int64_t>(max(raw, 0), cap) & ~127;
  const bool bad = lane < E && (c != raw || raw < lane_below(raw));
  const bool any_bad = __any(bad);   // every lane votes
  if (reporter && threadIdx.x == 0 && any_bad && dev_err) atomicOr(dev_err, 1);
  const int32_t run = wave_scan<true>(lane < E ? c : 0);
  WaveGroups w;
  w.end = lane < E ? run : (lane == E ? (int32_t)cap : 0);
  w.start = lane_below(w.end);
  return w;
}

// ---------------------------------------------------------------- kernels

__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_dense(GemmArgs a) {
  const int mt = (int)((a.M + kBM - 1) / kBM), nt = (int)((a.N + kBN - 1) / kBN);
  int tm, tn, bfirst, brows;
  const int t = xcd_chunked<kOrderDense.chunk>(blockIdx.x, mt * nt);
  if (t < 0) return;
  band_order<kOrderDense.band>(t, mt, nt, tm, tn, bfirst, brows);
  const int64_t m0 = (int64_t)tm * kBM;
  const int64_t n0 = (int64_t)tn * kBN;
  TileSpec ts;
  const int64_t steps = a.K / kBK;
  ts.a = a.qa + m0 * a.lda;
  ts.sa = a.sa + m0 * 4;
  ts.b = a.qb + n0 * a.ldb;
  ts.sb = a.sb + n0 * 4;
  ts.lda = a.lda;
  ts.ldb = a.ldb;
  ts.sstep_a = 4 * a.srows_a;
  ts.sstep_b = 4 * a.srows_b;
  ts.sbytes_a = steps * ts.sstep_a - m0 * 4;
  ts.sbytes_b = steps * ts.sstep_b - n0 * 4;
  ts.valid_m = (int)min<int64_t>(kBM, a.M - m0);
  ts.valid_n = (int)min<int64_t>(kBN, a.N - n0);
  ts.k_begin = 0;
  ts.nk = (int)steps;
  set_prefetch_shares<kOrderDense.a_share>(ts, tn, tm - bfirst, brows);
  const int esz = a.out_f32 ? 4 : 2;
  ts.out = reinterpret_cast<uint8_t*>(a.out) + (m0 * a.ldo + n0) * esz;
  ts.ldo = a.ldo;
  ts.out_f32 = a.out_f32;
  gemm_tile(ts);
}

// Row tiles: 256-row tiles of the groups in order (a group of r rows has
// ceil(r / 256) tiles; the last may hold only 128 rows), followed by the
// tiles of the tail [ends[E-1], Tcap), which are written as zeros. The grid
// is an upper bound on row tiles x column tiles; surplus workgroups exit.
// FUSED: the w13 forward with SwiGLU + dual quantization in the epilogue.
// Its tile t covers h columns [128 t, 128 t + 128): B rows [128 t, + 128) of
// the expert's w13 (gate) and [H + 128 t, + 128) (up); z columns likewise.
template <bool FUSED>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_grouped(GemmArgs a) {
  __shared__ int32_t ends[kMaxGroups + 1];
  __shared__ int32_t tile_end[kMaxGroups + 1];   // inclusive prefix of row-tile counts
  __shared__ int32_t tok[kMaxGroups + 1];        // token-order output: first row of each group
  const bool reporter = blockIdx.x == 0;
  const bool small = a.E <= kWaveGroups;
  // small: lane g of every wave holds group g's rows, its row tiles
  // [tstart, te) and (token order) its first output row tok; lane E the tail
  const int lane = threadIdx.x & 63;
  WaveGroups wg{};
  int32_t te = 0, tstart = 0, tokv = 0;
  int mt, mt_groups;   // row tiles: all (the tail's included), the groups'
  if (small) {
    wg = wave_group_ends(a.offs, a.E, a.M, a.dev_err, reporter);
    const int32_t count = lane <= a.E ? (wg.end - wg.start + kBM - 1) / kBM : 0;
    te = wave_scan<false>(count);
    tstart = te - count;
    mt = __builtin_amdgcn_readlane(te, a.E);
    mt_groups = __builtin_amdgcn_readlane(te, a.E - 1);
    if (a.sizes) {
      // exclusive prefix of the token counts, reported as below (bit 2)
      int32_t n = lane < a.E ? a.sizes[lane] : 0;
      const int32_t slot = wg.end - wg.start;
      const bool bad = lane < a.E && (n < 0 || n > slot);
      n = lane < a.E ? min(max(n, 0), slot) : 0;
      const int32_t incl = wave_scan<false>(n);
      tokv = incl - n;   // lane E: the total
      const bool any_bad = __any(bad) || (int64_t)__builtin_amdgcn_readlane(incl, 63) > a.out_rows;
      if (reporter && threadIdx.x == 0 && any_bad && a.dev_err) atomicOr(a.dev_err, 4);
    }
  } else {
    load_group_ends(a.offs, a.E, a.M, ends, a.dev_err, reporter);
    if (a.sizes && threadIdx.x < 64) {
      // exclusive prefix of the token counts; a count beyond its group's
      // padded slot, or a total beyond out_rows, is reported (bit 2)
      int32_t carry = 0;
      bool bad = false;
      for (int g0 = 0; g0 < a.E; g0 += 64) {
        const int g = g0 + lane;
        int32_t n = g < a.E ? a.sizes[g] : 0;
        if (g < a.E) {
          const int32_t slot = ends[g] - (int32_t)group_start(ends, g);
          bad |= n < 0 || n > slot;
          n = min(max(n, 0), slot);
        }
        int32_t v = n;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int32_t o = __shfl_up(v, d);
          if (lane >= d) v += o;
        }
        if (g < a.E) tok[g] = carry + v - n;
        carry += __shfl(v, 63);
      }
      bad |= (int64_t)carry > a.out_rows;
      const bool any_bad = __any(bad);   // every lane votes
      if (lane == 0) tok[a.E] = carry;
      if (reporter && lane == 0 && any_bad && a.dev_err) atomicOr(a.dev_err, 4);
    }
    if (threadIdx.x < 64) {
      // row-tile counts of groups 0..E (E = the tail), inclusive prefix sum
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
    mt = tile_end[a.E];
    mt_groups = tile_end[a.E - 1];
  }
  const int64_t H = a.N / 2;   // FUSED: z is [Tcap, 2H]
  const int nt = FUSED ? (int)(H / 128) : (int)((a.N + kBN - 1) / kBN);
  const int b = (int)blockIdx.x;
  // the groups' tiles are dealt to the XCDs in chunks; the tail's zero tiles
  // follow the span of that deal, so no XCD's share is padded with them
  const int span = (int)xcd_chunked_span<kOrderGrouped.chunk>((int64_t)mt_groups * nt);
  int tile, tn, bfirst, brows;
  if (b < span) {
    const int t = xcd_chunked<kOrderGrouped.chunk>(b, mt_groups * nt);
    if (t < 0) return;
    band_order<kOrderGrouped.band>(t, mt_groups, nt, tile, tn, bfirst, brows);
  } else {
    const int z = b - span;
    if (z >= (mt - mt_groups) * nt) return;
    tile = mt_groups + z / nt;
    tn = z % nt;
    bfirst = tile;
    brows = 1;
  }
  // the first group whose row-tile range ends past `tile`
  int g, first, tend;
  int64_t gs, gend;
  if (small) {
    const uint64_t hit = __ballot(lane <= a.E && te > tile);
    g = hit ? __builtin_ctzll(hit) : a.E;
    first = __builtin_amdgcn_readlane(tstart, g);
    tend = __builtin_amdgcn_readlane(te, g);
    gs = __builtin_amdgcn_readlane(wg.start, g);
    gend = __builtin_amdgcn_readlane(wg.end, g);
  } else {
    int lo = 0, hi = a.E;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (tile_end[mid] > tile) hi = mid; else lo = mid + 1;
    }
    g = lo;
    first = g == 0 ? 0 : tile_end[g - 1];
    tend = tile_end[g];
    gs = group_start(ends, g);
    gend = ends[g];
  }
  const int64_t m0 = gs + (int64_t)(tile - first) * kBM;
  const int64_t n0 = FUSED ? (int64_t)tn * 128 : (int64_t)tn * kBN;
  TileSpec ts;
  const int gb = min(g, a.E - 1);
  const int64_t steps = a.K / kBK;
  ts.a = a.qa + m0 * a.lda;
  ts.sa = a.sa + m0 * 4;
  ts.b = a.qb + gb * a.b_group_stride + n0 * a.ldb;
  ts.sb = a.sb + gb * a.sb_group_stride + n0 * 4;
  ts.lda = a.lda;
  ts.ldb = a.ldb;
  ts.sstep_a = 4 * a.srows_a;
  ts.sstep_b = 4 * a.srows_b;
  ts.sbytes_a = steps * ts.sstep_a - m0 * 4;
  ts.sbytes_b = steps * ts.sstep_b - n0 * 4;
  ts.valid_m = (int)min<int64_t>(kBM, gend - m0);
  ts.valid_n = FUSED ? kBN : (int)min<int64_t>(kBN, a.N - n0);
  ts.k_begin = 0;
  ts.nk = g < a.E ? (int)(a.K / kBK) : 0;
  if constexpr (FUSED) {
    ts.b_hi = H - 128;
    ts.out_hi = H - 128;
  }
  int64_t out_row = m0;
  if (a.sizes) {
    // token order: only the group's real rows, shifted to its token range
    if (g >= a.E) return;                              // no tail rows
    const int32_t tok0 = small ? __builtin_amdgcn_readlane(tokv, g) : tok[g];
    const int32_t tok1 = small ? __builtin_amdgcn_readlane(tokv, g + 1) : tok[g + 1];
    const int64_t in_group = m0 - gs;
    const int64_t real = (int64_t)(tok1 - tok0) - in_group;
    out_row = tok0 + in_group;
    const int64_t room = a.out_rows - out_row;
    const int64_t rows = min<int64_t>(min<int64_t>(real, room), ts.valid_m);
    if (rows <= 0) return;
    ts.valid_m = (int)rows;
  }
  {
    // the band's row tiles that belong to group g share its B tiles
    const int lo = max(bfirst, first), hi = min(bfirst + brows, tend);
    set_prefetch_shares<kOrderGrouped.a_share>(ts, tn, tile - lo, hi - lo);
  }
  const int esz = a.out_f32 ? 4 : 2;
  ts.out = reinterpret_cast<uint8_t*>(a.out) + (out_row * a.ldo + n0) * esz;
  ts.ldo = a.ldo;
  ts.out_f32 = a.out_f32;
  if constexpr (FUSED) {
    const SwigluOut so{a.hq_row, a.hs_row, a.hq_col, a.hs_col, a.h_out, a.M, H, a.rceil};
    gemm_tile<true>(ts, &so, m0, n0);
  } else {
    gemm_tile(ts);
  }
}

// The grid covers E x (N tiles) x (K tiles) of dW. Tile indices run over the
// groups ranked by token count, largest first (the longest tiles start
// first); within a group's [N, K] rectangle tiles follow the band order.
// HP: the bf16 wgrad_with_hp operands (G, X as [Tcap, N], [Tcap, K]); else
// the MXFP8 column-wise operands ([N, Tcap], [K, Tcap] codes).
template <bool HP>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_wgrad(GemmArgs a) {
  __shared__ int32_t ends[kMaxGroups + 1];
  __shared__ int32_t pick;
  const int nt_n = (int)((a.N + kBM - 1) / kBM);
  const int nt_k = (int)((a.K + kBN - 1) / kBN);
  const int per = nt_n * nt_k;
  const int want = min((int)blockIdx.x / per, a.E - 1);   // group rank
  const int u = xcd_remap((int)blockIdx.x - ((int)blockIdx.x / per) * per, per);
  // the group whose rank (descending size, ties by index) equals `want`
  int g;
  int64_t ts0, gend;
  if (a.E <= kWaveGroups) {
    const int lane = threadIdx.x & 63;
    const WaveGroups wg = wave_group_ends(a.offs, a.E, a.M, a.dev_err, blockIdx.x == 0);
    const int32_t size = wg.end - wg.start;
    int rank = 0;
    for (int h = 0; h < a.E; ++h) {
      const int32_t sh = __builtin_amdgcn_readlane(size, h);
      rank += (sh > size) || (sh == size && h < lane);
    }
    const uint64_t hit = __ballot(lane < a.E && rank == want);
    g = hit ? __builtin_ctzll(hit) : want;
    ts0 = __builtin_amdgcn_readlane(wg.start, g);
    gend = __builtin_amdgcn_readlane(wg.end, g);
  } else {
    if (threadIdx.x == 0) pick = want;
    load_group_ends(a.offs, a.E, a.M, ends, a.dev_err, blockIdx.x == 0);   // ends with a barrier
    for (int gg = threadIdx.x; gg < a.E; gg += blockDim.x) {
      const int32_t sg = ends[gg] - (int32_t)group_start(ends, gg);
      int rank = 0;
      for (int h = 0; h < a.E; ++h) {
        const int32_t sh = ends[h] - (int32_t)group_start(ends, h);
        rank += (sh > sg) || (sh == sg && h < gg);
      }
      if (rank == want) pick = gg;
    }
    __syncthreads();
    g = pick;
    ts0 = group_start(ends, g);
    gend = ends[g];
  }
  int tn, tk, bfirst, brows;
  band_order<kOrderWgrad.band>(u, nt_n, nt_k, tn, tk, bfirst, brows);
  const int64_t n0 = (int64_t)tn * kBM;   // rows of dW = rows of A (= N)
  const int64_t k0 = (int64_t)tk * kBN;   // cols of dW = rows of B (= K)
  TileSpec ts;
  const int64_t steps = a.M / kBK;   // 128-token steps of Tcap
  if constexpr (HP) {
    ts.a = a.qa + n0 * 2;
    ts.b = a.qb + k0 * 2;
    ts.sbytes_a = a.M * a.lda - n0 * 2;
    ts.sbytes_b = a.M * a.ldb - k0 * 2;
  } else {
    ts.a = a.qa + n0 * a.lda;
    ts.sa = a.sa + n0 * 4;
    ts.b = a.qb + k0 * a.ldb;
    ts.sb = a.sb + k0 * 4;
    ts.sstep_a = 4 * a.srows_a;
    ts.sstep_b = 4 * a.srows_b;
    ts.sbytes_a = steps * ts.sstep_a - n0 * 4;
    ts.sbytes_b = steps * ts.sstep_b - k0 * 4;
  }
  ts.lda = a.lda;
  ts.ldb = a.ldb;
  ts.valid_m = (int)min<int64_t>(kBM, a.N - n0);
  ts.valid_n = (int)min<int64_t>(kBN, a.K - k0);
  ts.k_begin = ts0;
  ts.nk = (int)((gend - ts0) / (HP ? kHpT : kBK));
  set_prefetch_shares<kOrderWgrad.a_share>(ts, tk, tn - bfirst, brows);
  const int esz = a.out_f32 ? 4 : 2;
  ts.out = reinterpret_cast<uint8_t*>(a.out) + (g * a.out_group_stride + n0 * a.ldo + k0) * esz;
  ts.ldo = a.ldo;
  ts.out_f32 = a.out_f32;
  if constexpr (HP)
    gemm_tile_hp(ts);
  else
    gemm_tile<false, true>(ts);
}

// ---------------------------------------------------------------- launch


hipError_t launch_gemm_dense(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles = xcd_chunked_span<kOrderDense.chunk>(((a.N + kBN - 1) / kBN) * ((a.M + kBM - 1) / kBM));
  hipLaunchKernelGGL(k_gemm_dense, dim3((unsigned)tiles), dim3(kGemmThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_grouped(const GemmArgs& a, hipStream_t s) {
  // sum over E groups + tail of ceil(rows / 256) with rows multiples of 128
  const int64_t mtiles = a.M / kBM + (a.E + 2) / 2 + 1;
  // the chunked deal of the groups' tiles spans at most 8 * chunk - 1
  // indices more than the tiles themselves
  const int64_t tiles = mtiles * ((a.N + kBN - 1) / kBN) + 8 * kOrderGrouped.chunk;
  hipLaunchKernelGGL(k_gemm_grouped<false>, dim3((unsigned)tiles), dim3(kGemmThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_grouped_swiglu(const GemmArgs& a, hipStream_t s) {
  const int64_t mtiles = a.M / kBM + (a.E + 2) / 2 + 1;
  const int64_t tiles = mtiles * (a.N / 2 / 128) + 8 * kOrderGrouped.chunk;
  hipLaunchKernelGGL(k_gemm_grouped<true>, dim3((unsigned)tiles), dim3(kGemmThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_wgrad(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles = ((a.K + kBN - 1) / kBN) * ((a.N + kBM - 1) / kBM) * a.E;
  hipLaunchKernelGGL(k_gemm_wgrad<false>, dim3((unsigned)tiles), dim3(kGemmThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_wgrad_hp(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles = ((a.K + kBN - 1) / kBN) * ((a.N + kBM - 1) / kBM) * a.E;
  hipLaunchKernelGGL(k_gemm_wgrad<true>, dim3((unsigned)tiles), dim3(kGemmThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mxk
