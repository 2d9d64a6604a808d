// Kernel argument blocks and launch entry points of libmxfp8.so (internal to
// the library; the public interface is include/mxfp8.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {

// Scale layouts (mx_scale_layout of the C ABI): plain [R, C/32], or k128
// [C/128, R, 4] (the 4 block scales of a 128-wide step of each row in one
// dword, rows contiguous per step).
struct QuantArgs {
  const uint16_t* x;
  int64_t rows, cols, ld;
  bool rceil, k128;
  uint8_t *q_row, *s_row, *q_col, *s_col;
  // optional row gather (one matrix only): output row r quantizes input row
  // src_row[r] of x, or zeros where src_row[r] is negative or >= src_rows
  const int32_t* src_row = nullptr;
  int64_t src_rows = 0;
};

struct SwigluFwdArgs {
  const uint16_t *a, *b;
  int64_t ld_ab, rows, hidden;
  bool rceil, k128;
  uint8_t *q_row, *s_row, *q_col, *s_col;
  uint16_t* h_out;
};

struct SwigluBwdArgs {
  const uint16_t *dh, *a, *b;
  int64_t ld_dh, ld_ab, rows, hidden;
  bool rceil, k128;
  uint8_t *q_row, *s_row, *q_col, *s_col;
  uint16_t* dab_out;
};

struct DequantArgs {
  const uint8_t *q, *s;
  int64_t rows, cols;
  bool out_f32, k128;
  void* out;
};

// C[m, n] = sum_k A[m, k] B[n, k] over MX operands (see mx_gemm.hip); the
// scales are in the k128 layout.
struct GemmArgs {
  const uint8_t *qa, *sa, *qb, *sb;
  int64_t M, N, K;          // dense: sizes; grouped: M = Tcap
  int64_t lda, ldb;         // code bytes per operand row
  int64_t srows_a, srows_b; // rows of each operand's scale matrix (one matrix per expert for B)
  int64_t b_group_stride;   // grouped fwd/dgrad: bytes between experts' B
  int64_t sb_group_stride;  // and between their scales
  int64_t out_group_stride; // wgrad: elements between experts' outputs
  void* out;
  int64_t ldo;              // output elements per row
  bool out_f32;
  const int32_t* offs;
  int32_t E;
  int32_t* dev_err;
  // grouped fwd/dgrad with the output in token order (optional): group g's
  // first sizes[g] rows go to out rows [sum(sizes[0:g]), + sizes[g]); pad
  // rows and the tail are not written. out has out_rows rows.
  const int32_t* sizes = nullptr;
  int64_t out_rows = 0;
  // grouped w13 forward with fused SwiGLU (N = 2H): h = silu(z[:, :H]) *
  // z[:, H:] quantized both ways (k128 scales), bf16 h optional
  uint8_t *hq_row = nullptr, *hs_row = nullptr, *hq_col = nullptr, *hs_col = nullptr;
  uint16_t* h_out = nullptr;
  bool rceil = true;
};

// FP8 row-scaled quantization (one scale per row; column-wise: per column
// and segment of rows). Codes are row-major [batch, rows, cols] (row-wise)
// or [batch, cols, rows] (column-wise); scales in the k128 layout.
struct Fp8Args {
  const uint16_t* x;
  int64_t batch, rows, cols, ld;
  uint8_t *q, *s;
  const int32_t* offs;   // column-wise: segment ends along rows (nullable)
  int32_t E;
  int64_t segments;      // column-wise: E + 1 with offsets, else 1
  int32_t* work;         // column-wise: [batch, segments, cols] int32 maxima
  // both directions at once (launch_fp8_dual): q, s take the row-wise codes
  uint8_t* q_col = nullptr;
  uint8_t* s_col = nullptr;
  int32_t* row_max = nullptr;   // [batch, rows], directly after work
  int32_t* dev_err = nullptr;   // bit 0: bad segment offsets (nullable)
};

struct PadArgs {
  const uint8_t* x;
  const int32_t* sizes;
  int32_t E;
  int64_t T, row_bytes, Tcap;
  int32_t multiple;
  uint8_t* x_pad;
  int32_t *offs_pad, *src_row, *dev_err;
};

struct UnpadArgs {
  const uint8_t* y_pad;
  const int32_t* src_row;
  int64_t Tcap, T, row_bytes;
  uint8_t* y;
};


// Launchers: return hipSuccess or the launch error. Shapes are validated by
// the caller (mx_abi.cpp).
hipError_t launch_quant(const QuantArgs& a, int64_t batch, hipStream_t s);
hipError_t launch_swiglu_fwd(const SwigluFwdArgs& a, hipStream_t s);
hipError_t launch_swiglu_bwd(const SwigluBwdArgs& a, hipStream_t s);
hipError_t launch_dequant(const DequantArgs& a, hipStream_t s);
hipError_t launch_gemm_dense(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_grouped(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_grouped_swiglu(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_wgrad(const GemmArgs& a, hipStream_t s);
// bf16 wgrad_with_hp: qa / qb are G [M = Tcap, N] and X [Tcap, K] bf16,
// lda / ldb their row pitches in bytes, out bf16 [E, N, K].
hipError_t launch_gemm_wgrad_hp(const GemmArgs& a, hipStream_t s);
hipError_t launch_pad(const PadArgs& a, hipStream_t s);
hipError_t launch_fp8_rowscale(const Fp8Args& a, hipStream_t s);
hipError_t launch_fp8_colscale(const Fp8Args& a, hipStream_t s);
hipError_t launch_fp8_dual(const Fp8Args& a, hipStream_t s);
// The library's own work area for the dual FP8 quantizer (int32 elements):
// fp8_scratch returns its device address on the current device, looked up
// once per device.
constexpr int64_t kFp8ScratchInts = int64_t(1) << 20;   // 4 MiB
hipError_t fp8_scratch(int32_t** ptr);
hipError_t launch_pad_map(const PadArgs& a, hipStream_t s);   // offs_pad and src_row only
hipError_t launch_unpad(const UnpadArgs& a, hipStream_t s);

}  // namespace mxk
