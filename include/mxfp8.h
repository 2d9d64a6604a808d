/*
 * mxfp8.h -- C ABI of libmxfp8.so: the MXFP8 training hot path on MI355X
 * (gfx950), as hand-written HIP kernels.
 *
 * What is computed comes from three pages:
 *   [P1] "TrainingWeightWrapperTensor base class; subclasses for FP8/MXFP8 with
 *        grouped_mm and linear overrides" (pytorch/ao pull request 3968)
 *   [P2] "[mxfp8 training] unified MXFP8TrainingConfig and MXFP8TrainingTensor"
 *        (pytorch/ao pull request 3948)
 *   [P3] "Add MXFP8 fused-MLP overrides in torchtitan" (pytorch/torchtitan
 *        pull request 4257)
 * The pages name MXFP8 but do not define it; MXFP8 is the OCP Microscaling
 * (MX) v1.0 format: blocks of 32 contiguous values sharing one E8M0 scale
 * byte (value 2^(byte-127), 0xFF = NaN), elements in FP8 E4M3 ("E4M3FN":
 * bias 7, no infinities, 0x7F/0xFF = NaN, largest finite 448).
 *
 * Conventions shared by every call
 *  - Pointers are device pointers (hipMalloc'd or from any allocator on the
 *    current device) unless stated. The caller owns every buffer; the library
 *    never allocates or frees device memory and keeps no pointer after return.
 *  - bf16 tensors are 16-bit bfloat16; E4M3 codes and E8M0 scales are bytes.
 *    All tensors are row-major. Block j of row r of an [R, C] code tensor
 *    covers columns 32j..32j+31; its scale byte is stored in one of two
 *    layouts (mx_scale_layout):
 *      MX_SCALES_PLAIN  [R, C/32]: byte r * (C/32) + j;
 *      MX_SCALES_K128   [C/128, R, 4]: byte ((j/4) * R + r) * 4 + j%4, i.e.
 *                       for each 128-column step the four block scales of
 *                       every row form one dword, rows contiguous. Needs
 *                       C % 128 == 0. The GEMMs read this layout: a tile's
 *                       scales for one K step are one contiguous run.
 *    A batch of matrices (or E experts) stores one such tensor per matrix,
 *    R * C/32 bytes apart, in either layout.
 *  - "Row-wise" quantization blocks the contiguous (last) axis. "Column-wise"
 *    quantization of an [R, C] tensor is row-wise quantization of its
 *    transpose and is stored transposed: codes [C, R] with the scales of that
 *    [C, R] tensor.
 *  - Every GEMM is C = A * B^T with the contraction axis contiguous in both
 *    operands (A [M, K], B [N, K]), float32 accumulation.
 *  - `stream` is a hipStream_t (NULL = the null stream). Every call only
 *    enqueues work on it: no call synchronizes, and no call reads device
 *    memory on the host, so calls can be captured in a HIP graph.
 *  - Pointers to bf16 data, E4M3 codes and GEMM outputs must be 16-byte
 *    aligned; scale pointers 4-byte aligned in the MX_SCALES_K128 layout
 *    (any alignment in MX_SCALES_PLAIN); int32 arrays 4-byte aligned.
 *    Leading dimensions are given in elements and must keep every row
 *    16-byte aligned.
 *  - Errors: every argument is checked on the host before anything is
 *    enqueued. A non-zero status means nothing was enqueued; mx_last_error()
 *    then returns a message for the calling thread. There is no fallback path:
 *    if the library cannot run a call on the current device it fails.
 *  - Grouped calls take 1 <= E <= 1024 groups (MX_ERR_SHAPE otherwise) and
 *    per-group offsets in device memory (int32 [E], exclusive ends: group g
 *    owns rows [offs[g-1], offs[g]) with offs[-1] = 0).
 *    Offsets are never read on the host. Kernels check them on the device:
 *    they must be non-decreasing multiples of 128 no larger than the padded
 *    capacity Tcap. If they are not and `dev_err` is non-NULL, bit 0 of
 *    *dev_err is set (it is never cleared by the library); every access stays
 *    in bounds but the output values are then unspecified.
 */
#ifndef MXFP8_H
#define MXFP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MX_OK = 0,
  MX_ERR_NULL = 1,   /* a required pointer is NULL */
  MX_ERR_SHAPE = 2,  /* a size is negative, or not the multiple it must be */
  MX_ERR_ALIGN = 3,  /* a pointer or leading dimension breaks 16-byte alignment */
  MX_ERR_ARG = 4,    /* an enum or flag argument is out of range */
  MX_ERR_DEVICE = 5, /* no HIP device, or the current device is not gfx950 */
  MX_ERR_HIP = 6     /* the HIP runtime reported an error while enqueueing */
} mx_status;

/* Scale rounding modes. FLOOR is the OCP MX v1.0 rule:
 *   E = floor(log2(amax)) - 8   (8 = exponent of 448, the largest E4M3 value);
 * scaled elements above 448 saturate to +-448.
 * RCEIL ([P1], review thread, ScaleCalculationMode.RCEIL): the scale is
 * amax / 448 rounded up to a power of two, the smallest E with
 * amax <= 448 * 2^E, so nothing saturates.
 * Both clamp E to [-127, 127]; an all-zero block gets E = -127 (byte 0x00).
 * A block holding a NaN or infinity gets scale 0xFF and codes 0x7F with each
 * element's sign. Elements are v * 2^-E rounded to nearest E4M3, ties to even,
 * sign kept (-0 -> 0x80). bf16 subnormal inputs are not flushed. */
typedef enum { MX_RCEIL = 0, MX_FLOOR = 1 } mx_scale_mode;

/* Output element types of GEMMs and dequantization. */
typedef enum { MX_BF16 = 0, MX_F32 = 1 } mx_dtype;

/* Scale storage layouts (see the conventions above). */
typedef enum { MX_SCALES_PLAIN = 0, MX_SCALES_K128 = 1 } mx_scale_layout;

/* Direction bits for mx_quantize. */
enum { MX_ROWWISE = 1, MX_COLWISE = 2 };

/* Version of this ABI (changes when a signature or a layout changes). */
int mx_abi_version(void);

/* Message of the last non-OK status returned on the calling thread. */
const char* mx_last_error(void);

/* Checks that the current HIP device is a gfx950, loads the kernels and
 * looks up the device address of the work area of
 * mx_quantize_fp8_dual_scratch on it. Calling it is optional: every entry
 * point does the same check, and that entry point the same look-up. */
mx_status mx_init(void);

/* MX block quantization ("cast" kernels of [P3], Summary; the operand
 * quantization of the MXFP8 linear and grouped_mm overrides of [P1],
 * Autograd function changes).
 * x: bf16, `batch` matrices of [rows, cols]; element (b, r, c) is at
 *    x[(b * rows + r) * ld + c] (ld >= cols, in elements).
 * dirs: MX_ROWWISE and/or MX_COLWISE. Both together read x once.
 * layout: storage of both directions' scales.
 * Row-wise (needs cols % 32 == 0, % 128 for MX_SCALES_K128): q_row
 *    [batch, rows, cols] codes, s_row the scales of each [rows, cols] matrix.
 * Column-wise (needs rows % 32 == 0, % 128 for MX_SCALES_K128): q_col
 *    [batch, cols, rows], s_col the scales of each [cols, rows] matrix (per
 *    expert for 3-D weights).
 * Pointers of a direction not requested may be NULL; scale pointers must be
 * 4-byte aligned for MX_SCALES_K128. */
mx_status mx_quantize(const void* x, int64_t batch, int64_t rows, int64_t cols,
                      int64_t ld, mx_scale_mode mode, unsigned dirs,
                      mx_scale_layout layout, uint8_t* q_row, uint8_t* s_row,
                      uint8_t* q_col, uint8_t* s_col, void* stream);

/* Dequantization: out[r, c] = E4M3(q[r, c]) * 2^(scale(r, c/32) - 127),
 * exact in float32 (out_dtype MX_F32) or rounded to nearest-even bf16
 * (MX_BF16). The pages use MXFP8 values without defining them; this is the
 * value of an MX element under the OCP MX v1.0 definition above (the
 * element's E4M3 value times its block's power-of-two scale), i.e. the
 * inverse the quantization rounds against. A NaN code or a 0xFF scale gives
 * NaN. q [rows, cols], s in `layout`, out [rows, cols] contiguous;
 * cols % 32 == 0 (% 128 for MX_SCALES_K128). */
mx_status mx_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows,
                        int64_t cols, mx_scale_layout layout,
                        mx_dtype out_dtype, void* out, void* stream);

/* Fused SwiGLU + dual MXFP8 quantization, forward ([P3], Summary).
 * a, b: bf16 [rows, hidden], row stride ld_ab elements: the gate half (w1
 *    output) and up half (w3 output) of the w13 GEMM output; for a packed
 *    [rows, 2*hidden] output pass a = base, b = base + hidden, ld_ab = 2*hidden.
 * h = silu(a) * b is evaluated in float32, rounded to bf16 (the tensor the
 * unfused path would hold; it is not written unless h_out is non-NULL) and
 * quantized twice (scales in `layout`):
 *    row-wise along hidden:  q_row [rows, hidden], s_row of [rows, hidden]
 *    column-wise along rows: q_col [hidden, rows], s_col of [hidden, rows]
 * h_out: optional bf16 [rows, hidden] copy of h (NULL to skip); used by the
 *    wgrad_with_hp recipe. Needs rows % 32 == 0 and hidden % 32 == 0 (both
 *    % 128 for MX_SCALES_K128). */
mx_status mx_swiglu_quant_fwd(const void* a, const void* b, int64_t ld_ab,
                              int64_t rows, int64_t hidden, mx_scale_mode mode,
                              mx_scale_layout layout, uint8_t* q_row,
                              uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                              void* h_out, void* stream);

/* Fused SwiGLU backward + dual MXFP8 quantization ([P3], Summary).
 * dh: bf16 [rows, hidden], row stride ld_dh (gradient of h, from the w2
 *    input-gradient GEMM); a, b as in the forward.
 * With s = sigmoid(a): dA = dh*b*s*(1 + a*(1-s)), dB = dh*a*s, in float32,
 * rounded to bf16, laid out as dZ = [dA | dB] [rows, 2*hidden] and quantized
 * (scales in `layout`):
 *    row-wise along 2*hidden: q_row [rows, 2*hidden], s_row of [rows, 2*hidden]
 *    column-wise along rows:  q_col [2*hidden, rows], s_col of [2*hidden, rows]
 * dab_out: optional bf16 [rows, 2*hidden] copy of dZ (NULL to skip).
 * Needs rows % 32 == 0 and hidden % 32 == 0 (both % 128 for MX_SCALES_K128). */
mx_status mx_swiglu_quant_bwd(const void* dh, int64_t ld_dh, const void* a,
                              const void* b, int64_t ld_ab, int64_t rows,
                              int64_t hidden, mx_scale_mode mode,
                              mx_scale_layout layout, uint8_t* q_row,
                              uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                              void* dab_out, void* stream);

/* MXFP8 scaled GEMM for the linear override ([P1], Autograd function
 * changes: _to_mxfp8_then_scaled_mm). out[m, n] = sum_k A[m,k] * B[n,k] with
 * A = deq(qa [M, K], sa) and B = deq(qb [N, K], sb), float32 accumulation,
 * then rounded to out_dtype (bf16: nearest-even).
 * Every GEMM of this library reads its scales in the MX_SCALES_K128 layout
 * only (4-byte aligned): a tile's scales for one K step are then one
 * contiguous run. Scales written in MX_SCALES_PLAIN must be re-quantized (or
 * permuted) into MX_SCALES_K128 before they are passed to a GEMM; the GEMMs
 * cannot tell the layouts apart and would read wrong scales.
 * out row stride ld_out elements (>= N, rows 16-byte aligned). K % 128 == 0,
 * K < 2^23 (a tile's 256 operand rows are addressed with 32-bit offsets);
 * M, N >= 0 (an empty output enqueues nothing).
 * The same call serves the forward, the input gradient (A = dY row-wise,
 * B = W column-wise) and the weight gradient (A = dY column-wise, B = X
 * column-wise). */
mx_status mx_scaled_mm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb,
                       const uint8_t* sb, int64_t M, int64_t N, int64_t K,
                       mx_dtype out_dtype, void* out, int64_t ld_out,
                       void* stream);

/* MXFP8 grouped GEMM, 2-D x 3-D, forward ([P1], Tensor subclass changes:
 * the grouped_mm override; [P3], Summary: the grouped MLP GEMMs).
 * qa [Tcap, K], sa: tokens in padded expert-major order.
 * qw [E, N, K], sw: per-expert weights quantized along K.
 * All scales in the MX_SCALES_K128 layout (per expert for sw).
 * offs: device int32 [E] (see the conventions above).
 * out [Tcap, N] (out_dtype): rows of group g are A_g * W_g^T; rows at or past
 * offs[E-1] are written as zeros. K % 128 == 0, K < 2^23, N % 16 == 0,
 * Tcap % 128 == 0.
 * dev_err: optional device int32 (see the conventions above). */
mx_status mx_scaled_grouped_mm_fwd(const uint8_t* qa, const uint8_t* sa,
                                   const uint8_t* qw, const uint8_t* sw,
                                   const int32_t* offs, int32_t E, int64_t Tcap,
                                   int64_t N, int64_t K, mx_dtype out_dtype,
                                   void* out, int32_t* dev_err, void* stream);

/* MXFP8 grouped GEMM, input gradient: dX_g = dY_g * W_g, the backward of
 * the grouped_mm override's input ([P1], Tensor subclass changes: the
 * overrides dispatch to autograd functions wrapping these kernels; [P2],
 * Autograd func changes: the MXFP8 grouped GEMM autograd function). Same
 * contraction and argument meaning as the forward with qa = dY [Tcap, N_fwd]
 * quantized along N_fwd (row-wise) and qw = each expert's weight quantized
 * along N_fwd (column-wise of W [E, N_fwd, K_fwd]: [E, K_fwd, N_fwd]); here
 * the call's N is K_fwd and its K is N_fwd. */
mx_status mx_scaled_grouped_mm_dgrad(const uint8_t* qa, const uint8_t* sa,
                                     const uint8_t* qw, const uint8_t* sw,
                                     const int32_t* offs, int32_t E,
                                     int64_t Tcap, int64_t N, int64_t K,
                                     mx_dtype out_dtype, void* out,
                                     int32_t* dev_err, void* stream);

/* The w13 grouped forward fused with the SwiGLU + dual MX quantization that
 * follows it ([P3], The integration: fully fused grouped MLPs are the next
 * MXFP8 fusion path): one launch computes z = deq(A) deq(W13_g)^T exactly as
 * mx_scaled_grouped_mm_fwd does (W13 [E, 2H, K] = [w1; w3] per expert, gate
 * rows first) and writes it to z (bf16 [Tcap, 2H], kept for the backward),
 * and from the same tiles h = silu(z[:, :H]) * z[:, H:] quantized as
 * mx_swiglu_quant_fwd would quantize it from z: q_row [Tcap, H] with s_row
 * [H/128, Tcap, 4], q_col [H, Tcap] with s_col [Tcap/128, H, 4] (K128
 * scales), the same bytes. h_out (bf16 [Tcap, H]) is optional. Rows past
 * offs[E-1] give z = 0 and h = 0. H % 128 == 0, K % 128 == 0,
 * Tcap % 128 == 0, (H + 128) * K < 2^31 (a tile's gate and up rows are
 * addressed with 32-bit offsets). */
mx_status mx_scaled_grouped_mm_swiglu_fwd(const uint8_t* qa, const uint8_t* sa,
                                          const uint8_t* qw13,
                                          const uint8_t* sw13,
                                          const int32_t* offs, int32_t E,
                                          int64_t Tcap, int64_t H, int64_t K,
                                          mx_scale_mode mode, void* z,
                                          uint8_t* q_row, uint8_t* s_row,
                                          uint8_t* q_col, uint8_t* s_col,
                                          void* h_out, int32_t* dev_err,
                                          void* stream);

/* The grouped forward and input gradient with the result in token order:
 * the per-group padding is undone by the GEMM itself (the padded expert-major
 * layout exists only for the kernels, [P3], The integration). Arguments as
 * for mx_scaled_grouped_mm_fwd / _dgrad, plus group_sizes: device int32 [E],
 * the tokens of each group (the sizes given to mx_pad_groups /
 * mx_pad_quantize), and T, the routed tokens. out [T, N]: group g's first
 * group_sizes[g] rows of its padded slot go, in order, to out rows
 * [sum(group_sizes[0:g]), + group_sizes[g]). Pad rows and the tail are
 * computed nowhere and written nowhere. The same as unpadding the padded
 * result (mx_unpad_groups) bit for bit. A size that is negative or exceeds
 * its group's padded slot, or sizes summing past T, set bit 2 of *dev_err;
 * rows that would fall outside the slot or out are then dropped. */
mx_status mx_scaled_grouped_mm_fwd_unpad(const uint8_t* qa, const uint8_t* sa,
                                         const uint8_t* qw, const uint8_t* sw,
                                         const int32_t* offs,
                                         const int32_t* group_sizes, int32_t E,
                                         int64_t Tcap, int64_t T, int64_t N,
                                         int64_t K, mx_dtype out_dtype,
                                         void* out, int32_t* dev_err,
                                         void* stream);
mx_status mx_scaled_grouped_mm_dgrad_unpad(const uint8_t* qa, const uint8_t* sa,
                                           const uint8_t* qw, const uint8_t* sw,
                                           const int32_t* offs,
                                           const int32_t* group_sizes,
                                           int32_t E, int64_t Tcap, int64_t T,
                                           int64_t N, int64_t K,
                                           mx_dtype out_dtype, void* out,
                                           int32_t* dev_err, void* stream);

/* MXFP8 grouped GEMM, weight gradient, 2-D x 2-D: the backward of the
 * grouped_mm override's weight ([P1], Tensor subclass changes; [P2],
 * Autograd func changes: the MXFP8 grouped GEMM autograd function, whose
 * default recipe computes the weight gradient in MXFP8). The contraction
 * runs over each group's own tokens:
 * dW[g] = deq(G^T)[:, s_g:e_g] * deq(X^T)[:, s_g:e_g]^T
 * qg [N, Tcap], sg: dY column-wise (quantized along tokens).
 * qx [K, Tcap], sx: X column-wise. Scales in the MX_SCALES_K128 layout.
 * out [E, N, K] (out_dtype); an empty group's slice is written as zeros.
 * N % 16 == 0, K % 16 == 0, Tcap % 128 == 0, Tcap < 2^23 (a tile's 256
 * operand rows of Tcap codes are addressed with 32-bit offsets), and
 * ceil(N/256) * ceil(K/256) * E below 2^31 (one workgroup per tile);
 * MX_ERR_SHAPE otherwise.
 * No workspace: every 256 x 256 tile of dW is computed whole by one
 * workgroup over its group's full token range and written once from
 * registers (no split of the contraction, so no partial sums to stage);
 * groups are scheduled largest first to balance the load. */
mx_status mx_scaled_grouped_mm_wgrad(const uint8_t* qg, const uint8_t* sg,
                                     const uint8_t* qx, const uint8_t* sx,
                                     const int32_t* offs, int32_t E,
                                     int64_t Tcap, int64_t N, int64_t K,
                                     mx_dtype out_dtype, void* out,
                                     int32_t* dev_err, void* stream);

/* Grouped weight gradient for the wgrad_with_hp recipe ([P1], Autograd
 * function changes; [P2], Autograd func changes): the same per-group
 * contraction on the unquantized bf16 operands, float32 accumulation, bf16
 * (nearest-even) result. g [Tcap, N] and x [Tcap, K] bf16 row-major (tokens
 * are the strided axis); out bf16 [E, N, K]. N % 16 == 0, K % 16 == 0,
 * Tcap % 128 == 0. No workspace, for the same reason as above. */
mx_status mx_grouped_mm_wgrad_hp(const void* g, const void* x,
                                 const int32_t* offs, int32_t E, int64_t Tcap,
                                 int64_t N, int64_t K, void* out,
                                 int32_t* dev_err, void* stream);

/* FP8 (non-MX) with one power-of-two scale per row: the FP8 grouped-mm
 * training variant ([P1], review thread: FP8GroupedMMConfig; [P2], Autograd
 * func changes: FP8 MoE training, ~10% tokens/s on Llama4 Scout). The pages
 * do not give its scaling; here each row of the quantized axis gets the
 * scale the RCEIL rule picks for the whole row (nothing saturates), and a row
 * with a NaN or infinity gets scale 0xFF and codes 0x7F with the element's
 * sign. The byte is written once per 32-block in the MX_SCALES_K128 layout,
 * so these are MX operands whose block scales along a row are equal: the
 * MXFP8 GEMMs above compute the row-scaled FP8 GEMMs unchanged.
 *
 * Row-wise: x bf16 [batch, rows, cols] (row stride ld) -> q [batch, rows,
 * cols], s [batch, cols/128, rows, 4]. cols % 128 == 0. */
mx_status mx_quantize_fp8_rowwise(const void* x, int64_t batch, int64_t rows,
                                  int64_t cols, int64_t ld, uint8_t* q,
                                  uint8_t* s, void* stream);

/* Column-wise: q [batch, cols, rows] with one scale per column, or, with
 * offs (device int32 [E], exclusive ends along rows, multiples of 128, as
 * the grouped GEMMs take them), one scale per (column, group) and one for
 * the rows after offs[E-1] (the weight gradient contracts each group's tokens
 * separately). s [batch, rows/128, cols, 4]. rows % 128 == 0,
 * cols % 128 == 0. work: caller-owned device scratch of batch * (E + 1) *
 * cols int32 (batch * cols without offs), overwritten. Three kernels.
 * offs are checked on the device as the grouped GEMMs check theirs
 * (non-decreasing multiples of 128, at most rows); if they are not and
 * dev_err is non-NULL, bit 0 of *dev_err is set and the scales are then
 * unspecified. */
mx_status mx_quantize_fp8_colwise(const void* x, int64_t batch, int64_t rows,
                                  int64_t cols, int64_t ld,
                                  const int32_t* offs, int32_t E, uint8_t* q,
                                  uint8_t* s, int32_t* work, int32_t* dev_err,
                                  void* stream);

/* Both directions of the same tensor at once: the codes and scales that
 * mx_quantize_fp8_rowwise and mx_quantize_fp8_colwise (with the same offs)
 * write, bit for bit, from two reads of x instead of four. One pass folds
 * row and column maxima into work; a second quantizes each 128 x 128 tile
 * both ways. q_row [batch, rows, cols], s_row [batch, cols/128, rows, 4];
 * q_col [batch, cols, rows], s_col [batch, rows/128, cols, 4].
 * rows % 128 == 0, cols % 128 == 0. work: caller-owned device scratch of
 * batch * ((E + 1) * cols + rows) int32 (batch * (cols + rows) without
 * offs), overwritten. Three kernels. offs and dev_err as for
 * mx_quantize_fp8_colwise. */
mx_status mx_quantize_fp8_dual(const void* x, int64_t batch, int64_t rows,
                               int64_t cols, int64_t ld, const int32_t* offs,
                               int32_t E, uint8_t* q_row, uint8_t* s_row,
                               uint8_t* q_col, uint8_t* s_col, int32_t* work,
                               int32_t* dev_err, void* stream);

/* mx_quantize_fp8_dual without the caller's work area, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): same arguments, results and
 * errors as mx_quantize_fp8_dual, bit for bit, minus `work`. The work area
 * is the library's own: a 4 MiB device array per GPU (1 Mi int32), held
 * until the process ends. The call needs batch * ((E + 1) * cols + rows)
 * int32 of it (batch * (cols + rows) without offs); larger calls are
 * rejected with MX_ERR_SHAPE before anything is enqueued. It allocates and
 * frees nothing. Every call on one GPU shares that GPU's array and clears
 * what it uses first: calls that overlap in time on one GPU (other streams,
 * other threads) race on it and must be ordered by the caller. */
mx_status mx_quantize_fp8_dual_scratch(const void* x, int64_t batch,
                                       int64_t rows, int64_t cols, int64_t ld,
                                       const int32_t* offs, int32_t E,
                                       uint8_t* q_row, uint8_t* s_row,
                                       uint8_t* q_col, uint8_t* s_col,
                                       int32_t* dev_err, void* stream);

/* Per-group token padding ([P1], the torchtitan commit adding
 * pad_token_groups_for_grouped_mm; [P3], The integration: pad_multiple=128).
 * x: [T, row_bytes] rows (any element type), tokens grouped by expert in
 *    expert order. group_sizes: device int32 [E], tokens per expert.
 * Group g is copied, in order, to the start of a slot of
 * ceil(n_g / pad_multiple) * pad_multiple rows; slots follow each other.
 * x_pad [Tcap, row_bytes]: pad rows and the tail past the last slot are
 *    written as zeros.
 * offs_pad: device int32 [E], exclusive slot ends (the grouped GEMM offsets).
 * src_row: device int32 [Tcap], source row of each padded row, -1 for padding.
 * row_bytes % 16 == 0; pad_multiple a positive multiple of 32; Tcap >= 0.
 * If the sizes are negative, do not sum to T, or the slots exceed Tcap,
 * bit 1 of *dev_err is set (if dev_err is non-NULL) and rows that would fall
 * outside x or x_pad are treated as padding. */
mx_status mx_pad_groups(const void* x, const int32_t* group_sizes, int32_t E,
                        int64_t T, int64_t row_bytes, int32_t pad_multiple,
                        int64_t Tcap, void* x_pad, int32_t* offs_pad,
                        int32_t* src_row, int32_t* dev_err, void* stream);

/* Per-group padding fused with MX quantization: the result equals
 * mx_pad_groups (row_bytes = 2 * cols) followed by mx_quantize of the bf16
 * x_pad [Tcap, cols], but x_pad is never written. The padded layout is what
 * the grouped GEMMs consume ([P3], The integration: the dispatcher hands the
 * kernels a padded expert-major layout, pad_multiple=128; [P1], the
 * torchtitan commit on dynamic per-group padding kernels); writing it
 * straight in MXFP8 is this library's fusion of those two steps.
 * x: bf16 [T, cols] row-major, tokens grouped by expert in expert order.
 * group_sizes: device int32 [E]. Outputs as mx_quantize writes them for
 * [Tcap, cols] (pad rows and the tail quantize to code 0x00 with scale
 * 0x00), plus offs_pad [E] and src_row [Tcap] as mx_pad_groups writes them.
 * cols % 32 == 0 (% 128 for K128 row-wise scales); column-wise output needs
 * Tcap % 32 == 0 (% 128 for K128). Size errors are reported in *dev_err as
 * by mx_pad_groups. Two kernels are enqueued on `stream`. */
mx_status mx_pad_quantize(const void* x, const int32_t* group_sizes, int32_t E,
                          int64_t T, int64_t cols, int32_t pad_multiple,
                          int64_t Tcap, mx_scale_mode mode, unsigned dirs,
                          mx_scale_layout layout, uint8_t* q_row,
                          uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                          int32_t* offs_pad, int32_t* src_row,
                          int32_t* dev_err, void* stream);

/* Inverse of mx_pad_groups ([P1], the torchtitan commit adding
 * pad_token_groups_for_grouped_mm: per-group padding kernels for the MXFP8
 * grouped mm, whose padded results go back to token order; [P3], The
 * integration: the padded expert-major layout exists for the kernels only):
 * y[src_row[r]] = y_pad[r] for every padded row r with 0 <= src_row[r] < T.
 * y_pad [Tcap, row_bytes], y [T, row_bytes]. Rows of y that no padded row
 * maps to are left untouched. */
mx_status mx_unpad_groups(const void* y_pad, const int32_t* src_row,
                          int64_t Tcap, int64_t T, int64_t row_bytes, void* y,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_H */
