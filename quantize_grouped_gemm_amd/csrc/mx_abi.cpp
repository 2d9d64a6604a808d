// C ABI of libmxfp8.so (declared and documented in include/mxfp8.h):
// argument validation on the host, device check, and kernel launch on the
// caller's stream. Nothing here reads device memory or synchronizes.

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/mxfp8.h"
#include "mx_kernels.h"

namespace {

thread_local char g_err[512] = "";

mx_status fail(mx_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// The GEMMs address a K128 scale matrix with 32-bit buffer offsets.
bool scales_fit(int64_t rows, int64_t k) { return rows * (k / 32) < (1ll << 31); }
// A GEMM tile's 256 operand rows of K codes are addressed with 32-bit offsets.
bool k_fits(int64_t k) { return k * 256 < (1ll << 31); }

// 0 = unknown, 1 = gfx950, -1 = other
int g_dev_ok[64];

mx_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0)
    return fail(MX_ERR_DEVICE, "no HIP device (%s)", hipGetErrorString(e));
  if (dev < 64 && g_dev_ok[dev] == 1) return MX_OK;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(MX_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_dev_ok[dev] = ok ? 1 : -1;
  if (!ok) return fail(MX_ERR_DEVICE, "device %d is %s; libmxfp8 runs on gfx950 only", dev, prop.gcnArchName);
  return MX_OK;
}

mx_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MX_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

#define MX_REQUIRE(cond, st, ...) \
  do {                            \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

#define MX_DEVICE()                          \
  do {                                       \
    mx_status st_ = check_device();          \
    if (st_ != MX_OK) return st_;            \
  } while (0)

extern "C" {

int mx_abi_version(void) { return 3; }

const char* mx_last_error(void) { return g_err; }

mx_status mx_init(void) {
  mx_status st = check_device();
  if (st != MX_OK) return st;
  int32_t* scratch = nullptr;   // set-up of the allocation-free entry point's work area on this device
  return launched(mxk::fp8_scratch(&scratch), "mx_init");
}

mx_status mx_quantize(const void* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld,
                      mx_scale_mode mode, unsigned dirs, mx_scale_layout layout, uint8_t* q_row,
                      uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, void* stream) {
  MX_REQUIRE(mode == MX_RCEIL || mode == MX_FLOOR, MX_ERR_ARG, "mx_quantize: bad scale mode %d", (int)mode);
  MX_REQUIRE(dirs != 0 && (dirs & ~3u) == 0, MX_ERR_ARG, "mx_quantize: dirs must be MX_ROWWISE|MX_COLWISE");
  MX_REQUIRE(layout == MX_SCALES_PLAIN || layout == MX_SCALES_K128, MX_ERR_ARG, "mx_quantize: bad scale layout");
  const bool k128 = layout == MX_SCALES_K128;
  MX_REQUIRE(!k128 || !(dirs & MX_ROWWISE) || cols % 128 == 0, MX_ERR_SHAPE,
             "mx_quantize: K128 row-wise scales need cols (%lld) to be a multiple of 128", (long long)cols);
  MX_REQUIRE(!k128 || !(dirs & MX_COLWISE) || rows % 128 == 0, MX_ERR_SHAPE,
             "mx_quantize: K128 column-wise scales need rows (%lld) to be a multiple of 128", (long long)rows);
  MX_REQUIRE(batch >= 0 && rows >= 0 && cols >= 0, MX_ERR_SHAPE, "mx_quantize: negative size");
  MX_REQUIRE(cols % 32 == 0, MX_ERR_SHAPE, "mx_quantize: cols (%lld) must be a multiple of 32", (long long)cols);
  MX_REQUIRE(!(dirs & MX_COLWISE) || rows % 32 == 0, MX_ERR_SHAPE,
             "mx_quantize: column-wise needs rows (%lld) to be a multiple of 32", (long long)rows);
  MX_REQUIRE(ld >= cols && ld % 8 == 0, MX_ERR_ALIGN, "mx_quantize: ld (%lld) must be >= cols and a multiple of 8", (long long)ld);
  MX_REQUIRE((rows + 127) / 128 <= 65535 && batch <= 65535, MX_ERR_SHAPE, "mx_quantize: too many rows or matrices for one launch");
  if (batch == 0 || rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(x, MX_ERR_NULL, "mx_quantize: x is NULL");
  MX_REQUIRE(al16(x), MX_ERR_ALIGN, "mx_quantize: x must be 16-byte aligned");
  if (dirs & MX_ROWWISE) {
    MX_REQUIRE(q_row && s_row, MX_ERR_NULL, "mx_quantize: q_row/s_row NULL");
    MX_REQUIRE(al16(q_row), MX_ERR_ALIGN, "mx_quantize: q_row must be 16-byte aligned");
    MX_REQUIRE(!k128 || al4(s_row), MX_ERR_ALIGN, "mx_quantize: K128 s_row must be 4-byte aligned");
  }
  if (dirs & MX_COLWISE) {
    MX_REQUIRE(q_col && s_col, MX_ERR_NULL, "mx_quantize: q_col/s_col NULL");
    MX_REQUIRE(al16(q_col), MX_ERR_ALIGN, "mx_quantize: q_col must be 16-byte aligned");
    MX_REQUIRE(!k128 || al4(s_col), MX_ERR_ALIGN, "mx_quantize: K128 s_col must be 4-byte aligned");
  }
  MX_DEVICE();
  mxk::QuantArgs a{static_cast<const uint16_t*>(x), rows, cols, ld, mode == MX_RCEIL, k128,
                   (dirs & MX_ROWWISE) ? q_row : nullptr, (dirs & MX_ROWWISE) ? s_row : nullptr,
                   (dirs & MX_COLWISE) ? q_col : nullptr, (dirs & MX_COLWISE) ? s_col : nullptr};
  return launched(mxk::launch_quant(a, batch, as_stream(stream)), "mx_quantize");
}

mx_status mx_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols,
                        mx_scale_layout layout, mx_dtype out_dtype, void* out, void* stream) {
  MX_REQUIRE(out_dtype == MX_BF16 || out_dtype == MX_F32, MX_ERR_ARG, "mx_dequantize: bad dtype");
  MX_REQUIRE(layout == MX_SCALES_PLAIN || layout == MX_SCALES_K128, MX_ERR_ARG, "mx_dequantize: bad scale layout");
  const bool k128 = layout == MX_SCALES_K128;
  MX_REQUIRE(rows >= 0 && cols >= 0 && cols % (k128 ? 128 : 32) == 0, MX_ERR_SHAPE,
             "mx_dequantize: cols must be a multiple of 32 (128 for K128 scales)");
  if (rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(q && s && out, MX_ERR_NULL, "mx_dequantize: NULL pointer");
  MX_REQUIRE(al16(q) && al16(out), MX_ERR_ALIGN, "mx_dequantize: q/out must be 16-byte aligned");
  MX_DEVICE();
  mxk::DequantArgs a{q, s, rows, cols, out_dtype == MX_F32, k128, out};
  return launched(mxk::launch_dequant(a, as_stream(stream)), "mx_dequantize");
}

static mx_status check_swiglu_common(const char* fn, int64_t rows, int64_t hidden, mx_scale_mode mode,
                                     mx_scale_layout layout, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                                     uint8_t* s_col) {
  MX_REQUIRE(mode == MX_RCEIL || mode == MX_FLOOR, MX_ERR_ARG, "%s: bad scale mode", fn);
  MX_REQUIRE(layout == MX_SCALES_PLAIN || layout == MX_SCALES_K128, MX_ERR_ARG, "%s: bad scale layout", fn);
  const int64_t m = layout == MX_SCALES_K128 ? 128 : 32;
  MX_REQUIRE(rows >= 0 && hidden >= 0 && rows % m == 0 && hidden % m == 0, MX_ERR_SHAPE,
             "%s: rows and hidden must be non-negative multiples of %lld", fn, (long long)m);
  MX_REQUIRE((rows + 127) / 128 <= 65535, MX_ERR_SHAPE, "%s: too many rows for one launch", fn);
  if (rows == 0 || hidden == 0) return MX_OK;
  MX_REQUIRE(q_row && s_row && q_col && s_col, MX_ERR_NULL, "%s: NULL output", fn);
  MX_REQUIRE(al16(q_row) && al16(q_col), MX_ERR_ALIGN, "%s: code outputs must be 16-byte aligned", fn);
  MX_REQUIRE(m == 32 || (al4(s_row) && al4(s_col)), MX_ERR_ALIGN, "%s: K128 scales must be 4-byte aligned", fn);
  return MX_OK;
}

mx_status mx_swiglu_quant_fwd(const void* a, const void* b, int64_t ld_ab, int64_t rows, int64_t hidden,
                              mx_scale_mode mode, mx_scale_layout layout, uint8_t* q_row, uint8_t* s_row,
                              uint8_t* q_col, uint8_t* s_col, void* h_out, void* stream) {
  mx_status st =
      check_swiglu_common("mx_swiglu_quant_fwd", rows, hidden, mode, layout, q_row, s_row, q_col, s_col);
  if (st != MX_OK || rows == 0 || hidden == 0) return st;
  MX_REQUIRE(a && b, MX_ERR_NULL, "mx_swiglu_quant_fwd: a/b NULL");
  MX_REQUIRE(al16(a) && al16(b) && ld_ab >= hidden && ld_ab % 8 == 0, MX_ERR_ALIGN,
             "mx_swiglu_quant_fwd: a/b must be 16-byte aligned, ld_ab >= hidden and a multiple of 8");
  MX_REQUIRE(!h_out || al16(h_out), MX_ERR_ALIGN, "mx_swiglu_quant_fwd: h_out must be 16-byte aligned");
  MX_DEVICE();
  mxk::SwigluFwdArgs k{static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), ld_ab, rows, hidden,
                       mode == MX_RCEIL, layout == MX_SCALES_K128, q_row, s_row, q_col, s_col,
                       static_cast<uint16_t*>(h_out)};
  return launched(mxk::launch_swiglu_fwd(k, as_stream(stream)), "mx_swiglu_quant_fwd");
}

mx_status mx_swiglu_quant_bwd(const void* dh, int64_t ld_dh, const void* a, const void* b, int64_t ld_ab,
                              int64_t rows, int64_t hidden, mx_scale_mode mode, mx_scale_layout layout,
                              uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, void* dab_out,
                              void* stream) {
  mx_status st =
      check_swiglu_common("mx_swiglu_quant_bwd", rows, hidden, mode, layout, q_row, s_row, q_col, s_col);
  if (st != MX_OK || rows == 0 || hidden == 0) return st;
  MX_REQUIRE(dh && a && b, MX_ERR_NULL, "mx_swiglu_quant_bwd: dh/a/b NULL");
  MX_REQUIRE(al16(dh) && al16(a) && al16(b) && ld_ab >= hidden && ld_ab % 8 == 0 && ld_dh >= hidden &&
                 ld_dh % 8 == 0,
             MX_ERR_ALIGN, "mx_swiglu_quant_bwd: inputs must be 16-byte aligned with ld >= hidden, ld % 8 == 0");
  MX_REQUIRE(!dab_out || al16(dab_out), MX_ERR_ALIGN, "mx_swiglu_quant_bwd: dab_out must be 16-byte aligned");
  MX_DEVICE();
  mxk::SwigluBwdArgs k{static_cast<const uint16_t*>(dh), static_cast<const uint16_t*>(a),
                       static_cast<const uint16_t*>(b), ld_dh, ld_ab, rows, hidden, mode == MX_RCEIL,
                       layout == MX_SCALES_K128, q_row, s_row, q_col, s_col, static_cast<uint16_t*>(dab_out)};
  return launched(mxk::launch_swiglu_bwd(k, as_stream(stream)), "mx_swiglu_quant_bwd");
}

static mx_status check_mx_operand(const char* fn, const char* name, const uint8_t* q, const uint8_t* s) {
  MX_REQUIRE(q && s, MX_ERR_NULL, "%s: %s codes/scales NULL", fn, name);
  MX_REQUIRE(al16(q), MX_ERR_ALIGN, "%s: %s codes must be 16-byte aligned", fn, name);
  MX_REQUIRE(al4(s), MX_ERR_ALIGN, "%s: %s scales must be 4-byte aligned", fn, name);
  return MX_OK;
}

#define MX_CHECK(expr)              \
  do {                              \
    mx_status st_ = (expr);         \
    if (st_ != MX_OK) return st_;   \
  } while (0)

mx_status mx_scaled_mm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb,
                       int64_t M, int64_t N, int64_t K, mx_dtype out_dtype, void* out, int64_t ld_out,
                       void* stream) {
  const char* fn = "mx_scaled_mm";
  MX_REQUIRE(out_dtype == MX_BF16 || out_dtype == MX_F32, MX_ERR_ARG, "%s: bad dtype", fn);
  MX_REQUIRE(M >= 0 && N >= 0 && K > 0 && K % 128 == 0, MX_ERR_SHAPE, "%s: K (%lld) must be a positive multiple of 128", fn, (long long)K);
  MX_REQUIRE((M + 255) / 256 <= 65535 && (N + 255) / 256 <= 65535, MX_ERR_SHAPE, "%s: M or N too large", fn);
  MX_REQUIRE((M + 255) / 256 * ((N + 255) / 256) + 4096 <= 0x7FFFFFFF, MX_ERR_SHAPE,
             "%s: too many tiles for one launch", fn);
  MX_REQUIRE(scales_fit(M, K) && scales_fit(N, K), MX_ERR_SHAPE, "%s: scale matrices too large", fn);
  MX_REQUIRE(k_fits(K), MX_ERR_SHAPE, "%s: K (%lld) must be below 2^23", fn, (long long)K);
  if (M == 0 || N == 0) return MX_OK;
  MX_CHECK(check_mx_operand(fn, "A", qa, sa));
  MX_CHECK(check_mx_operand(fn, "B", qb, sb));
  const int esz = out_dtype == MX_F32 ? 4 : 2;
  MX_REQUIRE(out, MX_ERR_NULL, "%s: out NULL", fn);
  MX_REQUIRE(al16(out) && ld_out >= N && (ld_out * esz) % 16 == 0, MX_ERR_ALIGN,
             "%s: out must be 16-byte aligned and ld_out >= N with 16-byte rows", fn);
  MX_DEVICE();
  mxk::GemmArgs a{};
  a.qa = qa; a.sa = sa; a.qb = qb; a.sb = sb;
  a.M = M; a.N = N; a.K = K;
  a.lda = K; a.ldb = K; a.srows_a = M; a.srows_b = N;
  a.out = out; a.ldo = ld_out; a.out_f32 = out_dtype == MX_F32;
  return launched(mxk::launch_gemm_dense(a, as_stream(stream)), fn);
}

static mx_status grouped_2d3d(const char* fn, const uint8_t* qa, const uint8_t* sa, const uint8_t* qw,
                              const uint8_t* sw, const int32_t* offs, int32_t E, int64_t Tcap, int64_t N,
                              int64_t K, mx_dtype out_dtype, void* out, int32_t* dev_err, void* stream,
                              const int32_t* sizes = nullptr, int64_t T = 0) {
  MX_REQUIRE(out_dtype == MX_BF16 || out_dtype == MX_F32, MX_ERR_ARG, "%s: bad dtype", fn);
  MX_REQUIRE(E >= 1 && E <= 1024, MX_ERR_SHAPE, "%s: E (%d) must be in [1, 1024]", fn, E);
  MX_REQUIRE(Tcap >= 0 && Tcap % 128 == 0, MX_ERR_SHAPE, "%s: Tcap must be a multiple of 128", fn);
  MX_REQUIRE(N > 0 && N % 16 == 0, MX_ERR_SHAPE, "%s: N must be a positive multiple of 16", fn);
  MX_REQUIRE(K > 0 && K % 128 == 0, MX_ERR_SHAPE, "%s: K must be a positive multiple of 128", fn);
  MX_REQUIRE(Tcap / 256 + E <= 65535 && (N + 255) / 256 <= 65535, MX_ERR_SHAPE, "%s: too large", fn);
  // the launch covers every possible row tile times the column tiles (plus
  // the slack of the XCD deal) in one 1-D grid of int-indexed workgroups
  MX_REQUIRE((Tcap / 256 + (E + 2) / 2 + 1) * ((N + 255) / 256) + 4096 <= 0x7FFFFFFF, MX_ERR_SHAPE,
             "%s: too many tiles for one launch", fn);
  MX_REQUIRE(scales_fit(Tcap, K) && scales_fit(N, K), MX_ERR_SHAPE, "%s: scale matrices too large", fn);
  MX_REQUIRE(k_fits(K), MX_ERR_SHAPE, "%s: K (%lld) must be below 2^23", fn, (long long)K);
  if (Tcap == 0) return MX_OK;
  MX_CHECK(check_mx_operand(fn, "A", qa, sa));
  MX_CHECK(check_mx_operand(fn, "W", qw, sw));
  MX_REQUIRE(offs && out, MX_ERR_NULL, "%s: offs/out NULL", fn);
  MX_REQUIRE(al16(out), MX_ERR_ALIGN, "%s: out must be 16-byte aligned", fn);
  MX_DEVICE();
  mxk::GemmArgs a{};
  a.qa = qa; a.sa = sa; a.qb = qw; a.sb = sw;
  a.M = Tcap; a.N = N; a.K = K;
  a.lda = K; a.ldb = K; a.srows_a = Tcap; a.srows_b = N;
  a.b_group_stride = N * K; a.sb_group_stride = N * (K / 32);
  a.out = out; a.ldo = N; a.out_f32 = out_dtype == MX_F32;
  a.offs = offs; a.E = E; a.dev_err = dev_err;
  a.sizes = sizes; a.out_rows = T;
  return launched(mxk::launch_gemm_grouped(a, as_stream(stream)), fn);
}

mx_status mx_scaled_grouped_mm_swiglu_fwd(const uint8_t* qa, const uint8_t* sa, const uint8_t* qw,
                                          const uint8_t* sw, const int32_t* offs, int32_t E, int64_t Tcap,
                                          int64_t H, int64_t K, mx_scale_mode mode, void* z, uint8_t* q_row,
                                          uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, void* h_out,
                                          int32_t* dev_err, void* stream) {
  const char* fn = "mx_scaled_grouped_mm_swiglu_fwd";
  MX_REQUIRE(mode == MX_RCEIL || mode == MX_FLOOR, MX_ERR_ARG, "%s: bad scale mode %d", fn, (int)mode);
  MX_REQUIRE(E >= 1 && E <= 1024, MX_ERR_SHAPE, "%s: E (%d) must be in [1, 1024]", fn, E);
  MX_REQUIRE(Tcap >= 0 && Tcap % 128 == 0, MX_ERR_SHAPE, "%s: Tcap must be a multiple of 128", fn);
  MX_REQUIRE(H > 0 && H % 128 == 0, MX_ERR_SHAPE, "%s: H must be a positive multiple of 128", fn);
  MX_REQUIRE(K > 0 && K % 128 == 0, MX_ERR_SHAPE, "%s: K must be a positive multiple of 128", fn);
  MX_REQUIRE(Tcap / 256 + E <= 65535 && H / 128 <= 65535, MX_ERR_SHAPE, "%s: too large", fn);
  MX_REQUIRE((Tcap / 256 + (E + 2) / 2 + 1) * (H / 128) + 4096 <= 0x7FFFFFFF, MX_ERR_SHAPE,
             "%s: too many tiles for one launch", fn);
  MX_REQUIRE(scales_fit(Tcap, K) && scales_fit(2 * H, K), MX_ERR_SHAPE, "%s: scale matrices too large", fn);
  MX_REQUIRE(Tcap * 2 * H * 2 < (1ll << 40), MX_ERR_SHAPE, "%s: z too large", fn);
  // a tile's B rows span the gate rows and the up rows H rows further
  MX_REQUIRE((H + 128) * K < (1ll << 31), MX_ERR_SHAPE, "%s: (H + 128) x K must be below 2^31", fn);
  if (Tcap == 0) return MX_OK;
  MX_CHECK(check_mx_operand(fn, "A", qa, sa));
  MX_CHECK(check_mx_operand(fn, "W13", qw, sw));
  MX_REQUIRE(offs && z && q_row && s_row && q_col && s_col, MX_ERR_NULL, "%s: NULL pointer", fn);
  MX_REQUIRE(al16(z) && al16(q_row) && al16(q_col) && al4(s_row) && al4(s_col) && (!h_out || al16(h_out)),
             MX_ERR_ALIGN, "%s: z/q/h must be 16-byte and scales 4-byte aligned", fn);
  MX_DEVICE();
  mxk::GemmArgs a{};
  a.qa = qa; a.sa = sa; a.qb = qw; a.sb = sw;
  a.M = Tcap; a.N = 2 * H; a.K = K;
  a.lda = K; a.ldb = K; a.srows_a = Tcap; a.srows_b = 2 * H;
  a.b_group_stride = 2 * H * K; a.sb_group_stride = 2 * H * (K / 32);
  a.out = z; a.ldo = 2 * H; a.out_f32 = false;
  a.offs = offs; a.E = E; a.dev_err = dev_err;
  a.hq_row = q_row; a.hs_row = s_row; a.hq_col = q_col; a.hs_col = s_col;
  a.h_out = static_cast<uint16_t*>(h_out); a.rceil = mode == MX_RCEIL;
  return launched(mxk::launch_gemm_grouped_swiglu(a, as_stream(stream)), fn);
}

// Token-order variants: the output holds the T routed tokens, not the
// padded rows.
static mx_status grouped_2d3d_unpad(const char* fn, const uint8_t* qa, const uint8_t* sa, const uint8_t* qw,
                                    const uint8_t* sw, const int32_t* offs, const int32_t* group_sizes,
                                    int32_t E, int64_t Tcap, int64_t T, int64_t N, int64_t K, mx_dtype out_dtype,
                                    void* out, int32_t* dev_err, void* stream) {
  MX_REQUIRE(T >= 0 && T <= Tcap, MX_ERR_SHAPE, "%s: T (%lld) must be in [0, Tcap]", fn, (long long)T);
  MX_REQUIRE(Tcap == 0 || group_sizes, MX_ERR_NULL, "%s: group_sizes NULL", fn);
  if (T == 0) return MX_OK;
  return grouped_2d3d(fn, qa, sa, qw, sw, offs, E, Tcap, N, K, out_dtype, out, dev_err, stream, group_sizes, T);
}

mx_status mx_scaled_grouped_mm_fwd_unpad(const uint8_t* qa, const uint8_t* sa, const uint8_t* qw,
                                         const uint8_t* sw, const int32_t* offs, const int32_t* group_sizes,
                                         int32_t E, int64_t Tcap, int64_t T, int64_t N, int64_t K,
                                         mx_dtype out_dtype, void* out, int32_t* dev_err, void* stream) {
  return grouped_2d3d_unpad("mx_scaled_grouped_mm_fwd_unpad", qa, sa, qw, sw, offs, group_sizes, E, Tcap, T, N,
                            K, out_dtype, out, dev_err, stream);
}

mx_status mx_scaled_grouped_mm_dgrad_unpad(const uint8_t* qa, const uint8_t* sa, const uint8_t* qw,
                                           const uint8_t* sw, const int32_t* offs, const int32_t* group_sizes,
                                           int32_t E, int64_t Tcap, int64_t T, int64_t N, int64_t K,
                                           mx_dtype out_dtype, void* out, int32_t* dev_err, void* stream) {
  return grouped_2d3d_unpad("mx_scaled_grouped_mm_dgrad_unpad", qa, sa, qw, sw, offs, group_sizes, E, Tcap, T,
                            N, K, out_dtype, out, dev_err, stream);
}

mx_status mx_scaled_grouped_mm_fwd(const uint8_t* qa, const uint8_t* sa, const uint8_t* qw, const uint8_t* sw,
                                   const int32_t* offs, int32_t E, int64_t Tcap, int64_t N, int64_t K,
                                   mx_dtype out_dtype, void* out, int32_t* dev_err, void* stream) {
  return grouped_2d3d("mx_scaled_grouped_mm_fwd", qa, sa, qw, sw, offs, E, Tcap, N, K, out_dtype, out,
                      dev_err, stream);
}

mx_status mx_scaled_grouped_mm_dgrad(const uint8_t* qa, const uint8_t* sa, const uint8_t* qw,
                                     const uint8_t* sw, const int32_t* offs, int32_t E, int64_t Tcap,
                                     int64_t N, int64_t K, mx_dtype out_dtype, void* out, int32_t* dev_err,
                                     void* stream) {
  return grouped_2d3d("mx_scaled_grouped_mm_dgrad", qa, sa, qw, sw, offs, E, Tcap, N, K, out_dtype, out,
                      dev_err, stream);
}

mx_status mx_scaled_grouped_mm_wgrad(const uint8_t* qg, const uint8_t* sg, const uint8_t* qx,
                                     const uint8_t* sx, const int32_t* offs, int32_t E, int64_t Tcap,
                                     int64_t N, int64_t K, mx_dtype out_dtype, void* out, int32_t* dev_err,
                                     void* stream) {
  const char* fn = "mx_scaled_grouped_mm_wgrad";
  MX_REQUIRE(out_dtype == MX_BF16 || out_dtype == MX_F32, MX_ERR_ARG, "%s: bad dtype", fn);
  MX_REQUIRE(E >= 1 && E <= 1024 && E <= 65535, MX_ERR_SHAPE, "%s: E must be in [1, 1024]", fn);
  MX_REQUIRE(Tcap >= 0 && Tcap % 128 == 0, MX_ERR_SHAPE, "%s: Tcap must be a multiple of 128", fn);
  MX_REQUIRE(N > 0 && N % 16 == 0 && K > 0 && K % 16 == 0, MX_ERR_SHAPE, "%s: N and K must be positive multiples of 16", fn);
  MX_REQUIRE((N + 255) / 256 <= 65535 && (K + 255) / 256 <= 65535, MX_ERR_SHAPE, "%s: too large", fn);
  // one workgroup per 256 x 256 tile of every group's dW, in a 1-D grid
  MX_REQUIRE((N + 255) / 256 * ((K + 255) / 256) * E <= 0x7FFFFFFF, MX_ERR_SHAPE,
             "%s: too many tiles for one launch", fn);
  MX_REQUIRE(scales_fit(N, Tcap) && scales_fit(K, Tcap), MX_ERR_SHAPE, "%s: scale matrices too large", fn);
  MX_REQUIRE(Tcap * 256 < (1ll << 31), MX_ERR_SHAPE,
             "%s: Tcap (%lld) must be below 2^23: a tile's 256 operand rows are addressed with 32-bit offsets", fn,
             (long long)Tcap);
  MX_CHECK(check_mx_operand(fn, "G", qg, sg));
  MX_CHECK(check_mx_operand(fn, "X", qx, sx));
  MX_REQUIRE(offs && out, MX_ERR_NULL, "%s: offs/out NULL", fn);
  MX_REQUIRE(al16(out), MX_ERR_ALIGN, "%s: out must be 16-byte aligned", fn);
  MX_DEVICE();
  mxk::GemmArgs a{};
  a.qa = qg; a.sa = sg; a.qb = qx; a.sb = sx;
  a.M = Tcap; a.N = N; a.K = K;
  a.lda = Tcap; a.ldb = Tcap; a.srows_a = N; a.srows_b = K;
  a.out_group_stride = N * K;
  a.out = out; a.ldo = K; a.out_f32 = out_dtype == MX_F32;
  a.offs = offs; a.E = E; a.dev_err = dev_err;
  return launched(mxk::launch_gemm_wgrad(a, as_stream(stream)), fn);
}

mx_status mx_grouped_mm_wgrad_hp(const void* g, const void* x, const int32_t* offs, int32_t E, int64_t Tcap,
                                 int64_t N, int64_t K, void* out, int32_t* dev_err, void* stream) {
  const char* fn = "mx_grouped_mm_wgrad_hp";
  MX_REQUIRE(E >= 1 && E <= 1024, MX_ERR_SHAPE, "%s: E must be in [1, 1024]", fn);
  MX_REQUIRE(Tcap >= 0 && Tcap % 128 == 0, MX_ERR_SHAPE, "%s: Tcap must be a multiple of 128", fn);
  MX_REQUIRE(N > 0 && N % 16 == 0 && K > 0 && K % 16 == 0, MX_ERR_SHAPE, "%s: N and K must be positive multiples of 16", fn);
  MX_REQUIRE((N + 255) / 256 * ((K + 255) / 256) * E <= 0x7FFFFFFF, MX_ERR_SHAPE, "%s: too large", fn);
  // the kernel addresses each operand with 32-bit buffer offsets
  MX_REQUIRE(Tcap * N * 2 < (1ll << 31) && Tcap * K * 2 < (1ll << 31), MX_ERR_SHAPE, "%s: operands too large", fn);
  MX_REQUIRE(g && x && offs && out, MX_ERR_NULL, "%s: NULL pointer", fn);
  MX_REQUIRE(al16(g) && al16(x) && al16(out), MX_ERR_ALIGN, "%s: g/x/out must be 16-byte aligned", fn);
  MX_DEVICE();
  mxk::GemmArgs a{};
  a.qa = static_cast<const uint8_t*>(g); a.qb = static_cast<const uint8_t*>(x);
  a.M = Tcap; a.N = N; a.K = K;
  a.lda = 2 * N; a.ldb = 2 * K;
  a.out_group_stride = N * K;
  a.out = out; a.ldo = K; a.out_f32 = false;
  a.offs = offs; a.E = E; a.dev_err = dev_err;
  return launched(mxk::launch_gemm_wgrad_hp(a, as_stream(stream)), fn);
}

mx_status mx_pad_groups(const void* x, const int32_t* group_sizes, int32_t E, int64_t T, int64_t row_bytes,
                        int32_t pad_multiple, int64_t Tcap, void* x_pad, int32_t* offs_pad, int32_t* src_row,
                        int32_t* dev_err, void* stream) {
  const char* fn = "mx_pad_groups";
  MX_REQUIRE(E >= 1 && E <= 1024, MX_ERR_SHAPE, "%s: E must be in [1, 1024]", fn);
  MX_REQUIRE(T >= 0 && Tcap >= 0 && T < (1ll << 31) && Tcap < (1ll << 31), MX_ERR_SHAPE, "%s: T/Tcap out of range", fn);
  MX_REQUIRE(row_bytes > 0 && row_bytes % 16 == 0, MX_ERR_SHAPE, "%s: row_bytes must be a positive multiple of 16", fn);
  MX_REQUIRE(pad_multiple > 0 && pad_multiple % 32 == 0, MX_ERR_SHAPE, "%s: pad_multiple must be a positive multiple of 32", fn);
  MX_REQUIRE(group_sizes && offs_pad && (Tcap == 0 || (x_pad && src_row)) && (T == 0 || x), MX_ERR_NULL,
             "%s: NULL pointer", fn);
  MX_REQUIRE((T == 0 || al16(x)) && (Tcap == 0 || al16(x_pad)), MX_ERR_ALIGN, "%s: x/x_pad must be 16-byte aligned", fn);
  MX_DEVICE();
  mxk::PadArgs a{static_cast<const uint8_t*>(x), group_sizes, E, T, row_bytes, Tcap, pad_multiple,
                 static_cast<uint8_t*>(x_pad), offs_pad, src_row, dev_err};
  return launched(mxk::launch_pad(a, as_stream(stream)), fn);
}

mx_status mx_pad_quantize(const void* x, const int32_t* group_sizes, int32_t E, int64_t T, int64_t cols,
                          int32_t pad_multiple, int64_t Tcap, mx_scale_mode mode, unsigned dirs,
                          mx_scale_layout layout, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                          int32_t* offs_pad, int32_t* src_row, int32_t* dev_err, void* stream) {
  const char* fn = "mx_pad_quantize";
  MX_REQUIRE(mode == MX_RCEIL || mode == MX_FLOOR, MX_ERR_ARG, "%s: bad scale mode %d", fn, (int)mode);
  MX_REQUIRE(dirs != 0 && (dirs & ~3u) == 0, MX_ERR_ARG, "%s: dirs must be MX_ROWWISE|MX_COLWISE", fn);
  MX_REQUIRE(layout == MX_SCALES_PLAIN || layout == MX_SCALES_K128, MX_ERR_ARG, "%s: bad scale layout", fn);
  const bool k128 = layout == MX_SCALES_K128;
  MX_REQUIRE(E >= 1 && E <= 1024, MX_ERR_SHAPE, "%s: E must be in [1, 1024]", fn);
  MX_REQUIRE(T >= 0 && Tcap >= 0 && T < (1ll << 31) && Tcap < (1ll << 31), MX_ERR_SHAPE, "%s: T/Tcap out of range", fn);
  MX_REQUIRE(cols > 0 && cols % 32 == 0, MX_ERR_SHAPE, "%s: cols (%lld) must be a positive multiple of 32", fn,
             (long long)cols);
  MX_REQUIRE(pad_multiple > 0 && pad_multiple % 32 == 0, MX_ERR_SHAPE,
             "%s: pad_multiple must be a positive multiple of 32", fn);
  MX_REQUIRE(!k128 || !(dirs & MX_ROWWISE) || cols % 128 == 0, MX_ERR_SHAPE,
             "%s: K128 row-wise scales need cols (%lld) to be a multiple of 128", fn, (long long)cols);
  MX_REQUIRE(!(dirs & MX_COLWISE) || Tcap % (k128 ? 128 : 32) == 0, MX_ERR_SHAPE,
             "%s: column-wise output needs Tcap (%lld) to be a multiple of %d", fn, (long long)Tcap, k128 ? 128 : 32);
  MX_REQUIRE((Tcap + 127) / 128 <= 65535, MX_ERR_SHAPE, "%s: Tcap too large for one launch", fn);
  MX_REQUIRE(group_sizes && offs_pad && (Tcap == 0 || src_row) && (T == 0 || x), MX_ERR_NULL, "%s: NULL pointer", fn);
  MX_REQUIRE(T == 0 || al16(x), MX_ERR_ALIGN, "%s: x must be 16-byte aligned", fn);
  if (Tcap > 0 && (dirs & MX_ROWWISE)) {
    MX_REQUIRE(q_row && s_row, MX_ERR_NULL, "%s: q_row/s_row NULL", fn);
    MX_REQUIRE(al16(q_row) && (!k128 || al4(s_row)), MX_ERR_ALIGN, "%s: q_row must be 16-byte and K128 s_row 4-byte aligned", fn);
  }
  if (Tcap > 0 && (dirs & MX_COLWISE)) {
    MX_REQUIRE(q_col && s_col, MX_ERR_NULL, "%s: q_col/s_col NULL", fn);
    MX_REQUIRE(al16(q_col) && (!k128 || al4(s_col)), MX_ERR_ALIGN, "%s: q_col must be 16-byte and K128 s_col 4-byte aligned", fn);
  }
  MX_DEVICE();
  hipStream_t st = as_stream(stream);
  mxk::PadArgs p{static_cast<const uint8_t*>(x), group_sizes, E, T, cols * 2, Tcap, pad_multiple, nullptr,
                 offs_pad, src_row, dev_err};
  mx_status r = launched(mxk::launch_pad_map(p, st), fn);
  if (r != MX_OK || Tcap == 0) return r;
  mxk::QuantArgs a{static_cast<const uint16_t*>(x), Tcap, cols, cols, mode == MX_RCEIL, k128,
                   (dirs & MX_ROWWISE) ? q_row : nullptr, (dirs & MX_ROWWISE) ? s_row : nullptr,
                   (dirs & MX_COLWISE) ? q_col : nullptr, (dirs & MX_COLWISE) ? s_col : nullptr,
                   src_row, T};
  return launched(mxk::launch_quant(a, 1, st), fn);
}

mx_status mx_quantize_fp8_rowwise(const void* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld,
                                  uint8_t* q, uint8_t* s, void* stream) {
  const char* fn = "mx_quantize_fp8_rowwise";
  MX_REQUIRE(batch >= 0 && rows >= 0 && cols >= 0, MX_ERR_SHAPE, "%s: negative size", fn);
  MX_REQUIRE(cols % 128 == 0, MX_ERR_SHAPE, "%s: cols (%lld) must be a multiple of 128", fn, (long long)cols);
  MX_REQUIRE(ld >= cols && ld % 8 == 0, MX_ERR_ALIGN, "%s: ld must be >= cols and a multiple of 8", fn);
  MX_REQUIRE((rows + 15) / 16 <= 0x7FFFFFFF && batch <= 65535, MX_ERR_SHAPE, "%s: too large for one launch", fn);
  if (batch == 0 || rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(x && q && s, MX_ERR_NULL, "%s: NULL pointer", fn);
  MX_REQUIRE(al16(x) && al16(q) && al4(s), MX_ERR_ALIGN, "%s: x/q must be 16-byte and s 4-byte aligned", fn);
  MX_DEVICE();
  mxk::Fp8Args a{static_cast<const uint16_t*>(x), batch, rows, cols, ld, q, s, nullptr, 0, 1, nullptr};
  return launched(mxk::launch_fp8_rowscale(a, as_stream(stream)), fn);
}

mx_status mx_quantize_fp8_colwise(const void* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld,
                                  const int32_t* offs, int32_t E, uint8_t* q, uint8_t* s, int32_t* work,
                                  int32_t* dev_err, void* stream) {
  const char* fn = "mx_quantize_fp8_colwise";
  MX_REQUIRE(batch >= 0 && rows >= 0 && cols >= 0, MX_ERR_SHAPE, "%s: negative size", fn);
  MX_REQUIRE(rows % 128 == 0 && cols % 128 == 0, MX_ERR_SHAPE, "%s: rows and cols must be multiples of 128", fn);
  MX_REQUIRE(ld >= cols && ld % 8 == 0, MX_ERR_ALIGN, "%s: ld must be >= cols and a multiple of 8", fn);
  MX_REQUIRE(!offs || (E >= 1 && E <= 1024), MX_ERR_SHAPE, "%s: E must be in [1, 1024] with offsets", fn);
  MX_REQUIRE(rows / 128 <= 65535 && cols / 128 <= 0x7FFFFFFF && batch <= 65535, MX_ERR_SHAPE,
             "%s: too large for one launch", fn);
  if (batch == 0 || rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(x && q && s && work, MX_ERR_NULL, "%s: NULL pointer", fn);
  MX_REQUIRE(al16(x) && al16(q) && al4(s) && al4(work), MX_ERR_ALIGN, "%s: misaligned pointer", fn);
  MX_DEVICE();
  mxk::Fp8Args a{static_cast<const uint16_t*>(x), batch, rows, cols, ld, q, s, offs, offs ? E : 0,
                 offs ? (int64_t)E + 1 : 1, work};
  a.dev_err = dev_err;
  return launched(mxk::launch_fp8_colscale(a, as_stream(stream)), fn);
}

mx_status mx_quantize_fp8_dual(const void* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld,
                               const int32_t* offs, int32_t E, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                               uint8_t* s_col, int32_t* work, int32_t* dev_err, void* stream) {
  const char* fn = "mx_quantize_fp8_dual";
  MX_REQUIRE(batch >= 0 && rows >= 0 && cols >= 0, MX_ERR_SHAPE, "%s: negative size", fn);
  MX_REQUIRE(rows % 128 == 0 && cols % 128 == 0, MX_ERR_SHAPE, "%s: rows and cols must be multiples of 128", fn);
  MX_REQUIRE(ld >= cols && ld % 8 == 0, MX_ERR_ALIGN, "%s: ld must be >= cols and a multiple of 8", fn);
  MX_REQUIRE(!offs || (E >= 1 && E <= 1024), MX_ERR_SHAPE, "%s: E must be in [1, 1024] with offsets", fn);
  MX_REQUIRE(rows / 128 <= 65535 && cols / 128 <= 0x7FFFFFFF && batch <= 65535, MX_ERR_SHAPE,
             "%s: too large for one launch", fn);
  if (batch == 0 || rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(x && q_row && s_row && q_col && s_col && work, MX_ERR_NULL, "%s: NULL pointer", fn);
  MX_REQUIRE(al16(x) && al16(q_row) && al16(q_col) && al4(s_row) && al4(s_col) && al4(work), MX_ERR_ALIGN,
             "%s: misaligned pointer", fn);
  MX_DEVICE();
  const int64_t segments = offs ? (int64_t)E + 1 : 1;
  mxk::Fp8Args a{static_cast<const uint16_t*>(x), batch, rows, cols, ld, q_row, s_row, offs, offs ? E : 0,
                 segments, work};
  a.q_col = q_col;
  a.s_col = s_col;
  a.row_max = work + batch * segments * cols;
  a.dev_err = dev_err;
  return launched(mxk::launch_fp8_dual(a, as_stream(stream)), fn);
}

mx_status mx_quantize_fp8_dual_scratch(const void* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld,
                                       const int32_t* offs, int32_t E, uint8_t* q_row, uint8_t* s_row,
                                       uint8_t* q_col, uint8_t* s_col, int32_t* dev_err, void* stream) {
  const char* fn = "mx_quantize_fp8_dual_scratch";
  MX_REQUIRE(batch >= 0 && rows >= 0 && cols >= 0, MX_ERR_SHAPE, "%s: negative size", fn);
  MX_REQUIRE(rows % 128 == 0 && cols % 128 == 0, MX_ERR_SHAPE, "%s: rows and cols must be multiples of 128", fn);
  MX_REQUIRE(ld >= cols && ld % 8 == 0, MX_ERR_ALIGN, "%s: ld must be >= cols and a multiple of 8", fn);
  MX_REQUIRE(!offs || (E >= 1 && E <= 1024), MX_ERR_SHAPE, "%s: E must be in [1, 1024] with offsets", fn);
  MX_REQUIRE(rows / 128 <= 65535 && cols / 128 <= 0x7FFFFFFF && batch <= 65535, MX_ERR_SHAPE,
             "%s: too large for one launch", fn);
  const int64_t segments = offs ? (int64_t)E + 1 : 1;
  const int64_t need = batch * (segments * cols + rows);
  MX_REQUIRE(need <= mxk::kFp8ScratchInts, MX_ERR_SHAPE,
             "%s: needs %lld int32 of work area, more than the %lld (4 MiB) the library holds; use "
             "mx_quantize_fp8_dual with a caller workspace", fn, (long long)need, (long long)mxk::kFp8ScratchInts);
  if (batch == 0 || rows == 0 || cols == 0) return MX_OK;
  MX_REQUIRE(x && q_row && s_row && q_col && s_col, MX_ERR_NULL, "%s: NULL pointer", fn);
  MX_REQUIRE(al16(x) && al16(q_row) && al16(q_col) && al4(s_row) && al4(s_col), MX_ERR_ALIGN,
             "%s: misaligned pointer", fn);
  MX_DEVICE();
  int32_t* work = nullptr;
  mx_status r = launched(mxk::fp8_scratch(&work), fn);
  if (r != MX_OK) return r;
  mxk::Fp8Args a{static_cast<const uint16_t*>(x), batch, rows, cols, ld, q_row, s_row, offs, offs ? E : 0,
                 segments, work};
  a.q_col = q_col;
  a.s_col = s_col;
  a.row_max = work + batch * segments * cols;
  a.dev_err = dev_err;
  return launched(mxk::launch_fp8_dual(a, as_stream(stream)), fn);
}

mx_status mx_unpad_groups(const void* y_pad, const int32_t* src_row, int64_t Tcap, int64_t T, int64_t row_bytes,
                          void* y, void* stream) {
  const char* fn = "mx_unpad_groups";
  MX_REQUIRE(T >= 0 && Tcap >= 0 && Tcap < (1ll << 31), MX_ERR_SHAPE, "%s: T/Tcap out of range", fn);
  MX_REQUIRE(row_bytes > 0 && row_bytes % 16 == 0, MX_ERR_SHAPE, "%s: row_bytes must be a positive multiple of 16", fn);
  if (Tcap == 0 || T == 0) return MX_OK;
  MX_REQUIRE(y_pad && src_row && y, MX_ERR_NULL, "%s: NULL pointer", fn);
  MX_REQUIRE(al16(y_pad) && al16(y), MX_ERR_ALIGN, "%s: y/y_pad must be 16-byte aligned", fn);
  MX_DEVICE();
  mxk::UnpadArgs a{static_cast<const uint8_t*>(y_pad), src_row, Tcap, T, row_bytes, static_cast<uint8_t*>(y)};
  return launched(mxk::launch_unpad(a, as_stream(stream)), fn);
}

}  // extern "C"
