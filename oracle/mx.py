"""MXFP8 training hot path: plain CPU definitions in numpy float64.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.

Pages followed
  [P1] "TrainingWeightWrapperTensor base class; subclasses for FP8/MXFP8 with
       grouped_mm and linear overrides" (pytorch/ao pull request 3968)
  [P2] "[mxfp8 training] unified MXFP8TrainingConfig and MXFP8TrainingTensor"
       (pytorch/ao pull request 3948)
  [P3] "Add MXFP8 fused-MLP overrides in torchtitan" (pytorch/torchtitan
       pull request 4257)

The pages name the method's parts (MXFP8 linear and grouped_mm training, the
RCEIL scale mode, wgrad_with_hp, per-group token padding to a multiple of 128,
the fused SwiGLU + dual MXFP8 quantization boundary) but never define the
number formats. MXFP8 is the OCP Microscaling Formats (MX) v1.0 format: blocks
of 32 contiguous values, one E8M0 power-of-two scale per block, FP8 E4M3
("E4M3FN": no infinities, 0x7F/0xFF are NaN, largest finite 448) elements.
Steps the pages leave open are marked READING below.

Conventions
  * bf16 tensors travel as uint16 bit patterns, E4M3 codes and E8M0 scales as
    uint8, offsets as int32. Everything is row-major.
  * Row-wise quantization ("row-q") blocks the last axis: an [R, C] tensor
    gives codes [R, C] and scales [R, C/32]. Column-wise ("col-q") is row-q of
    the transpose: codes [C, R], scales [C, R/32].
  * Every GEMM is C = A . B^T with the contraction axis contiguous in both
    operands.

Parity status: every function here is pinned by tests/test_oracle_*.py
against closed forms, exhaustive enumeration, exact rational brute force or an
independent library routine (torch CPU casts, torch autograd). The two MLP
compositions at the bottom chain pinned functions; they are pinned stage by
stage against a second CPU implementation written with torch primitives
(torch's float8 casts, float64 matmuls, silu and autograd), each stage fed
the oracle's own inputs to it, so every operand, axis, scale mode and bf16
rounding of the wiring is checked (tests/test_oracle_mlp_stages.py).
"""

import numpy as np

BLOCK = 32                 # OCP MX block size
E4M3_MAX = 448.0           # largest finite E4M3 value, 1.75 * 2**8
E4M3_EMAX = 8              # exponent of that value; OCP MX's emax for E4M3
E4M3_EMIN = -6             # exponent of the smallest normal E4M3 value
E8M0_BIAS = 127
SCALE_MIN_EXP = -127       # E8M0 byte 0x00
SCALE_MAX_EXP = 127        # E8M0 byte 0xFE; 0xFF is NaN

RCEIL = 0
FLOOR = 1
MODES = {"rceil": RCEIL, "floor": FLOOR, RCEIL: RCEIL, FLOOR: FLOOR}

__all__ = [
    "BLOCK", "E4M3_MAX", "RCEIL", "FLOOR", "E4M3_VALUES",
    "bf16_to_f64", "f64_to_bf16", "f64_to_f32", "e8m0_to_f64",
    "scale_exponent", "e4m3_encode", "quantize", "quantize_bf16",
    "quantize_fp8_rows", "quantize_fp8_bf16",
    "dequantize", "silu", "swiglu_f64", "swiglu_grad_f64", "swiglu_fwd",
    "swiglu_bwd",
    "swiglu_quant_fwd", "swiglu_quant_bwd", "scaled_mm", "grouped_mm",
    "grouped_mm_wgrad", "grouped_mm_wgrad_hp", "pad_groups", "unpad_groups",
    "dense_mlp_step", "moe_mlp_step",
]


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def bf16_to_f64(bits):
    """bf16 bit patterns -> float64. bf16 is the top half of an IEEE float32,
    so this is exact for every pattern (subnormals, infinities, NaN)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_f32(x):
    """float64 -> float32, IEEE round-to-nearest-even (numpy's cast)."""
    return np.asarray(x, np.float64).astype(np.float32)


def f64_to_bf16(x):
    """float64 -> bf16 bit patterns, rounded once to nearest, ties to even.

    Rounding is done directly on the float64 value (no float32 stop), on the
    bf16 grid: 7 stored mantissa bits, normal exponents down to -126 and
    subnormal spacing 2**-133 below that. Values that round past the largest
    finite bf16 become infinity, as IEEE rounding prescribes.
    """
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    finite = np.isfinite(a)
    af = np.where(finite & (a > 0), a, 1.0)
    _, ex = np.frexp(af)                       # af = f * 2**ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -126)               # binade of a; subnormals use -126
    ulp = np.ldexp(1.0, e - 7)
    with np.errstate(over="ignore"):
        q = np.rint(np.where(finite, a, 0.0) / ulp) * ulp   # exact scaling by 2**k
        q = np.where(q >= 2.0 ** 128, np.inf, q)
    q = np.where(finite, q, a)                 # inf stays inf, NaN stays NaN
    bits = (q.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return (bits | np.where(np.signbit(x), np.uint16(0x8000), np.uint16(0))).astype(np.uint16)


def _e4m3_table():
    """Decoded value of each of the 256 E4M3 codes (OCP E4M3FN)."""
    c = np.arange(256)
    sign = c >> 7
    exp = (c >> 3) & 0xF
    man = c & 0x7
    mag = np.where(exp == 0,
                   man / 8.0 * 2.0 ** E4M3_EMIN,                 # subnormal
                   (1.0 + man / 8.0) * np.ldexp(1.0, exp - 7))   # normal, bias 7
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)        # 0x7F, 0xFF
    return np.where(sign == 1, -mag, mag)


E4M3_VALUES = _e4m3_table()


def e8m0_to_f64(s):
    """E8M0 scale byte -> 2**(s - 127); 0xFF is NaN."""
    s = np.asarray(s).astype(np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - E8M0_BIAS))


# --------------------------------------------------------------------------
# MX block quantization
# --------------------------------------------------------------------------

def scale_exponent(amax, mode):
    """Shared block exponent E (scale 2**E) for block maxima ``amax`` >= 0.

    FLOOR (the OCP MX v1.0 rule): E = floor(log2(amax)) - emax, emax = 8 for
    E4M3. The scaled maximum then lies in [256, 512), so values above 448
    saturate.
    RCEIL (named on [P1], review thread, as ScaleCalculationMode.RCEIL; its
    formula is not on the pages). READING: the scale is amax / 448 rounded up
    to a power of two, i.e. the smallest integer E with amax <= 448 * 2**E.
    Nothing saturates in this mode.
    READING for amax = 0 (pages silent): E = -127, the smallest E8M0 scale.
    Both modes clamp E to the E8M0 range [-127, 127]. Non-finite amax is
    handled by the caller.
    """
    mode = MODES[mode]
    amax = np.asarray(amax, np.float64)
    pos = np.isfinite(amax) & (amax > 0)
    _, ex = np.frexp(np.where(pos, amax, 1.0))
    ea = ex - 1                                # floor(log2(amax)), exact
    if mode == FLOOR:
        E = ea - E4M3_EMAX
    else:
        # Candidate E = ea - 8 gives 448 * 2**E = 1.75 * 2**ea: it holds the
        # block exactly when amax <= that. E = ea - 9 (0.875 * 2**ea) never
        # does since amax >= 2**ea; E = ea - 7 (3.5 * 2**ea) always does.
        bound = np.ldexp(E4M3_MAX, ea - E4M3_EMAX)
        E = np.where(amax <= bound, ea - E4M3_EMAX, ea - E4M3_EMAX + 1)
    E = np.where(pos, E, SCALE_MIN_EXP)
    return np.clip(E, SCALE_MIN_EXP, SCALE_MAX_EXP).astype(np.int64)


def e4m3_encode(y):
    """float64 -> E4M3 code: saturate |y| to 448, round to nearest with ties
    to even, keep the sign (so -0 -> 0x80). NaN -> 0x7F with its sign."""
    y = np.asarray(y, np.float64)
    neg = np.signbit(y)
    nan = np.isnan(y)
    a = np.minimum(np.where(nan, 0.0, np.abs(y)), E4M3_MAX)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex - 1, E4M3_EMIN)          # subnormals share 2**-6's spacing
    step = np.ldexp(1.0, e - 3)                # 3 mantissa bits
    q = np.rint(a / step) * step               # numpy rint: ties to even
    # code of the grid value q
    _, exq = np.frexp(np.where(q > 0, q, 1.0))
    eq = exq - 1
    normal = q >= 2.0 ** E4M3_EMIN
    man_n = np.where(normal, q / np.ldexp(1.0, eq) * 8 - 8, 0).astype(np.int64)
    code_n = ((eq + 7) << 3) | man_n
    code_s = (q / 2.0 ** -9).astype(np.int64)  # 0..7 (8 would be 2**-6, normal)
    code = np.where(normal, code_n, code_s)
    code = np.where(nan, 0x7F, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize(x, mode):
    """Row-wise MX quantization of float64 values along the last axis.

    Per block of 32: amax = max |v|; E from ``scale_exponent``; elements
    y = v * 2**-E (exact in float64, a power-of-two scaling far from the
    float64 range limits) encoded by ``e4m3_encode``. Scale byte = E + 127.
    READING (pages silent, OCP's NaN rule): a block holding a NaN or infinity
    gets scale 0xFF and every code 0x7F with the element's sign.
    Returns (codes uint8 [..., C], scales uint8 [..., C/32]).
    """
    x = np.asarray(x, np.float64)
    C = x.shape[-1]
    if C % BLOCK:
        raise ValueError("quantized axis must be a multiple of 32")
    blk = x.reshape(x.shape[:-1] + (C // BLOCK, BLOCK))
    with np.errstate(invalid="ignore"):
        amax = np.max(np.abs(blk), axis=-1)
    finite = np.isfinite(amax)
    E = scale_exponent(np.where(finite, amax, 0.0), mode)
    y = blk * np.ldexp(1.0, -E)[..., None]
    codes = e4m3_encode(np.where(finite[..., None], y, 0.0))
    bad = (0x7F | np.where(np.signbit(blk), 0x80, 0)).astype(np.uint8)
    codes = np.where(finite[..., None], codes, bad)
    scales = np.where(finite, E + E8M0_BIAS, 255).astype(np.uint8)
    return codes.reshape(x.shape), scales


def quantize_bf16(bits, mode, rowwise=True, colwise=False):
    """MX quantization of a bf16 tensor [..., R, C].

    Row-q blocks along C; col-q blocks along R and returns the transposed
    layout [..., C, R] with scales [..., C, R/32]. Leading axes are a batch
    (e.g. experts) quantized independently.
    Returns a dict with keys 'q_row', 's_row', 'q_col', 's_col' as requested.
    """
    x = bf16_to_f64(bits)
    out = {}
    if rowwise:
        out["q_row"], out["s_row"] = quantize(x, mode)
    if colwise:
        out["q_col"], out["s_col"] = quantize(np.swapaxes(x, -1, -2), mode)
    return out


# --------------------------------------------------------------------------
# FP8 with one scale per row (the non-MX FP8 grouped-mm training variant;
# [P1], review thread: FP8GroupedMMConfig; [P2], Autograd func changes: FP8
# MoE training, about 10% more tokens/s on Llama4 Scout. Its scaling is not
# on the pages.)
# --------------------------------------------------------------------------

def quantize_fp8_rows(x):
    """READING: FP8 E4M3 with one power-of-two scale per row of the quantized
    (last) axis, chosen by the RCEIL rule over the whole row: the smallest E
    with amax(row) <= 448 * 2**E, so nothing saturates; elements are encoded
    as in ``quantize``; a row holding a NaN or infinity gets scale 0xFF and
    codes 0x7F with the element's sign. The row's scale byte is returned once
    per 32-block, so the result is an MX operand whose block scales along a
    row are all equal (the MX GEMMs then compute the FP8 row-scaled GEMM).
    Returns (codes uint8 [..., C], scales uint8 [..., C/32])."""
    x = np.asarray(x, np.float64)
    C = x.shape[-1]
    if C % BLOCK:
        raise ValueError("quantized axis must be a multiple of 32")
    with np.errstate(invalid="ignore"):
        amax = np.max(np.abs(x), axis=-1)
    finite = np.isfinite(amax)
    E = scale_exponent(np.where(finite, amax, 0.0), RCEIL)
    y = x * np.ldexp(1.0, -E)[..., None]
    codes = e4m3_encode(np.where(finite[..., None], y, 0.0))
    bad = (np.signbit(x).astype(np.uint8) << 7) | np.uint8(0x7F)
    codes = np.where(finite[..., None], codes, bad).astype(np.uint8)
    sb = np.where(finite, E + E8M0_BIAS, 255).astype(np.uint8)
    return codes, np.repeat(sb[..., None], C // BLOCK, axis=-1)


def quantize_fp8_bf16(bits, rowwise=True, colwise=False, segments=None):
    """FP8 row-scaled quantization of a bf16 tensor [..., R, C]: row-wise
    scales one per row of [R, C]; column-wise quantizes the transpose
    [..., C, R] one scale per row of it, or, with ``segments`` (exclusive ends
    along R, the grouped GEMM offsets; READING: the weight gradient's
    contraction runs over each group's own tokens, so each column gets one
    scale per group), one scale per (column, segment); rows past the last end
    form a segment of their own. Returns a dict with q_row, s_row, q_col,
    s_col as requested (MX-style layouts)."""
    x = bf16_to_f64(bits)
    out = {}
    if rowwise:
        out["q_row"], out["s_row"] = quantize_fp8_rows(x)
    if colwise:
        xt = np.swapaxes(x, -1, -2)
        if segments is None:
            out["q_col"], out["s_col"] = quantize_fp8_rows(xt)
        else:
            R = xt.shape[-1]
            q = np.zeros(xt.shape, np.uint8)
            sc = np.zeros(xt.shape[:-1] + (R // BLOCK,), np.uint8)
            bounds = [0] + [int(e) for e in segments] + [R]
            for s, e in zip(bounds[:-1], bounds[1:]):
                if e > s:
                    q[..., s:e], sc[..., s // BLOCK:e // BLOCK] = quantize_fp8_rows(xt[..., s:e])
            out["q_col"], out["s_col"] = q, sc
    return out


def dequantize(codes, scales):
    """code value * 2**E, exact in float64. [..., C] codes, [..., C/32] scales."""
    v = E4M3_VALUES[np.asarray(codes).astype(np.int64)]
    s = e8m0_to_f64(scales)
    return v * np.repeat(s, BLOCK, axis=-1)


# --------------------------------------------------------------------------
# Fused SwiGLU boundary ([P3], Summary; Numerics and tests)
# --------------------------------------------------------------------------

def silu(a):
    """silu(a) = a * sigmoid(a) = a / (1 + exp(-a)), float64."""
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def swiglu_f64(a, b):
    """h = silu(a) * b in float64 (a = gate half from w1, b = up half from w3)."""
    return silu(a) * b


def swiglu_grad_f64(dh, a, b):
    """Gradients of h = silu(a) * b in float64. With s = sigmoid(a):
    dA = dh * b * s * (1 + a * (1 - s)),  dB = dh * a * s."""
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-a))
    return dh * b * s * (1.0 + a * (1.0 - s)), dh * a * s


def swiglu_fwd(a_bits, b_bits):
    """h = silu(a) * b from the bf16 gate half a (w1 output) and up half b
    (w3 output), evaluated in float64 and rounded once to bf16.

    READING: [P3] says the fused boundary never materializes the BF16
    post-activation tensor, and that its forward is bitwise equal to
    standalone-cast quantization. A standalone cast quantizes the BF16 tensor
    the unfused path writes, so the quantized h is the bf16-rounded value; the
    fused kernel only skips storing it.
    """
    return f64_to_bf16(swiglu_f64(bf16_to_f64(a_bits), bf16_to_f64(b_bits)))


def swiglu_bwd(dh_bits, a_bits, b_bits):
    """bf16 [T, 2H] = [dA | dB] (the layout of the w13 output): the float64
    gradients of swiglu_grad_f64 rounded once to bf16 (same READING as the
    forward: the unfused path would hold these as BF16 tensors)."""
    da, db = swiglu_grad_f64(bf16_to_f64(dh_bits), bf16_to_f64(a_bits),
                             bf16_to_f64(b_bits))
    return f64_to_bf16(np.concatenate([da, db], axis=-1))


def swiglu_quant_fwd(a_bits, b_bits, mode):
    """Fused SwiGLU + dual MXFP8 quantization, forward ([P3], Summary).

    h [T, H] is quantized row-wise along H (operand of the w2 forward GEMM)
    and column-wise along T (operand of the w2 weight-gradient GEMM).
    Returns dict(q_row [T,H], s_row [T,H/32], q_col [H,T], s_col [H,T/32],
    h [T,H] bf16 bits).
    """
    h = swiglu_fwd(a_bits, b_bits)
    out = quantize_bf16(h, mode, rowwise=True, colwise=True)
    out["h"] = h
    return out


def swiglu_quant_bwd(dh_bits, a_bits, b_bits, mode):
    """Fused SwiGLU backward + dual MXFP8 quantization ([P3], Summary).

    dZ = [dA | dB] [T, 2H] (bf16) is quantized row-wise along 2H (operand of
    the w13 input-gradient GEMM; H % 32 == 0 so no block straddles the two
    halves) and column-wise along T (operand of the w13 weight-gradient GEMM).
    Returns dict(q_row [T,2H], s_row, q_col [2H,T], s_col, dab [T,2H] bf16).
    """
    dab = swiglu_bwd(dh_bits, a_bits, b_bits)
    out = quantize_bf16(dab, mode, rowwise=True, colwise=True)
    out["dab"] = dab
    return out


# --------------------------------------------------------------------------
# Scaled GEMMs ([P1], Autograd function changes; [P2], Autograd func changes)
# --------------------------------------------------------------------------

def scaled_mm(qa, sa, qb, sb):
    """C = deq(A) . deq(B)^T with A [M, K], B [N, K] quantized along K.
    float64 accumulation; the caller rounds once to the output type."""
    return dequantize(qa, sa) @ dequantize(qb, sb).T


def _group_bounds(offs, limit):
    """(g, start, end) per group from exclusive-end offsets (offs[-1] := 0)."""
    offs = [int(v) for v in np.asarray(offs).ravel()]
    start = 0
    for g, end in enumerate(offs):
        if end < start or end > limit or end % 32:
            raise ValueError("offsets must be non-decreasing multiples of 32 "
                             "within the padded capacity")
        yield g, start, end
        start = end


def grouped_mm(qa, sa, qw, sw, offs):
    """MXFP8 grouped GEMM, 2-D x 3-D (forward and input-gradient).

    For each group g, rows [offs[g-1], offs[g]) of A [Tcap, K] times
    W[g]^T (W [E, N, K], quantized along K). Rows at or past offs[E-1] are 0
    (READING of the tail inertness in [P3], Numerics and tests).
    The input gradient uses the same contraction with A = dY quantized along
    N and W[g] = the transpose of the forward weight quantized along N.
    """
    Tcap = qa.shape[0]
    E, N, _ = qw.shape
    out = np.zeros((Tcap, N))
    for g, s, e in _group_bounds(offs, Tcap):
        if e > s:
            out[s:e] = scaled_mm(qa[s:e], sa[s:e], qw[g], sw[g])
    return out


def grouped_mm_wgrad(qgT, sgT, qxT, sxT, offs):
    """MXFP8 grouped weight gradient, 2-D x 2-D: the contraction runs over
    each group's own tokens.

    dW[g] = deq(G^T)[:, s:e] . deq(X^T)[:, s:e]^T with G^T [N, Tcap] and
    X^T [K, Tcap] quantized along tokens (col-q of dY and X). Group starts
    are multiples of 32, so col-q of the whole padded tensor is col-q of each
    group. An empty group gives 0. Returns float64 [E, N, K].
    """
    N, Tcap = qgT.shape
    K = qxT.shape[0]
    offs = np.asarray(offs)
    out = np.zeros((len(offs), N, K))
    for g, s, e in _group_bounds(offs, Tcap):
        if e > s:
            b0, b1 = s // BLOCK, e // BLOCK
            out[g] = scaled_mm(qgT[:, s:e], sgT[:, b0:b1], qxT[:, s:e], sxT[:, b0:b1])
    return out


def grouped_mm_wgrad_hp(g_bits, x_bits, offs):
    """wgrad_with_hp ([P1], Autograd function changes; [P2], Autograd func
    changes). READING: the weight-gradient GEMM runs on the unquantized bf16
    operands. dW[g] = G[s:e]^T . X[s:e] with G [Tcap, N], X [Tcap, K];
    float64 accumulation; the caller rounds to bf16. Returns [E, N, K]."""
    G = bf16_to_f64(g_bits)
    X = bf16_to_f64(x_bits)
    Tcap, N = G.shape
    K = X.shape[1]
    offs = np.asarray(offs)
    out = np.zeros((len(offs), N, K))
    for g, s, e in _group_bounds(offs, Tcap):
        if e > s:
            out[g] = G[s:e].T @ X[s:e]
    return out


# --------------------------------------------------------------------------
# Per-group token padding ([P1], torchtitan commit on
# pad_token_groups_for_grouped_mm; [P3], The integration: pad_multiple=128)
# --------------------------------------------------------------------------

def pad_groups(x_bits, sizes, multiple, Tcap):
    """Copy each expert's token group (groups are contiguous, in expert order,
    in x [T, D]) to the start of a slot of ceil(n_g / multiple) * multiple
    rows. Pad rows and the tail [offs[E-1], Tcap) are zero.
    Returns (x_pad [Tcap, D], offs int32 [E] exclusive ends,
    src_row int32 [Tcap] = source row of each padded row, -1 for padding)."""
    x = np.asarray(x_bits)
    T, D = x.shape
    sizes = np.asarray(sizes, np.int64)
    if (sizes < 0).any() or sizes.sum() != T:
        raise ValueError("group sizes must be >= 0 and sum to T")
    slots = (sizes + multiple - 1) // multiple * multiple
    offs = np.cumsum(slots)
    if len(offs) and offs[-1] > Tcap:
        raise ValueError("padded groups exceed the capacity")
    x_pad = np.zeros((Tcap, D), x.dtype)
    src_row = np.full(Tcap, -1, np.int32)
    src = 0
    dst = 0
    for g in range(len(sizes)):
        n = int(sizes[g])
        x_pad[dst:dst + n] = x[src:src + n]
        src_row[dst:dst + n] = np.arange(src, src + n)
        src += n
        dst = int(offs[g])
    return x_pad, offs.astype(np.int32), src_row


def pad_quantize(x_bits, sizes, multiple, Tcap, mode, rowwise=True, colwise=False):
    """Padding followed by MX quantization of the padded bf16 tensor: what a
    fused pad + quantize must produce. Composition of pad_groups and
    quantize_bf16; the dict also holds 'offs' and 'src_row'."""
    x_pad, offs, src_row = pad_groups(x_bits, sizes, multiple, Tcap)
    out = quantize_bf16(x_pad, mode, rowwise, colwise)
    out["offs"], out["src_row"] = offs, src_row
    return out


def unpad_groups(y_pad, src_row, T):
    """Inverse of pad_groups: y[src_row[r]] = y_pad[r] for every real row."""
    y_pad = np.asarray(y_pad)
    src_row = np.asarray(src_row)
    y = np.zeros((T,) + y_pad.shape[1:], y_pad.dtype)
    real = src_row >= 0
    y[src_row[real]] = y_pad[real]
    return y


# --------------------------------------------------------------------------
# MLP compositions ([P3], Summary: w13 GEMM -> fused SwiGLU + dual MXFP8
# quantization -> w2 GEMM, dense and grouped). These only chain the functions
# above, in the order the GPU pipeline runs them.
# --------------------------------------------------------------------------

def _rt(x, dtype):
    return f64_to_bf16(x) if dtype == "bf16" else f64_to_f32(x)


def dense_mlp_step(x, w1, w3, w2, dy, mode, wgrad_dtype="f32"):
    """One dense SwiGLU MLP forward + backward in MXFP8.

    x [T, D], w1/w3 [H, D], w2 [D, H], dy [T, D], all bf16 bits.
    w13 = cat(w1, w3) [2H, D] (READING: gate half first).
    Returns a dict of every stage output.
    """
    H = w1.shape[0]
    w13 = np.concatenate([w1, w3], axis=0)
    qx = quantize_bf16(x, mode, True, True)
    q13 = quantize_bf16(w13, mode, True, True)     # col: [D, 2H]
    q2 = quantize_bf16(w2, mode, True, True)       # row along H, col: [H, D]
    z = f64_to_bf16(scaled_mm(qx["q_row"], qx["s_row"], q13["q_row"], q13["s_row"]))
    sw = swiglu_quant_fwd(z[:, :H], z[:, H:], mode)
    y = f64_to_bf16(scaled_mm(sw["q_row"], sw["s_row"], q2["q_row"], q2["s_row"]))
    qdy = quantize_bf16(dy, mode, True, True)
    dh = f64_to_bf16(scaled_mm(qdy["q_row"], qdy["s_row"], q2["q_col"], q2["s_col"]))
    dw2 = _rt(scaled_mm(qdy["q_col"], qdy["s_col"], sw["q_col"], sw["s_col"]), wgrad_dtype)
    bw = swiglu_quant_bwd(dh, z[:, :H], z[:, H:], mode)
    dx = f64_to_bf16(scaled_mm(bw["q_row"], bw["s_row"], q13["q_col"], q13["s_col"]))
    dw13 = _rt(scaled_mm(bw["q_col"], bw["s_col"], qx["q_col"], qx["s_col"]), wgrad_dtype)
    return dict(z=z, h=sw["h"], y=y, dh=dh, dab=bw["dab"], dx=dx, dw2=dw2, dw13=dw13)


def moe_mlp_step(x, sizes, w1, w3, w2, dy, mode, Tcap, multiple=128,
                 wgrad="mx", wgrad_dtype="f32", recipe="mxfp8"):
    """One routed-experts grouped MLP forward + backward in MXFP8.

    x, dy [T, D] bf16 bits in expert-major order; sizes [E] tokens per
    expert; w1/w3 [E, H, D], w2 [E, D, H]. Groups are padded to ``multiple``
    rows (pad_groups), run through the grouped GEMMs and unpadded.
    wgrad = "mx" (MXFP8 weight gradients, float ``wgrad_dtype``) or "hp"
    (wgrad_with_hp: bf16 operands, bf16 result).
    recipe = "fp8_rowwise": every operand is quantized with one scale per
    row instead (quantize_fp8_bf16; the weight-gradient operands per column
    and group), h and dA|dB from their bf16 values.
    """
    if recipe == "fp8_rowwise":
        return _moe_mlp_step_fp8(x, sizes, w1, w3, w2, dy, Tcap, multiple, wgrad_dtype)
    T = x.shape[0]
    H = w1.shape[1]
    w13 = np.concatenate([w1, w3], axis=1)          # [E, 2H, D]
    x_pad, offs, src = pad_groups(x, sizes, multiple, Tcap)
    dy_pad, _, _ = pad_groups(dy, sizes, multiple, Tcap)
    qx = quantize_bf16(x_pad, mode, True, wgrad == "mx")
    q13 = quantize_bf16(w13, mode, True, True)       # col: [E, D, 2H]
    q2 = quantize_bf16(w2, mode, True, True)         # col: [E, H, D]
    z = f64_to_bf16(grouped_mm(qx["q_row"], qx["s_row"], q13["q_row"], q13["s_row"], offs))
    sw = swiglu_quant_fwd(z[:, :H], z[:, H:], mode)
    y_pad = f64_to_bf16(grouped_mm(sw["q_row"], sw["s_row"], q2["q_row"], q2["s_row"], offs))
    qdy = quantize_bf16(dy_pad, mode, True, wgrad == "mx")
    dh = f64_to_bf16(grouped_mm(qdy["q_row"], qdy["s_row"], q2["q_col"], q2["s_col"], offs))
    bw = swiglu_quant_bwd(dh, z[:, :H], z[:, H:], mode)
    dx_pad = f64_to_bf16(grouped_mm(bw["q_row"], bw["s_row"], q13["q_col"], q13["s_col"], offs))
    if wgrad == "mx":
        dw2 = _rt(grouped_mm_wgrad(qdy["q_col"], qdy["s_col"], sw["q_col"], sw["s_col"], offs), wgrad_dtype)
        dw13 = _rt(grouped_mm_wgrad(bw["q_col"], bw["s_col"], qx["q_col"], qx["s_col"], offs), wgrad_dtype)
    else:
        dw2 = f64_to_bf16(grouped_mm_wgrad_hp(dy_pad, sw["h"], offs))
        dw13 = f64_to_bf16(grouped_mm_wgrad_hp(bw["dab"], x_pad, offs))
    return dict(offs=offs, src_row=src, x_pad=x_pad, z=z, h=sw["h"],
                y=unpad_groups(y_pad, src, T), dh=dh, dab=bw["dab"],
                dx=unpad_groups(dx_pad, src, T), dw2=dw2, dw13=dw13)


def _moe_mlp_step_fp8(x, sizes, w1, w3, w2, dy, Tcap, multiple, wgrad_dtype):
    """moe_mlp_step with FP8 row-scaled operands (see quantize_fp8_bf16)."""
    T = x.shape[0]
    H = w1.shape[1]
    w13 = np.concatenate([w1, w3], axis=1)          # [E, 2H, D]
    x_pad, offs, src = pad_groups(x, sizes, multiple, Tcap)
    dy_pad, _, _ = pad_groups(dy, sizes, multiple, Tcap)
    qx = quantize_fp8_bf16(x_pad, True, True, segments=offs)
    q13 = quantize_fp8_bf16(w13, True, True)
    q2 = quantize_fp8_bf16(w2, True, True)
    z = f64_to_bf16(grouped_mm(qx["q_row"], qx["s_row"], q13["q_row"], q13["s_row"], offs))
    h = swiglu_fwd(z[:, :H], z[:, H:])
    qh = quantize_fp8_bf16(h, True, True, segments=offs)
    y_pad = f64_to_bf16(grouped_mm(qh["q_row"], qh["s_row"], q2["q_row"], q2["s_row"], offs))
    qdy = quantize_fp8_bf16(dy_pad, True, True, segments=offs)
    dh = f64_to_bf16(grouped_mm(qdy["q_row"], qdy["s_row"], q2["q_col"], q2["s_col"], offs))
    dab = swiglu_bwd(dh, z[:, :H], z[:, H:])
    qdz = quantize_fp8_bf16(dab, True, True, segments=offs)
    dx_pad = f64_to_bf16(grouped_mm(qdz["q_row"], qdz["s_row"], q13["q_col"], q13["s_col"], offs))
    dw2 = _rt(grouped_mm_wgrad(qdy["q_col"], qdy["s_col"], qh["q_col"], qh["s_col"], offs), wgrad_dtype)
    dw13 = _rt(grouped_mm_wgrad(qdz["q_col"], qdz["s_col"], qx["q_col"], qx["s_col"], offs), wgrad_dtype)
    return dict(offs=offs, src_row=src, x_pad=x_pad, z=z, h=h, y=unpad_groups(y_pad, src, T), dh=dh, dab=dab,
                dx=unpad_groups(dx_pad, src, T), dw2=dw2, dw13=dw13)
