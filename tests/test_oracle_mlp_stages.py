"""Stage-by-stage pins of the oracle's MLP compositions (dense_mlp_step and
moe_mlp_step) against the independent torch-CPU recomposition in torch_mx.

Each stage is recomputed from the oracle's own inputs to that stage and must
agree with the oracle's output of that stage: bf16 results equal or one bf16
ulp apart (torch's float64 -> bf16 cast rounds twice), float32 results equal
or one float32 ulp apart (the two float64 matmuls sum in different orders),
each on at most a small fraction of elements. The planted-mistake tests show
that a swapped gate and up half, a swapped scale mode or a row-wise operand
where a column-wise one belongs breaks these checks."""

import numpy as np
import pytest
import torch

import torch_mx as TM
from oracle import mx as O
from quantize_grouped_gemm_amd import synth


def _close(got, ref, kind, what, frac=2e-3):
    """got, ref float64 arrays; kind 'bf16' or 'f32' sets the unit."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, what
    mant = 7 if kind == "bf16" else 23
    mag = np.maximum(np.abs(got), np.abs(ref))
    e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    ulp = np.exp2(np.maximum(e, -126) - mant)
    d = np.abs(got - ref)
    assert np.all(d <= ulp), f"{what}: {int(np.sum(d > ulp))} elements more than one ulp apart"
    n_diff = int(np.sum(d > 0))
    assert n_diff <= max(3, frac * d.size), f"{what}: {n_diff} of {d.size} elements differ"
    return n_diff


def _bf(bits):
    return O.bf16_to_f64(bits)


def _t(bits):
    return TM.from_bits(bits)


def _inputs(T, D, H, E=None, seed=0):
    x, w1, w3, w2, dy = [synth.bits(t) for t in synth.mlp_inputs(T, D, H, E=E, seed=seed)]
    # larger gate/up weights give O(1) activations, so SwiGLU is not near-linear
    w1 = synth.bits(synth.from_bits(w1).float().mul(40).bfloat16())
    w3 = synth.bits(synth.from_bits(w3).float().mul(40).bfloat16())
    return x, w1, w3, w2, dy


def check_dense(out, x, w1, w3, w2, dy, mode):
    """Stage-wise check of a dense_mlp_step result; returns mismatch counts."""
    H = w1.shape[0]
    X, W2, DY = _t(x), _t(w2), _t(dy)
    W13 = torch.cat([_t(w1), _t(w3)], 0)
    n = {}
    z = TM.to_bf16(TM.mx_rows(X, mode) @ TM.mx_rows(W13, mode).T)
    n["z"] = _close(_bf(out["z"]), z, "bf16", "z")
    Z = _t(out["z"])
    a, b = Z[:, :H], Z[:, H:]
    n["h"] = _close(_bf(out["h"]), TM.to_bf16(TM.swiglu(a, b)), "bf16", "h")
    Hh = _t(out["h"])
    n["y"] = _close(_bf(out["y"]), TM.to_bf16(TM.mx_rows(Hh, mode) @ TM.mx_rows(W2, mode).T), "bf16", "y")
    n["dh"] = _close(_bf(out["dh"]), TM.to_bf16(TM.mx_rows(DY, mode) @ TM.mx_cols(W2, mode)), "bf16", "dh")
    n["dw2"] = _close(out["dw2"], (TM.mx_cols(DY, mode).T @ TM.mx_cols(Hh, mode)).to(torch.float32).double(),
                      "f32", "dw2")
    da, db = TM.swiglu_grads(_t(out["dh"]), a, b)
    n["dab"] = _close(_bf(out["dab"]), TM.to_bf16(torch.cat([da, db], 1)), "bf16", "dab")
    DAB = _t(out["dab"])
    n["dx"] = _close(_bf(out["dx"]), TM.to_bf16(TM.mx_rows(DAB, mode) @ TM.mx_cols(W13, mode)), "bf16", "dx")
    n["dw13"] = _close(out["dw13"], (TM.mx_cols(DAB, mode).T @ TM.mx_cols(X, mode)).to(torch.float32).double(),
                       "f32", "dw13")
    return n


def check_moe(out, x, sizes, w1, w3, w2, dy, mode, Tcap, wgrad="mx", recipe="mxfp8"):
    """Stage-wise check of a moe_mlp_step result."""
    E, H = w1.shape[0], w1.shape[1]
    T = x.shape[0]
    fp8 = recipe == "fp8_rowwise"
    X, DY, W2 = _t(x), _t(dy), _t(w2)
    W13 = torch.cat([_t(w1), _t(w3)], 1)
    Xp, ends, idx = TM.pad(X, sizes, 128, Tcap)
    DYp, _, _ = TM.pad(DY, sizes, 128, Tcap)
    assert list(out["offs"]) == ends
    src = np.full(Tcap, -1, np.int64)
    src[idx.numpy()] = np.arange(T)
    assert np.array_equal(out["src_row"], src)
    assert np.array_equal(_bf(out["x_pad"]), Xp.numpy())
    rows = (lambda t: TM.fp8_rows(t)) if fp8 else (lambda t: TM.mx_rows(t, mode))
    cols = (lambda t: TM.fp8_cols(t)) if fp8 else (lambda t: TM.mx_cols(t, mode))

    n = {}
    z = torch.zeros((Tcap, 2 * H), dtype=torch.float64)
    for g, s, e in TM.groups(ends):
        if e > s:
            z[s:e] = rows(Xp[s:e]) @ rows(W13[g]).T
    n["z"] = _close(_bf(out["z"]), TM.to_bf16(z), "bf16", "z")
    Z = _t(out["z"])
    a, b = Z[:, :H], Z[:, H:]
    n["h"] = _close(_bf(out["h"]), TM.to_bf16(TM.swiglu(a, b)), "bf16", "h")
    Hh = _t(out["h"])
    yp = torch.zeros((Tcap, W2.shape[1]), dtype=torch.float64)
    for g, s, e in TM.groups(ends):
        if e > s:
            yp[s:e] = rows(Hh[s:e]) @ rows(W2[g]).T
    n["y"] = _close(_bf(out["y"]), TM.to_bf16(yp)[idx], "bf16", "y")
    dh = torch.zeros((Tcap, H), dtype=torch.float64)
    for g, s, e in TM.groups(ends):
        if e > s:
            dh[s:e] = rows(DYp[s:e]) @ cols(W2[g])
    n["dh"] = _close(_bf(out["dh"]), TM.to_bf16(dh), "bf16", "dh")
    da, db = TM.swiglu_grads(_t(out["dh"]), a, b)
    n["dab"] = _close(_bf(out["dab"]), TM.to_bf16(torch.cat([da, db], 1)), "bf16", "dab")
    DAB = _t(out["dab"])
    dxp = torch.zeros((Tcap, X.shape[1]), dtype=torch.float64)
    for g, s, e in TM.groups(ends):
        if e > s:
            dxp[s:e] = rows(DAB[s:e]) @ cols(W13[g])
    n["dx"] = _close(_bf(out["dx"]), TM.to_bf16(dxp)[idx], "bf16", "dx")
    dw2 = torch.zeros((E,) + tuple(W2.shape[1:]), dtype=torch.float64)
    dw13 = torch.zeros((E,) + tuple(W13.shape[1:]), dtype=torch.float64)
    for g, s, e in TM.groups(ends):
        if e == s:
            continue
        if wgrad == "hp":
            dw2[g] = DYp[s:e].T @ Hh[s:e]
            dw13[g] = DAB[s:e].T @ Xp[s:e]
        else:
            # quantized along the group's own tokens
            dw2[g] = cols(DYp[s:e]).T @ cols(Hh[s:e])
            dw13[g] = cols(DAB[s:e]).T @ cols(Xp[s:e])
    if wgrad == "hp":
        n["dw2"] = _close(_bf(out["dw2"]), TM.to_bf16(dw2), "bf16", "dw2")
        n["dw13"] = _close(_bf(out["dw13"]), TM.to_bf16(dw13), "bf16", "dw13")
    else:
        n["dw2"] = _close(out["dw2"], dw2.to(torch.float32).double(), "f32", "dw2")
        n["dw13"] = _close(out["dw13"], dw13.to(torch.float32).double(), "f32", "dw13")
    return n


@pytest.mark.parametrize("mode", ["rceil", "floor"])
def test_dense_mlp_step_stagewise(mode):
    T, D, H = 96, 128, 64
    args = _inputs(T, D, H, seed=4)
    out = O.dense_mlp_step(*args, mode)
    check_dense(out, *args, mode)


@pytest.mark.parametrize("wgrad,recipe,mode", [("mx", "mxfp8", "rceil"), ("mx", "mxfp8", "floor"),
                                               ("hp", "mxfp8", "rceil"), ("mx", "fp8_rowwise", "rceil")])
def test_moe_mlp_step_stagewise(wgrad, recipe, mode):
    E, T, D, H = 4, 300, 64, 64
    sizes = np.array([100, 0, 170, 30])
    Tcap = synth.capacity(T, E)
    x, w1, w3, w2, dy = _inputs(T, D, H, E=E, seed=5)
    out = O.moe_mlp_step(x, sizes, w1, w3, w2, dy, mode, Tcap, wgrad=wgrad, recipe=recipe)
    check_moe(out, x, sizes, w1, w3, w2, dy, mode, Tcap, wgrad=wgrad, recipe=recipe)


# ---------------------------------------------------------------- planted mistakes

def _expect_caught(fn):
    with pytest.raises(AssertionError):
        fn()


def test_planted_gate_up_swap_is_caught(monkeypatch):
    T, D, H = 96, 128, 64
    args = _inputs(T, D, H, seed=4)
    real = O.swiglu_quant_fwd
    monkeypatch.setattr(O, "swiglu_quant_fwd", lambda a, b, mode: real(b, a, mode))
    out = O.dense_mlp_step(*args, "rceil")
    _expect_caught(lambda: check_dense(out, *args, "rceil"))


def test_planted_scale_mode_swap_is_caught(monkeypatch):
    """The weights quantized with FLOOR inside an RCEIL step."""
    T, D, H = 96, 128, 64
    args = _inputs(T, D, H, seed=4)
    real = O.quantize_bf16
    calls = {"n": 0}

    def q(bits, mode, rowwise=True, colwise=False):
        calls["n"] += 1
        if calls["n"] in (2, 3):     # w13 and w2
            mode = "floor"
        return real(bits, mode, rowwise, colwise)

    monkeypatch.setattr(O, "quantize_bf16", q)
    out = O.dense_mlp_step(*args, "rceil")
    _expect_caught(lambda: check_dense(out, *args, "rceil"))


def test_planted_wrong_quantization_axis_is_caught(monkeypatch):
    """The weight-gradient operand of x quantized along D (row-wise of the
    transpose of a square block) instead of along tokens."""
    T = D = 128
    H = 64
    args = _inputs(T, D, H, seed=6)
    real = O.quantize_bf16

    def q(bits, mode, rowwise=True, colwise=False):
        out = real(bits, mode, rowwise, colwise)
        if colwise and bits.shape == (T, D):
            # blocks along D, laid out as if they ran along tokens (same shapes)
            r = real(bits, mode, True, False)
            out["q_col"] = np.ascontiguousarray(r["q_row"].T)
            out["s_col"] = r["s_row"]
        return out

    monkeypatch.setattr(O, "quantize_bf16", q)
    out = O.dense_mlp_step(*args, "rceil")
    _expect_caught(lambda: check_dense(out, *args, "rceil"))


def test_planted_dropped_bf16_rounding_is_caught(monkeypatch):
    """h quantized from the float64 SwiGLU value instead of its bf16 rounding."""
    E, T, D, H = 4, 300, 64, 64
    sizes = np.array([100, 0, 170, 30])
    Tcap = synth.capacity(T, E)
    x, w1, w3, w2, dy = _inputs(T, D, H, E=E, seed=5)

    def fwd(a_bits, b_bits, mode):
        hf = O.swiglu_f64(O.bf16_to_f64(a_bits), O.bf16_to_f64(b_bits))
        out = dict(zip(("q_row", "s_row"), O.quantize(hf, mode)))
        out["q_col"], out["s_col"] = O.quantize(hf.T, mode)
        out["h"] = O.f64_to_bf16(hf)
        return out

    monkeypatch.setattr(O, "swiglu_quant_fwd", fwd)
    out = O.moe_mlp_step(x, sizes, w1, w3, w2, dy, "rceil", Tcap)
    _expect_caught(lambda: check_moe(out, x, sizes, w1, w3, w2, dy, "rceil", Tcap))
