"""The oracle's MLP compositions against torch float64 autograd of the
unquantized SwiGLU MLP. MXFP8 adds ~3% relative noise per operand, so each
output must keep an SQNR far above what a swapped or transposed operand, a
wrong gate half or a dropped term would leave (those give ~0 dB)."""

import numpy as np
import torch

from oracle import mx
from quantize_grouped_gemm_amd import synth


def _sqnr_db(ref, got):
    ref = np.asarray(ref, np.float64)
    err = np.asarray(got, np.float64) - ref
    return 10 * np.log10(np.sum(ref ** 2) / max(np.sum(err ** 2), 1e-300))


def _f(b):
    return torch.from_numpy(mx.bf16_to_f64(b))


def _torch_mlp(x, w1, w3, w2, dy):
    x = x.clone().requires_grad_()
    w1 = w1.clone().requires_grad_()
    w3 = w3.clone().requires_grad_()
    w2 = w2.clone().requires_grad_()
    a = x @ w1.T
    b = x @ w3.T
    y = (torch.nn.functional.silu(a) * b) @ w2.T
    y.backward(dy)
    return y.detach(), x.grad, w1.grad, w3.grad, w2.grad


def test_dense_mlp_step_tracks_float64_autograd():
    T, D, H = 128, 128, 96
    x, w1, w3, w2, dy = [synth.bits(t) for t in synth.mlp_inputs(T, D, H, seed=4)]
    w1 = synth.bits(synth.from_bits(w1).float().mul(50).bfloat16())    # O(1) activations
    w3 = synth.bits(synth.from_bits(w3).float().mul(50).bfloat16())
    for mode in ("rceil", "floor"):
        out = mx.dense_mlp_step(x, w1, w3, w2, dy, mode)
        y, dx, dw1, dw3, dw2 = _torch_mlp(_f(x), _f(w1), _f(w3), _f(w2), _f(dy))
        assert _sqnr_db(y, mx.bf16_to_f64(out["y"])) > 20
        assert _sqnr_db(dx, mx.bf16_to_f64(out["dx"])) > 20
        assert _sqnr_db(dw2, out["dw2"]) > 20
        assert _sqnr_db(torch.cat([dw1, dw3]), out["dw13"]) > 20


def test_moe_mlp_step_tracks_float64_autograd():
    E, T, D, H = 4, 300, 64, 64
    sizes = np.array([100, 0, 170, 30])
    Tcap = synth.capacity(T, E)
    x, w1, w3, w2, dy = [synth.bits(t) for t in synth.mlp_inputs(T, D, H, E=E, seed=5)]
    w1 = synth.bits(synth.from_bits(w1).float().mul(50).bfloat16())
    w3 = synth.bits(synth.from_bits(w3).float().mul(50).bfloat16())
    for wgrad in ("mx", "hp"):
        out = mx.moe_mlp_step(x, sizes, w1, w3, w2, dy, "rceil", Tcap, wgrad=wgrad)
        start = 0
        for g in range(E):
            n = int(sizes[g])
            sl = slice(start, start + n)
            start += n
            if n == 0:
                dw2 = out["dw2"] if wgrad == "mx" else mx.bf16_to_f64(out["dw2"])
                assert np.all(dw2[g] == 0)
                continue
            y, dx, dw1, dw3, dw2 = _torch_mlp(_f(x[sl]), _f(w1[g]), _f(w3[g]), _f(w2[g]), _f(dy[sl]))
            assert _sqnr_db(y, mx.bf16_to_f64(out["y"][sl])) > 20
            assert _sqnr_db(dx, mx.bf16_to_f64(out["dx"][sl])) > 20
            got_dw2 = out["dw2"][g] if wgrad == "mx" else mx.bf16_to_f64(out["dw2"][g])
            got_dw13 = out["dw13"][g] if wgrad == "mx" else mx.bf16_to_f64(out["dw13"][g])
            assert _sqnr_db(dw2, got_dw2) > 20
            assert _sqnr_db(torch.cat([dw1, dw3]), got_dw13) > 20
