"""GPU parity of group padding/unpadding (bit-exact) and of the composed
MXFP8 MLP steps (dense and routed experts) against the oracle's
compositions."""

import numpy as np
import pytest
import torch

from _helpers import bf16_host, dev, host, plain, to_dev
from oracle import mx as O
from quantize_grouped_gemm_amd import mlp, mx, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("sizes", [[3, 0, 130, 1], [128, 128], [0, 0, 5], [0], [700, 0, 0, 300, 129]])
def test_pad_unpad(gpu, sizes):
    sizes = np.array(sizes, np.int32)
    T = int(sizes.sum())
    Tcap = synth.capacity(T, len(sizes))
    rng = np.random.default_rng(T)
    xb = rng.integers(0, 1 << 16, (T, 96)).astype(np.uint16)
    x = to_dev(xb.view(np.int16)).view(torch.bfloat16) if T else torch.empty((0, 96), dtype=torch.bfloat16,
                                                                            device=dev())
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    x_pad, offs, src = mx.pad_groups(x, to_dev(sizes), Tcap, dev_err=err)
    rp, ro, rs = O.pad_groups(xb, sizes, 128, Tcap)
    np.testing.assert_array_equal(host(offs), ro)
    np.testing.assert_array_equal(host(src), rs)
    np.testing.assert_array_equal(bf16_host(x_pad), rp)
    assert int(err.item()) == 0
    y = torch.full((T, 96), 7.0, dtype=torch.bfloat16, device=dev())
    mx.unpad_groups(x_pad, src, T, out=y)
    np.testing.assert_array_equal(bf16_host(y), xb)


@pytest.mark.parametrize("layout", ["plain", "k128"])
@pytest.mark.parametrize("sizes,D", [([3, 0, 130, 1], 128), ([128, 128], 256), ([0, 0, 5], 128), ([0], 128),
                                     ([700, 0, 0, 300, 129], 384), ([257], 128)])
def test_pad_quantize(gpu, sizes, D, layout):
    """Fused pad + quantize: bytes equal the oracle's pad-then-quantize, and
    offs / src_row equal the padding kernel's."""
    sizes = np.array(sizes, np.int32)
    T = int(sizes.sum())
    Tcap = synth.capacity(T, len(sizes))
    g = synth.generator(T + D)
    xb = synth.bits(synth.normal_bf16((max(T, 1), D), 1.0, g))[:T]
    xb[T // 2: T // 2 + 1, :32] = 0          # a zero block inside a group
    x = to_dev(xb.view(np.int16)).view(torch.bfloat16) if T else torch.empty((0, D), dtype=torch.bfloat16,
                                                                            device=dev())
    for mode in ("rceil", "floor"):
        for row, col in ((True, False), (False, True), (True, True)):
            err = torch.zeros(1, dtype=torch.int32, device=dev())
            got = mx.pad_quantize(x, to_dev(sizes), Tcap, mode, row, col, layout=layout, dev_err=err)
            ref = O.pad_quantize(xb, sizes, 128, Tcap, mode, row, col)
            np.testing.assert_array_equal(host(got["offs"]), ref["offs"])
            np.testing.assert_array_equal(host(got["src_row"]), ref["src_row"])
            for k in (["q_row", "s_row"] if row else []) + (["q_col", "s_col"] if col else []):
                v = host(got[k])
                if k[0] == "s" and layout == "k128":
                    v = plain(v)
                np.testing.assert_array_equal(v, ref[k], err_msg=f"{k} {mode}")
            assert int(err.item()) == 0


def test_pad_quantize_full_size_equals_unfused(gpu):
    """At the MoE Scout shape (T=16384 tokens of dim 5120 over 16 experts),
    the fused path writes the same bytes as padding then quantizing."""
    E, T, D = 16, 16384, 5120
    sizes = synth.zipf_group_sizes(T, E, 14).astype(np.int32)
    Tcap = synth.capacity(T, E)
    g = synth.generator(5, device=dev())
    x = synth.normal_bf16((T, D), 1.0, g, device=dev())
    sz = to_dev(sizes)
    fused = mx.pad_quantize(x, sz, Tcap, "rceil", True, True)
    x_pad, offs, src = mx.pad_groups(x, sz, Tcap)
    ref = mx.quantize(x_pad, "rceil", True, True)
    assert torch.equal(fused["offs"], offs) and torch.equal(fused["src_row"], src)
    for k in ("q_row", "s_row", "q_col", "s_col"):
        assert torch.equal(fused[k], ref[k]), k


def test_pad_invalid_sizes_flag(gpu):
    x = torch.zeros((10, 32), dtype=torch.bfloat16, device=dev())
    for sizes, Tcap in (([5, 6], 256), ([-1, 11], 256), ([100, 100], 128)):
        err = torch.zeros(1, dtype=torch.int32, device=dev())
        mx.pad_groups(x, to_dev(np.array(sizes, np.int32)), Tcap, dev_err=err)
        torch.cuda.synchronize()
        assert int(err.item()) & 2, sizes


def _sqnr(ref, got):
    ref = np.asarray(ref, np.float64)
    err = np.asarray(got, np.float64) - ref
    return 10 * np.log10(np.sum(ref ** 2) / max(np.sum(err ** 2), 1e-300))


def test_dense_mlp_step_matches_oracle(gpu):
    T, D, H = 256, 256, 384
    x, w1, w3, w2, dy = synth.mlp_inputs(T, D, H, seed=2)
    net = mlp.DenseMLP(T, D, H, dev())
    w13 = torch.cat([w1, w3]).to(dev())
    net.step(x.to(dev()), w13, w2.to(dev()), dy.to(dev()))
    ref = O.dense_mlp_step(*[synth.bits(t) for t in (x, w1, w3, w2, dy)], "rceil")
    # whole-step comparison by SQNR (each stage is checked against the
    # oracle on its own inputs in test_gpu_mlp_stages.py); z comes from
    # bit-exact operands, so it agrees far more closely than the later stages
    assert _sqnr(O.bf16_to_f64(ref["z"]), O.bf16_to_f64(bf16_host(net.z))) > 50
    for k, got in (("y", net.y), ("dh", net.dh), ("dx", net.dx)):
        assert _sqnr(O.bf16_to_f64(ref[k]), O.bf16_to_f64(bf16_host(got))) > 35, k
    assert _sqnr(ref["dw2"], host(net.dw2)) > 35
    assert _sqnr(ref["dw13"], host(net.dw13)) > 35


@pytest.mark.parametrize("wgrad", ["mx", "hp"])
def test_moe_mlp_step_matches_oracle(gpu, wgrad):
    E, T, D, H = 4, 600, 256, 128
    sizes = np.array([250, 0, 300, 50], np.int32)
    Tcap = synth.capacity(T, E)
    x, w1, w3, w2, dy = synth.mlp_inputs(T, D, H, E=E, seed=3)
    net = mlp.MoEMLP(E, T, D, H, Tcap, dev(), wgrad=wgrad)
    w13 = torch.cat([w1, w3], dim=1).to(dev())
    net.step(x.to(dev()), to_dev(sizes), w13, w2.to(dev()), dy.to(dev()))
    ref = O.moe_mlp_step(*[synth.bits(t) for t in (x,)], sizes, *[synth.bits(t) for t in (w1, w3, w2, dy)],
                         "rceil", Tcap, wgrad=wgrad)
    torch.cuda.synchronize()
    assert int(net.err.item()) == 0
    np.testing.assert_array_equal(host(net.offs), ref["offs"])
    for k, got in (("y", net.y), ("dx", net.dx)):
        assert _sqnr(O.bf16_to_f64(ref[k]), O.bf16_to_f64(bf16_host(got))) > 35, k
    if wgrad == "mx":
        dw2, dw13 = host(net.dw2), host(net.dw13)
        rdw2, rdw13 = ref["dw2"], ref["dw13"]
    else:
        dw2, dw13 = O.bf16_to_f64(bf16_host(net.dw2)), O.bf16_to_f64(bf16_host(net.dw13))
        rdw2, rdw13 = O.bf16_to_f64(ref["dw2"]), O.bf16_to_f64(ref["dw13"])
    assert np.all(dw2[1] == 0) and np.all(dw13[1] == 0)
    for g in (0, 2, 3):
        assert _sqnr(rdw2[g], dw2[g]) > 35
        assert _sqnr(rdw13[g], dw13[g]) > 35


def test_moe_mlp_step_fp8_rowwise_matches_oracle(gpu):
    """The FP8 row-scaled recipe of the routed-experts step against the
    oracle's same composition (quantize_fp8_bf16 throughout)."""
    E, T, D, H = 4, 600, 256, 128
    sizes = np.array([250, 0, 300, 50], np.int32)
    Tcap = synth.capacity(T, E)
    x, w1, w3, w2, dy = synth.mlp_inputs(T, D, H, E=E, seed=6)
    net = mlp.MoEMLP(E, T, D, H, Tcap, dev(), recipe="fp8_rowwise")
    w13 = torch.cat([w1, w3], dim=1).to(dev())
    net.step(x.to(dev()), to_dev(sizes), w13, w2.to(dev()), dy.to(dev()))
    ref = O.moe_mlp_step(synth.bits(x), sizes, *[synth.bits(t) for t in (w1, w3, w2, dy)], "rceil", Tcap,
                         recipe="fp8_rowwise")
    torch.cuda.synchronize()
    assert int(net.err.item()) == 0
    for k, got in (("y", net.y), ("dx", net.dx)):
        assert _sqnr(O.bf16_to_f64(ref[k]), O.bf16_to_f64(bf16_host(got))) > 35, k
    dw2, dw13 = host(net.dw2), host(net.dw13)
    assert np.all(dw2[1] == 0) and np.all(dw13[1] == 0)
    for g in (0, 2, 3):
        assert _sqnr(ref["dw2"][g], dw2[g]) > 35
        assert _sqnr(ref["dw13"][g], dw13[g]) > 35


def test_moe_step_with_cached_weight_quantization(gpu):
    """Micro-batches of one optimizer step share one dual quantization of
    the expert weights: a step that reuses the cached MXFP8 weights gives the
    same bytes as a step that quantizes them again."""
    E, T, D, H = 4, 600, 256, 128
    sizes = to_dev(np.array([250, 0, 300, 50], np.int32))
    Tcap = synth.capacity(T, E)
    x, w1, w3, w2, dy = synth.mlp_inputs(T, D, H, E=E, seed=4)
    x2, _, _, _, dy2 = synth.mlp_inputs(T, D, H, E=E, seed=5)
    w13 = torch.cat([w1, w3], dim=1).to(dev())
    w2 = w2.to(dev())
    cached = mlp.MoEMLP(E, T, D, H, Tcap, dev())
    cached.step(x.to(dev()), sizes, w13, w2, dy.to(dev()))
    cached.step(x2.to(dev()), sizes, w13, w2, dy2.to(dev()), quantize_weights=False)
    fresh = mlp.MoEMLP(E, T, D, H, Tcap, dev())
    fresh.step(x2.to(dev()), sizes, w13, w2, dy2.to(dev()))
    for k in ("y", "dx", "dw13", "dw2"):
        assert torch.equal(getattr(cached, k), getattr(fresh, k)), k
