"""The entry points under HIP graph capture: no call allocates, syncs or reads
device memory on the host, so a captured chain replays with whatever the
device buffers hold at replay time, routing included. Each replay follows
eager work on the same buffers (new inputs, new group sizes written on the
device) and must equal the same chain run eagerly, bit for bit."""

import numpy as np
import pytest
import torch

from _helpers import dev, to_dev
from quantize_grouped_gemm_amd import mx, synth

pytestmark = pytest.mark.gpu

REPLAYS = 4


def test_graph_linear_forward(gpu):
    """Quantize x and W, then the scaled GEMM (the linear override's
    forward), captured once and replayed on new x and W."""
    x, w = synth.linear_inputs(seed=0, device=dev())
    qx = mx.quantize(x, "rceil")
    qw = mx.quantize(w, "rceil")
    out = mx.scaled_mm(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mx.quantize(x, "rceil", out=qx)
        mx.quantize(w, "rceil", out=qw)
        mx.scaled_mm(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"], out=out)
    for i in range(REPLAYS):
        xn, wn = synth.linear_inputs(seed=100 + i, device=dev())
        x.copy_(xn)
        w.copy_(wn)
        g.replay()
        torch.cuda.synchronize()
        ex = mx.quantize(xn, "rceil")
        ew = mx.quantize(wn, "rceil")
        ref = mx.scaled_mm(ex["q_row"], ex["s_row"], ew["q_row"], ew["s_row"])
        torch.cuda.synchronize()
        for k in ("q_row", "s_row"):
            assert torch.equal(qx[k], ex[k]) and torch.equal(qw[k], ew[k]), f"replay {i}: {k}"
        assert torch.equal(out, ref), f"replay {i}: output"


def test_graph_routed_forward_with_changing_routing(gpu):
    """The routed-experts MLP forward (padded quantization of the tokens,
    w13 grouped GEMM, fused SwiGLU + dual quantization, w2 grouped GEMM
    written in token order), captured once. Between replays the token values
    and the per-expert group sizes (device int32, same total) change, empty
    experts included; each replay equals the eager chain on that routing."""
    E, T, D, H = 4, 520, 256, 128
    Tcap = synth.capacity(T, E)
    x, w1, w3, w2, _ = synth.mlp_inputs(T, D, H, E=E, seed=0)
    qw13 = mx.quantize(torch.cat([w1, w3], 1).to(dev()), "rceil")
    qw2 = mx.quantize(w2.to(dev()), "rceil")
    xd = x.to(dev())
    sizes = to_dev(np.array([200, 0, 300, 20], np.int32))

    def chain(xt, sz, out=None):
        out = out or {}
        pq = mx.pad_quantize(xt, sz, Tcap, "rceil", out=out.get("pq"))
        z = mx.grouped_mm_fwd(pq["q_row"], pq["s_row"], qw13["q_row"], qw13["s_row"], pq["offs"],
                              out=out.get("z"))
        hq = mx.swiglu_quant_fwd(z[:, :H], z[:, H:], "rceil", out=out.get("hq"))
        y = mx.grouped_mm_fwd_unpad(hq["q_row"], hq["s_row"], qw2["q_row"], qw2["s_row"], pq["offs"], sz, T,
                                    out=out.get("y"))
        return {"pq": pq, "z": z, "hq": hq, "y": y}

    bufs = chain(xd, sizes)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain(xd, sizes, bufs)
    rng = np.random.default_rng(5)
    routings = [[0, 260, 0, 260], [520, 0, 0, 0], [1, 129, 255, 135], [130, 130, 130, 130]]
    for i, r in enumerate(routings[:REPLAYS]):
        assert sum(r) == T
        xn = torch.from_numpy(rng.standard_normal((T, D)).astype(np.float32)).to(torch.bfloat16).to(dev())
        xd.copy_(xn)
        sizes.copy_(to_dev(np.array(r, np.int32)))
        g.replay()
        torch.cuda.synchronize()
        ref = chain(xn, to_dev(np.array(r, np.int32)))
        torch.cuda.synchronize()
        assert torch.equal(bufs["pq"]["offs"], ref["pq"]["offs"]), f"replay {i}: offsets"
        for k in ("q_row", "s_row"):
            assert torch.equal(bufs["pq"][k], ref["pq"][k]), f"replay {i}: x {k}"
        assert torch.equal(bufs["z"], ref["z"]), f"replay {i}: z"
        for k in ("q_row", "s_row", "q_col", "s_col"):
            assert torch.equal(bufs["hq"][k], ref["hq"][k]), f"replay {i}: h {k}"
        assert torch.equal(bufs["y"], ref["y"]), f"replay {i}: y"
