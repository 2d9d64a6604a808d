"""Stage-by-stage parity of the composed MLP training steps at the full
benchmark shapes, in the launch configuration bench.py times (the same
DenseMLP / MoEMLP objects and calls):

  dense       T=8192, D=4096, H=14336 (Llama-3-8B-shaped)
  moe_scout   E=16, D=5120, H=8192, 16384 Zipf-routed tokens, Tcap 18432
  moe_dsv3    E=32, D=7168, H=2048, 65536 Dirichlet-routed slots, Tcap 69632,
              with MXFP8 weight gradients and with wgrad_with_hp
  N1          the Scout step run again on new tokens with the experts' MXFP8
              weights reused (quantize_weights=False)
  N3          the Scout w13 forward with SwiGLU + dual quantization fused
              into its epilogue

After one step, every stage is checked on samples of its output against the
oracle applied to the GPU's own inputs to that stage (sampled rows, columns
and 32-token blocks; every expert group, pad rows and the tail included):
  quantization (and padding)   codes and scales bit-exact
  SwiGLU forward / backward    within one E4M3 code, on at most 1e-5 of the
                               sampled elements (plus one, for the sample)
  GEMMs                        within the MFMA model's bound (check_gemm):
                               bf16 within 2 ulp unless the bound exceeds it
Per-stage statistics (strict 2-ulp failures, relative Frobenius error, code
differences) are appended as JSON lines to $MX_PARITY_REPORT when it is set.
The end-to-end SQNR of y and dx against a fully oracle-fed chain (no GPU
stage inputs) is reported the same way for sampled tokens; the pages give no
threshold for it."""

import json
import os

import numpy as np
import pytest
import torch

from _helpers import bf16_host, check_gemm, code_tolerance, dev, host, hp_bound, mfma_bound, plain
from oracle import mx as O
from quantize_grouped_gemm_amd import mlp, mx, synth

pytestmark = pytest.mark.gpu

MODE = "rceil"


def _report(workload, stage, **stats):
    path = os.environ.get("MX_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"workload": workload, "stage": stage, **stats}) + "\n")


def _ix(a):
    return torch.as_tensor(np.asarray(a, np.int64), device=dev())


def _qrows(q, s, rows):
    """Codes and plain scales of selected rows of a device MX tensor
    (codes [R, C], k128 scales [C/128, R, 4])."""
    return host(q[_ix(rows)]), plain(host(s[:, _ix(rows), :]))


def _bits(t):
    return bf16_host(t)


def _f64(t):
    if t.dtype == torch.float32:
        return host(t).astype(np.float64)
    return O.bf16_to_f64(bf16_host(t))


def _eq(got, ref, what):
    bad = np.argwhere(np.asarray(got) != np.asarray(ref))
    assert len(bad) == 0, f"{what}: {len(bad)} bytes differ, first at {bad[:3].tolist()}"


class Ctx:
    def __init__(self, name, seed):
        self.name = name
        self.rng = np.random.default_rng(seed)

    def pick(self, n, k):
        return np.sort(self.rng.choice(n, min(k, n), replace=False))

    # ------------------------------------------------------------ quantization
    def quant(self, stage, x_rows_bits, x_cols_bits, q, rows, cols):
        """x_rows_bits: bf16 bits of the sampled rows of the quantized tensor
        [len(rows), C]; x_cols_bits: its sampled columns as rows [len(cols), R]."""
        if rows is not None:
            ref = O.quantize_bf16(x_rows_bits, MODE)
            got = _qrows(q["q_row"], q["s_row"], rows)
            _eq(got[0], ref["q_row"], f"{self.name} {stage} row codes")
            _eq(got[1], ref["s_row"], f"{self.name} {stage} row scales")
        if cols is not None:
            ref = O.quantize_bf16(x_cols_bits, MODE)
            got = _qrows(q["q_col"], q["s_col"], cols)
            _eq(got[0], ref["q_row"], f"{self.name} {stage} col codes")
            _eq(got[1], ref["s_row"], f"{self.name} {stage} col scales")
        _report(self.name, stage, rows=0 if rows is None else len(rows), cols=0 if cols is None else len(cols),
                bit_exact=True)

    # ------------------------------------------------------------ GEMMs
    def gemm(self, stage, got, A, B, kind):
        """got: device sample of the output; A, B: float64 dequantized
        operand rows (C = A B^T)."""
        ref = A @ B.T
        st = check_gemm(_f64(got), ref, mfma_bound(A, B), kind, f"{self.name} {stage}")
        _report(self.name, stage, **st)
        return st

    def gemm_hp(self, stage, got, G, X):
        ref = G.T @ X
        st = check_gemm(_f64(got), ref, hp_bound(G, X), "bf16", f"{self.name} {stage}")
        _report(self.name, stage, **st)
        return st

    # ------------------------------------------------------------ SwiGLU
    def codes(self, stage, got, ref):
        nd, nb, n, ns = code_tolerance(got[0], got[1], ref[0], ref[1])
        assert nb == 0, f"{self.name} {stage}: {nb} elements beyond one E4M3 code"
        assert nd <= 1e-5 * n + 1, f"{self.name} {stage}: {nd} of {n} elements differ"
        return nd, n, ns

    def swiglu_fwd(self, stage, z, H, hq, rows, blocks, h_out=None):
        """z: device [R, 2H] (the GPU's w13 output); hq: the fused kernel's
        outputs; rows: sampled rows; blocks: sampled 32-row blocks (for the
        column-wise codes)."""
        zr = _bits(z[_ix(rows)])
        h = O.swiglu_fwd(zr[:, :H], zr[:, H:])            # the sampled rows only: row-wise codes
        ref = O.quantize_bf16(h, MODE, True, False)
        nd, n, ns = self.codes(stage + " row", _qrows(hq["q_row"], hq["s_row"], rows), (ref["q_row"], ref["s_row"]))
        if h_out is not None:
            hg = O.bf16_to_f64(_bits(h_out[_ix(rows)]))
            hr = O.bf16_to_f64(h)
            ulp = np.exp2(np.maximum(np.floor(np.log2(np.where(hr != 0, np.abs(hr), 1.0))), -126) - 7)
            assert np.all(np.abs(hg - hr) <= ulp), f"{self.name} {stage}: bf16 h beyond one ulp"
        ndc = nc = 0
        sc = plain(host(hq["s_col"]))
        for b in blocks:
            zb = _bits(z[32 * b:32 * b + 32])
            r = O.swiglu_quant_fwd(zb[:, :H], zb[:, H:], MODE)
            got = (host(hq["q_col"][:, 32 * b:32 * b + 32]), sc[:, b:b + 1])
            d, m, _ = self.codes(stage + " col", got, (r["q_col"], r["s_col"]))
            ndc += d
            nc += m
        _report(self.name, stage, row_elems=n, row_diff=nd, row_scale_diff=ns, col_elems=nc, col_diff=ndc)

    def swiglu_bwd(self, stage, dh, z, H, dzq, rows, blocks, dab_out=None):
        dr, zr = _bits(dh[_ix(rows)]), _bits(z[_ix(rows)])
        dab = O.swiglu_bwd(dr, zr[:, :H], zr[:, H:])
        ref = O.quantize_bf16(dab, MODE, True, False)
        nd, n, ns = self.codes(stage + " row", _qrows(dzq["q_row"], dzq["s_row"], rows),
                               (ref["q_row"], ref["s_row"]))
        if dab_out is not None:
            g = O.bf16_to_f64(_bits(dab_out[_ix(rows)]))
            r = O.bf16_to_f64(dab)
            ulp = np.exp2(np.maximum(np.floor(np.log2(np.where(r != 0, np.abs(r), 1.0))), -126) - 7)
            assert np.all(np.abs(g - r) <= ulp), f"{self.name} {stage}: bf16 dA|dB beyond one ulp"
        ndc = nc = 0
        sc = plain(host(dzq["s_col"]))
        for b in blocks:
            db, zb = _bits(dh[32 * b:32 * b + 32]), _bits(z[32 * b:32 * b + 32])
            r = O.swiglu_quant_bwd(db, zb[:, :H], zb[:, H:], MODE)
            got = (host(dzq["q_col"][:, 32 * b:32 * b + 32]), sc[:, b:b + 1])
            d, m, _ = self.codes(stage + " col", got, (r["q_col"], r["s_col"]))
            ndc += d
            nc += m
        _report(self.name, stage, row_elems=n, row_diff=nd, row_scale_diff=ns, col_elems=nc, col_diff=ndc)


def _deq(q, s):
    return O.dequantize(q, s)


def _sqnr(ref, got):
    ref = np.asarray(ref, np.float64)
    err = np.asarray(got, np.float64) - ref
    return float(10 * np.log10(np.sum(ref * ref) / max(np.sum(err * err), 1e-300)))


# ====================================================================== dense

def _dense_stages(ctx, net, x, w13, w2, dy):
    T, D, H = net.T, net.D, net.H
    r_t, c_d, c_h, c_2h = ctx.pick(T, 48), ctx.pick(D, 48), ctx.pick(H, 48), ctx.pick(2 * H, 48)
    # quantizations of x, w13, w2, dy (rows and columns)
    ctx.quant("quant_x", _bits(x[_ix(r_t)]), _bits(x[:, _ix(c_d)].T.contiguous()), net.qx, r_t, c_d)
    ctx.quant("quant_w13", _bits(w13[_ix(c_2h)]), _bits(w13[:, _ix(c_d)].T.contiguous()), net.q13, c_2h, c_d)
    ctx.quant("quant_w2", _bits(w2[_ix(c_d)]), _bits(w2[:, _ix(c_h)].T.contiguous()), net.q2, c_d, c_h)
    ctx.quant("quant_dy", _bits(dy[_ix(r_t)]), _bits(dy[:, _ix(c_d)].T.contiguous()), net.qdy, r_t, c_d)
    # w13 forward: z = x w13^T (K = D)
    A = _deq(*_qrows(net.qx["q_row"], net.qx["s_row"], r_t))
    B = _deq(*_qrows(net.q13["q_row"], net.q13["s_row"], c_2h))
    ctx.gemm("gemm_w13_fwd", net.z[_ix(r_t)][:, _ix(c_2h)], A, B, "bf16")
    blocks = ctx.pick(T // 32, 3)
    ctx.swiglu_fwd("swiglu_fwd", net.z, H, net.hq, r_t, blocks)
    # w2 forward: y = h w2^T (K = H)
    A = _deq(*_qrows(net.hq["q_row"], net.hq["s_row"], r_t))
    B = _deq(*_qrows(net.q2["q_row"], net.q2["s_row"], c_d))
    ctx.gemm("gemm_w2_fwd", net.y[_ix(r_t)][:, _ix(c_d)], A, B, "bf16")
    # w2 input gradient: dh = dy w2 (K = D, w2 quantized along D)
    A = _deq(*_qrows(net.qdy["q_row"], net.qdy["s_row"], r_t))
    B = _deq(*_qrows(net.q2["q_col"], net.q2["s_col"], c_h))
    ctx.gemm("gemm_w2_dgrad", net.dh[_ix(r_t)][:, _ix(c_h)], A, B, "bf16")
    # w2 weight gradient: dW2 = dy^T h (K = T)
    A = _deq(*_qrows(net.qdy["q_col"], net.qdy["s_col"], c_d))
    B = _deq(*_qrows(net.hq["q_col"], net.hq["s_col"], c_h))
    ctx.gemm("gemm_w2_wgrad", net.dw2[_ix(c_d)][:, _ix(c_h)], A, B, "f32")
    ctx.swiglu_bwd("swiglu_bwd", net.dh, net.z, H, net.dzq, r_t, blocks)
    # w13 input gradient: dx = dZ w13 (K = 2H = 28672, the longest contraction)
    A = _deq(*_qrows(net.dzq["q_row"], net.dzq["s_row"], r_t))
    B = _deq(*_qrows(net.q13["q_col"], net.q13["s_col"], c_d))
    ctx.gemm("gemm_w13_dgrad", net.dx[_ix(r_t)][:, _ix(c_d)], A, B, "bf16")
    # w13 weight gradient: dW13 = dZ^T x (K = T)
    A = _deq(*_qrows(net.dzq["q_col"], net.dzq["s_col"], c_2h))
    B = _deq(*_qrows(net.qx["q_col"], net.qx["s_col"], c_d))
    ctx.gemm("gemm_w13_wgrad", net.dw13[_ix(c_2h)][:, _ix(c_d)], A, B, "f32")


def test_dense_step_full_size(gpu):
    c = synth.DENSE_MLP
    T, D, H = c["T"], c["D"], c["H"]
    x, w1, w3, w2, dy = synth.mlp_inputs(T, D, H, seed=0, device=dev())
    w13 = torch.cat([w1, w3], dim=0)
    del w1, w3
    net = mlp.DenseMLP(T, D, H, dev())
    net.step(x, w13, w2, dy)
    torch.cuda.synchronize()
    _dense_stages(Ctx("dense", 1), net, x, w13, w2, dy)


# ====================================================================== MoE

def _moe_setup(which, wgrad):
    if which == "scout":
        c = synth.MOE_SCOUT
        sizes = synth.zipf_group_sizes(c["T"], c["E"], 14)
    else:
        c = synth.MOE_DSV3
        sizes = synth.dirichlet_group_sizes(c["T"], c["E"], 0.3)
    E, T, D, H = c["E"], c["T"], c["D"], c["H"]
    Tcap = synth.capacity(T, E)
    x, w1, w3, w2, dy = synth.mlp_inputs(T, D, H, E=E, seed=0, device=dev())
    w13 = torch.cat([w1, w3], dim=1)
    del w1, w3
    sizes_d = torch.as_tensor(sizes.astype(np.int32), device=dev())
    net = mlp.MoEMLP(E, T, D, H, Tcap, dev(), wgrad=wgrad)
    return net, sizes, sizes_d, x, w13, w2, dy


def _moe_layout(sizes, Tcap):
    """Slot ends, padded row of each token and source token of each padded
    row (-1 for padding) from the oracle's padding."""
    offs, src = O.pad_groups(np.zeros((int(np.sum(sizes)), 1), np.uint16), sizes, 128, Tcap)[1:]
    pos = np.empty(int(np.sum(sizes)), np.int64)
    pos[src[src >= 0]] = np.nonzero(src >= 0)[0]
    return offs.astype(np.int64), src, pos


def _padded_rows_bits(x, src, rows):
    """bf16 bits of padded rows: x[src[r]] or zeros."""
    out = np.zeros((len(rows), x.shape[1]), np.uint16)
    s = src[rows]
    real = s >= 0
    if real.any():
        out[real] = _bits(x[_ix(s[real])])
    return out


def _padded_cols_bits(x, src, cols):
    """Sampled columns of the padded tensor, as rows [len(cols), Tcap]."""
    xc = x[:, _ix(cols)]
    full = torch.zeros((len(src), len(cols)), dtype=x.dtype, device=x.device)
    real = np.nonzero(src >= 0)[0]
    full[_ix(real)] = xc[_ix(src[real])]
    return _bits(full.T.contiguous())


def _group_rows(ctx, offs, per_group):
    """Sampled padded rows: per non-empty group, including its pad rows
    when it has some, plus rows of the tail."""
    rows = []
    start = 0
    for end in offs:
        if end > start:
            rows += list(ctx.rng.choice(np.arange(start, end), min(per_group, end - start), replace=False))
            rows.append(end - 1)             # the slot's last row (often padding)
        start = end
    return rows


def _moe_stages(ctx, net, sizes, x, w13, w2, dy, wgrad, check_weights=True):
    E, T, D, H, Tcap = net.E, net.T, net.D, net.H, net.Tcap
    offs, src, pos = _moe_layout(sizes, Tcap)
    _eq(host(net.offs), offs, f"{ctx.name} offs")
    _eq(host(net.src), src, f"{ctx.name} src_row")
    tail = np.arange(int(offs[-1]), Tcap)
    rows = np.unique(np.array(_group_rows(ctx, offs, 6) + list(ctx.rng.choice(tail, min(4, len(tail)),
                                                                                  replace=False))))
    gof = np.searchsorted(offs, rows, side="right")            # group of each padded row (E = tail)
    c_d, c_h, c_2h = ctx.pick(D, 40), ctx.pick(H, 40), ctx.pick(2 * H, 40)
    blocks = np.unique(np.concatenate([ctx.pick(Tcap // 32, 3), [offs[-1] // 32 - 1]]))
    mxw = wgrad == "mx"
    # padding + quantization of x (fused on the MXFP8 recipe)
    if mxw:
        ctx.quant("pad_quant_x", _padded_rows_bits(x, src, rows), _padded_cols_bits(x, src, c_d), net.qx, rows,
                  c_d)
    else:
        _eq(_bits(net.x_pad[_ix(rows)]), _padded_rows_bits(x, src, rows), f"{ctx.name} pad_x")
        ctx.quant("quant_x", _padded_rows_bits(x, src, rows), None, net.qx, rows, None)
    if check_weights:
        for e in ctx.pick(E, 3):
            ctx.quant(f"quant_w13[{e}]", _bits(w13[e][_ix(c_2h)]), _bits(w13[e][:, _ix(c_d)].T.contiguous()),
                      {k: v[e] for k, v in net.q13.items()}, c_2h, c_d)
            ctx.quant(f"quant_w2[{e}]", _bits(w2[e][_ix(c_d)]), _bits(w2[e][:, _ix(c_h)].T.contiguous()),
                      {k: v[e] for k, v in net.q2.items()}, c_d, c_h)

    def grouped(stage, out, a_q, w_q, cols, kind="bf16", token_order=False):
        """out rows (padded, or token order) against per-group oracle GEMMs
        on the GPU's own operands; tail rows must be zero (padded outputs)."""
        for g in range(E + 1):
            rg = rows[gof == g]
            if len(rg) == 0:
                continue
            if g == E:
                if not token_order:
                    assert torch.all(out[_ix(rg)] == 0), f"{ctx.name} {stage}: tail rows not zero"
                continue
            if token_order:
                rg = rg[src[rg] >= 0]
                if len(rg) == 0:
                    continue
                got = out[_ix(src[rg])][:, _ix(cols)]
            else:
                got = out[_ix(rg)][:, _ix(cols)]
            A = _deq(*_qrows(a_q["q_row"], a_q["s_row"], rg))
            wq = {k: v[g] for k, v in w_q.items()}
            B = _deq(*_qrows(wq["q"], wq["s"], cols))
            ctx.gemm(f"{stage} g{g}", got, A, B, kind)

    q13r = {"q": net.q13["q_row"], "s": net.q13["s_row"]}
    q13c = {"q": net.q13["q_col"], "s": net.q13["s_col"]}
    q2r = {"q": net.q2["q_row"], "s": net.q2["s_row"]}
    q2c = {"q": net.q2["q_col"], "s": net.q2["s_col"]}
    grouped("gemm_w13_fwd", net.z, net.qx, q13r, c_2h)
    ctx.swiglu_fwd("swiglu_fwd", net.z, H, net.hq, rows, blocks, h_out=net.hq.get("h"))
    grouped("gemm_w2_fwd(token order)", net.y, net.hq, q2r, c_d, token_order=True)
    if mxw:
        ctx.quant("pad_quant_dy", _padded_rows_bits(dy, src, rows), _padded_cols_bits(dy, src, c_d), net.qdy,
                  rows, c_d)
        _eq(host(net.offs2), offs, f"{ctx.name} offs (dy)")
    else:
        _eq(_bits(net.dy_pad[_ix(rows)]), _padded_rows_bits(dy, src, rows), f"{ctx.name} pad_dy")
        ctx.quant("quant_dy", _padded_rows_bits(dy, src, rows), None, net.qdy, rows, None)
    grouped("gemm_w2_dgrad", net.dh, net.qdy, q2c, c_h)
    ctx.swiglu_bwd("swiglu_bwd", net.dh, net.z, H, net.dzq, rows, blocks, dab_out=net.dzq.get("dab"))
    grouped("gemm_w13_dgrad(token order)", net.dx, net.dzq, q13c, c_d, token_order=True)
    # weight gradients: every group, sampled entries, contraction over the group's tokens
    n_d, n_h, n_2h = ctx.pick(D, 12), ctx.pick(H, 12), ctx.pick(2 * H, 12)
    start = 0
    for g in range(E):
        end = int(offs[g])
        if end == start:
            assert torch.all(net.dw2[g] == 0) and torch.all(net.dw13[g] == 0), f"{ctx.name} empty group {g}"
            continue
        if mxw:
            for stage, out, aq, bq, ra, rb in (("gemm_w2_wgrad", net.dw2, net.qdy, net.hq, n_d, n_h),
                                               ("gemm_w13_wgrad", net.dw13, net.dzq, net.qx, n_2h, n_d)):
                qa, sa = _qrows(aq["q_col"], aq["s_col"], ra)
                qb, sb = _qrows(bq["q_col"], bq["s_col"], rb)
                A = _deq(qa[:, start:end], sa[:, start // 32:end // 32])
                B = _deq(qb[:, start:end], sb[:, start // 32:end // 32])
                ctx.gemm(f"{stage} g{g}", out[g][_ix(ra)][:, _ix(rb)], A, B, "f32")
        else:
            Gd = O.bf16_to_f64(_bits(net.dy_pad[start:end][:, _ix(n_d)]))
            Hh = O.bf16_to_f64(_bits(net.hq["h"][start:end][:, _ix(n_h)]))
            ctx.gemm_hp(f"gemm_w2_wgrad_hp g{g}", net.dw2[g][_ix(n_d)][:, _ix(n_h)], Gd, Hh)
            Dz = O.bf16_to_f64(_bits(net.dzq["dab"][start:end][:, _ix(n_2h)]))
            Xp = O.bf16_to_f64(_bits(net.x_pad[start:end][:, _ix(n_d)]))
            ctx.gemm_hp(f"gemm_w13_wgrad_hp g{g}", net.dw13[g][_ix(n_2h)][:, _ix(n_d)], Dz, Xp)
        start = end


def _end_to_end(ctx, net, sizes, x, w13, w2, dy, groups=2, per_group=8, ncols=64):
    """SQNR of y and dx against a chain fed only by the oracle (bf16 inputs
    -> padding -> quantization -> GEMM -> SwiGLU -> ...), on sampled tokens
    of a few groups and sampled output columns. The forward and input-
    gradient chains are row-local, so a token's y and dx need only its own
    rows plus its expert's weights: w13 quantized along D (all rows, for z),
    w2 along D (all columns of dh), and sampled rows / columns of the others."""
    E, H = net.E, net.H
    offs, src, pos = _moe_layout(sizes, net.Tcap)
    nz = [g for g in range(E) if sizes[g] > 0]
    pick = [max(nz, key=lambda g: sizes[g]), min(nz, key=lambda g: sizes[g])][:groups]
    c_d = ctx.pick(net.D, ncols)
    ys, yg, dxs, dxg = [], [], [], []
    tok0 = np.concatenate([[0], np.cumsum(sizes)])
    for g in pick:
        tg = np.sort(ctx.rng.choice(np.arange(tok0[g], tok0[g + 1]), min(per_group, sizes[g]), replace=False))
        xb, dyb = _bits(x[_ix(tg)]), _bits(dy[_ix(tg)])
        qx = O.quantize_bf16(xb, MODE)
        q13 = O.quantize_bf16(_bits(w13[g]), MODE)                               # along D
        q2r = O.quantize_bf16(_bits(w2[g][_ix(c_d)]), MODE)                      # rows c_d, along H
        q2c = O.quantize_bf16(_bits(w2[g].T.contiguous()), MODE)                  # along D
        q13c = O.quantize_bf16(_bits(w13[g][:, _ix(c_d)].T.contiguous()), MODE)  # columns c_d, along 2H
        z = O.f64_to_bf16(O.scaled_mm(qx["q_row"], qx["s_row"], q13["q_row"], q13["s_row"]))
        qh = O.quantize_bf16(O.swiglu_fwd(z[:, :H], z[:, H:]), MODE)          # row-wise: y needs no more
        ys.append(O.scaled_mm(qh["q_row"], qh["s_row"], q2r["q_row"], q2r["s_row"]))
        qdy = O.quantize_bf16(dyb, MODE)
        dh = O.f64_to_bf16(O.scaled_mm(qdy["q_row"], qdy["s_row"], q2c["q_row"], q2c["s_row"]))
        qdz = O.quantize_bf16(O.swiglu_bwd(dh, z[:, :H], z[:, H:]), MODE)
        dxs.append(O.scaled_mm(qdz["q_row"], qdz["s_row"], q13c["q_row"], q13c["s_row"]))
        yg.append(_f64(net.y[_ix(tg)][:, _ix(c_d)]))
        dxg.append(_f64(net.dx[_ix(tg)][:, _ix(c_d)]))
    r = {"y": _sqnr(np.concatenate(ys), np.concatenate(yg)), "dx": _sqnr(np.concatenate(dxs), np.concatenate(dxg)),
         "groups": [int(g) for g in pick], "tokens_per_group": per_group, "columns": int(ncols)}
    _report(ctx.name, "end_to_end_sqnr_db", **r)
    return r


@pytest.mark.parametrize("which,wgrad", [("scout", "mx"), ("dsv3", "mx"), ("dsv3", "hp")])
def test_moe_step_full_size(gpu, which, wgrad):
    net, sizes, sizes_d, x, w13, w2, dy = _moe_setup(which, wgrad)
    net.step(x, sizes_d, w13, w2, dy)
    torch.cuda.synchronize()
    assert int(net.err.item()) == 0
    ctx = Ctx(f"moe_{which}_{wgrad}", 2)
    _moe_stages(ctx, net, sizes, x, w13, w2, dy, wgrad)
    r = _end_to_end(ctx, net, sizes, x, w13, w2, dy)
    assert r["y"] > 20 and r["dx"] > 20       # a swapped operand or half gives about 0 dB


def test_moe_cached_weights_step_full_size(gpu):
    """N1: the second micro-batch of an optimizer step, on new tokens, with
    the experts' MXFP8 weights from the first: the cached codes still match
    the oracle's quantization of the weights, and every stage of the second
    step matches the oracle on its own inputs."""
    net, sizes, sizes_d, x, w13, w2, dy = _moe_setup("scout", "mx")
    net.step(x, sizes_d, w13, w2, dy)
    c = synth.MOE_SCOUT
    x2, _, _, _, dy2 = synth.mlp_inputs(c["T"], c["D"], c["H"], E=None, seed=7, device=dev())
    net.step(x2, sizes_d, w13, w2, dy2, quantize_weights=False)
    torch.cuda.synchronize()
    assert int(net.err.item()) == 0
    _moe_stages(Ctx("moe_scout_cached_weights", 3), net, sizes, x2, w13, w2, dy2, "mx", check_weights=True)


def test_fused_w13_swiglu_full_size(gpu):
    """N3: the Scout w13 forward with SwiGLU + dual quantization in its
    epilogue. z against the oracle's grouped GEMM on the GPU's operands; h's
    codes (both directions) against the oracle's SwiGLU + quantization of the
    GPU's own z."""
    net, sizes, sizes_d, x, w13, w2, dy = _moe_setup("scout", "mx")
    E, Tcap, H = net.E, net.Tcap, net.H
    q = mx.pad_quantize(x, sizes_d, Tcap, MODE, True, False)
    qw = mx.quantize(w13, MODE)
    fo = mx.grouped_mm_swiglu_fwd(q["q_row"], q["s_row"], qw["q_row"], qw["s_row"], q["offs"], MODE)
    torch.cuda.synchronize()
    ctx = Ctx("fused_w13_swiglu", 4)
    offs, src, pos = _moe_layout(sizes, Tcap)
    tail = np.arange(int(offs[-1]), Tcap)
    rows = np.unique(np.array(_group_rows(ctx, offs, 6) + list(ctx.rng.choice(tail, 4, replace=False))))
    gof = np.searchsorted(offs, rows, side="right")
    cols = ctx.pick(2 * H, 48)
    for g in range(E + 1):
        rg = rows[gof == g]
        if len(rg) == 0:
            continue
        if g == E:
            assert torch.all(fo["z"][_ix(rg)] == 0)
            continue
        A = _deq(*_qrows(q["q_row"], q["s_row"], rg))
        B = _deq(*_qrows(qw["q_row"][g], qw["s_row"][g], cols))
        ctx.gemm(f"fused z g{g}", fo["z"][_ix(rg)][:, _ix(cols)], A, B, "bf16")
    blocks = np.unique(np.concatenate([ctx.pick(Tcap // 32, 3), [offs[-1] // 32 - 1]]))
    ctx.swiglu_fwd("fused swiglu", fo["z"], H, fo, rows, blocks)
