"""Benchmark of the MXFP8 training hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Default workload: one training step (forward + backward) of the routed-
experts MXFP8 SwiGLU MLP at one GPU's share of a Llama4-Scout-like MoE
(16 experts, dim 5120, expert hidden 8192, 16384 top-1 tokens with Zipf(1.1)
group sizes, two experts empty, groups padded to 128). A step runs every
kernel of the path: MX quantization of the activations (with the group
padding fused in) and of both weights (row- and column-wise), grouped MXFP8
GEMMs (forward, input and weight gradients; the two that produce y and dx
write token order, so unpadding is fused in), and the fused SwiGLU + dual
quantization boundary forward and backward. Inputs are seeded synthetic
tensors resident in HBM before timing starts.

Prints one JSON line. `value` is tokens per second of the whole step;
`roofline` is for the dominant kernel (the grouped MXFP8 GEMM), with its
useful flops per launch divided by its average launch time from HIP events
recorded around each launch inside the timed steps; `cpu_baseline` times the
CPU oracle on a bounded slice of the same workload. Secondary figures (the
other workloads, per-kernel times) go under `components`.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MXFP8 = 5.0e15      # MI355X dense MXFP8 / FP8 MFMA, FLOP/s
PEAK_BF16 = 2.5e15       # dense BF16 MFMA
PEAK_HBM = 8.0e12        # HBM3E bytes/s

WORKLOADS = ("moe_scout", "moe_scout_fp8", "moe_dsv3", "moe_dsv3_hp", "dense", "quant", "linear", "copy",
             "vendor_gemm")

# HBM traffic of the dominant kernel, from rocprofv3 FETCH_SIZE / WRITE_SIZE
# passes scaled by a 1 GiB copy (see the file); used only while the kernel's
# sources are the ones the counters were taken on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_gemm_grouped_moe_scout_traffic.md")
GEMM_SOURCES = ("quantize_grouped_gemm_amd/csrc/mx_gemm.hip", "quantize_grouped_gemm_amd/csrc/mx_kernels.h",
                "quantize_grouped_gemm_amd/csrc/mx_device.h", "quantize_grouped_gemm_amd/csrc/mx_tile.h",
                "quantize_grouped_gemm_amd/build.py")


def gemm_source_hash():
    """Hash of the GEMM kernel's code and build flags. Comments and blank
    lines of the C++ sources are left out, so editing a comment keeps the
    counters taken on the same code valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            text = f.read()
        if not rel.endswith(".py"):
            code = re.sub(rb"/\*.*?\*/", b"", text, flags=re.S)
            code = re.sub(rb"//[^\n]*", b"", code)
            text = b"\n".join(line.rstrip() for line in code.split(b"\n") if line.strip())
        h.update(text)
    return h.hexdigest()


# MFMA-busy fraction and engine clock of the dominant kernel, from a
# rocprofv3 pass over SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE (see the
# file); same source-hash rule.
MFMA_FILE = os.path.join(ROOT, "profiles", "gemm_mfma_utilization_moe_scout.md")


def _profile_values(path):
    """The "key: value" lines of a profile summary, or None if its counters
    were taken on other GEMM sources."""
    try:
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith(("#", " ", "|", "-")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        return kv if kv.get("source_sha256") == gemm_source_hash() else None
    except OSError:
        return None


def _measured_traffic():
    """Bytes per launch of k_gemm_grouped on the default workload, or None if
    the counters were taken on other kernel sources."""
    try:
        return float(_profile_values(TRAFFIC_FILE)["traffic_bytes_per_launch"])
    except (TypeError, KeyError, ValueError):
        return None


def _measured_mfma():
    """MFMA-busy fraction and engine clock (GHz) of k_gemm_grouped's launches
    on the default workload, or None."""
    try:
        kv = _profile_values(MFMA_FILE)
        return {"mfma_busy": float(kv["mfma_busy_per_launch"]), "sclk_ghz": float(kv["sclk_ghz_per_launch"])}
    except (TypeError, KeyError, ValueError):
        return None


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="moe_scout", choices=WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-components", action="store_true",
                    help="skip the secondary workloads (for profiling runs)")
    return ap.parse_args()


def _ensure_lib():
    from quantize_grouped_gemm_amd import mx
    if not os.path.exists(mx.LIB_PATH):
        from quantize_grouped_gemm_amd import build
        build.build()
    mx.lib()


def _build_workload(name, torch, dev, wgrad_dtype=None):
    """Returns (net, args, stages, tokens, description, config). wgrad_dtype:
    dW dtype of the MoE weight gradients (float32 unless given)."""
    import numpy as np
    from quantize_grouped_gemm_amd import mlp, synth
    if name.startswith("moe"):
        recipe = "mxfp8"
        if name in ("moe_scout", "moe_scout_fp8"):
            c = synth.MOE_SCOUT
            sizes = synth.zipf_group_sizes(c["T"], c["E"], 14)
            wgrad = "mx"
            desc = "Llama4-Scout-like routed experts, one GPU's share"
            if name == "moe_scout_fp8":
                recipe = "fp8_rowwise"
                desc += ", FP8 with one scale per row"
        else:
            c = synth.MOE_DSV3
            sizes = synth.dirichlet_group_sizes(c["T"], c["E"], 0.3)
            wgrad = "hp" if name.endswith("hp") else "mx"
            desc = "DeepSeek-V3-like fine-grained experts, one GPU's share"
        E, T, D, H = c["E"], c["T"], c["D"], c["H"]
        Tcap = synth.capacity(T, E)
        x, w1, w3, w2, dy = synth.mlp_inputs(T, D, H, E=E, seed=0, device=dev)
        w13 = torch.cat([w1, w3], dim=1)
        del w1, w3
        sizes_d = torch.from_numpy(sizes.astype(np.int32)).to(dev)
        dwt = wgrad_dtype or torch.float32
        net = mlp.MoEMLP(E, T, D, H, Tcap, dev, wgrad=wgrad, recipe=recipe, wgrad_dtype=dwt)
        args = (x, sizes_d, w13, w2, dy)
        fmt = "FP8 row-scaled" if recipe == "fp8_rowwise" else "MXFP8"
        config = {"workload": f"{name}: {fmt} SwiGLU MoE MLP fwd+bwd, E={E} D={D} H={H} T={T} "
                              f"(padded to 128, Tcap={Tcap}), wgrad={'bf16 wgrad_with_hp' if wgrad == 'hp' else 'mxfp8'}"
                              + (", dW bf16" if dwt == torch.bfloat16 else ""),
                  "experts": E, "dim": D, "hidden": H, "tokens": T, "capacity": Tcap,
                  "group_sizes": [int(v) for v in sizes], "scale_mode": "rceil", "description": desc}
        return net, args, net.stages(*args), T, config
    if name == "dense":
        c = synth.DENSE_MLP
        T, D, H = c["T"], c["D"], c["H"]
        x, w1, w3, w2, dy = synth.mlp_inputs(T, D, H, seed=0, device=dev)
        w13 = torch.cat([w1, w3], dim=0)
        net = mlp.DenseMLP(T, D, H, dev)
        args = (x, w13, w2, dy)
        config = {"workload": f"dense: MXFP8 SwiGLU MLP fwd+bwd (Llama-3-8B-shaped) T={T} D={D} H={H}",
                  "tokens": T, "dim": D, "hidden": H, "scale_mode": "rceil"}
        return net, args, net.stages(*args), T, config
    raise ValueError(name)


def _time_stages(stages, steps, warmup, torch):
    """Runs warmup steps, then `steps` timed steps (bare launches, bracketed
    by synchronizations: the step time), then `steps` more with a HIP event
    pair around every launch (the per-stage times). Recording the events
    between launches costs about 1% of the step, so it stays out of the
    timed region. Returns (step_seconds, per-stage mean seconds)."""
    for _ in range(warmup):
        for st in stages:
            st.fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for st in stages:
            st.fn()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in stages] for _ in range(steps)]
    for k in range(steps):
        for i, st in enumerate(stages):
            ev[k][i][0].record()
            st.fn()
            ev[k][i][1].record()
    torch.cuda.synchronize()
    per = [sum(ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(steps)) / steps / 1e3
           for i in range(len(stages))]
    return wall, per


def _kernel_table(stages, per, gemm_bytes=None):
    """Per-kernel time, rate and roofline. gemm_bytes: algorithmic HBM bytes
    of each GEMM stage (operands read once, output written once); a GEMM
    kernel is then also priced against max(flops / MFMA peak, bytes / HBM
    peak), the bound its launches cannot beat."""
    gemm_bytes = gemm_bytes or {}
    table = {}
    for st, t in zip(stages, per):
        e = table.setdefault(st.kernel, {"launches": 0, "seconds": 0.0, "flops": 0.0, "bytes": 0.0,
                                         "floor": 0.0, "mfma_floor": 0.0, "hbm_floor": 0.0})
        e["launches"] += 1
        e["seconds"] += t
        e["flops"] += st.flops
        e["bytes"] += st.bytes
        if st.flops:
            peak = PEAK_BF16 if st.kernel.endswith("_hp") else PEAK_MXFP8
            mf, hb = st.flops / peak, gemm_bytes.get(st.name, 0.0) / PEAK_HBM
            e["mfma_floor"] += mf
            e["hbm_floor"] += hb
            e["floor"] += max(mf, hb)
    out = {}
    for k, e in table.items():
        r = {"launches_per_step": e["launches"], "ms_per_step": round(e["seconds"] * 1e3, 4),
             "avg_launch_us": round(e["seconds"] / e["launches"] * 1e6, 2)}
        if e["flops"]:
            r["useful_tflops"] = round(e["flops"] / e["seconds"] / 1e12, 1)
            r["mfma_floor_us"] = round(e["mfma_floor"] / e["launches"] * 1e6, 1)
            r["hbm_floor_us"] = round(e["hbm_floor"] / e["launches"] * 1e6, 1)
            r["roofline_frac"] = round(e["floor"] / e["seconds"], 4)
        if e["bytes"]:
            r["gbps"] = round(e["bytes"] / e["seconds"] / 1e9, 1)
        out[k] = r
    return out, table


def _roofline_gemm(table, kernel, peak, traffic=None, padded_ratio=None, mfma=None):
    """Useful flops (real tokens) per launch over the launch time; with
    padded_ratio (padded tokens / real tokens) also the rate over the
    padded groups the kernel multiplies. mfma: the profiled MFMA-busy
    fraction and engine clock of the kernel (the published peak assumes the
    2.4 GHz peak clock)."""
    e = table[kernel]
    achieved = e["flops"] / e["seconds"]       # per-launch flops / per-launch time, averaged
    r = {"kernel": kernel, "bound": "mfma", "achieved": round(achieved / 1e12, 1), "peak": peak / 1e12,
         "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
         "per_launch_flops": e["flops"] / e["launches"], "avg_launch_us": round(e["seconds"] / e["launches"] * 1e6, 2)}
    if padded_ratio is not None:
        r["padded_tflops"] = round(achieved * padded_ratio / 1e12, 1)
    if traffic is not None:
        r["traffic_unit"] = "bytes per launch (HBM, rocprofv3 FETCH_SIZE x2 + WRITE_SIZE)"
    if mfma is not None:
        r["mfma_busy_profiled"] = mfma["mfma_busy"]
        r["sclk_ghz_profiled"] = mfma["sclk_ghz"]
    return r


def _padded_ratio(config):
    """Tokens after padding each group to 128, over real tokens (MoE only)."""
    sizes = config.get("group_sizes")
    if not sizes:
        return None
    return sum(-(-n // 128) * 128 for n in sizes) / sum(sizes)


def _quant_component(torch, dev, reps=10):
    """MX dual (row + column) and row-only quantization of the [32768, 7168]
    stress tensor, RCEIL. A 1 GiB buffer is read between launches, so the
    tensor comes from HBM, not the last-level cache. The flush reads rather
    than writes: a written buffer leaves its dirty lines in L2 and the
    last-level cache, and the timed kernel would pay for their write-back."""
    from quantize_grouped_gemm_amd import mx, synth
    R, C = synth.STRESS_SHAPE
    x = synth.stress_tensor(R, C, seed=0, device=dev)
    flush = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    res = {}
    for label, row, col in (("dual", True, True), ("rowwise", True, False), ("colwise", False, True)):
        out = mx.quantize(x, "rceil", row, col)
        nbytes = R * C * (2 + (int(row) + int(col)) * (1 + 1 / 32))
        ts = []
        for _ in range(reps):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            mx.quantize(x, "rceil", row, col, out=out)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / 1e3)
        t = sorted(ts)[len(ts) // 2]
        res[label] = {"us": round(t * 1e6, 1), "gbps": round(nbytes / t / 1e9, 1),
                      "frac_hbm": round(nbytes / t / PEAK_HBM, 3)}
    # dequantization of the row-wise codes (the round trip's second half):
    # 1 + 1/32 B read, 2 B (bf16) or 4 B (float32) written per element
    q = mx.quantize(x, "rceil", True, False)
    for label, dt, esz in (("dequant_bf16", torch.bfloat16, 2), ("dequant_f32", torch.float32, 4)):
        out = mx.dequantize(q["q_row"], q["s_row"], dt)
        nbytes = R * C * (1 + 1 / 32 + esz)
        ts = []
        for _ in range(reps):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            mx.dequantize(q["q_row"], q["s_row"], dt, out=out)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / 1e3)
        t = sorted(ts)[len(ts) // 2]
        res[label] = {"us": round(t * 1e6, 1), "gbps": round(nbytes / t / 1e9, 1),
                      "frac_hbm": round(nbytes / t / PEAK_HBM, 3)}
        del out
    del x, flush, q
    return res


def _linear_component(torch, dev, reps=50):
    from quantize_grouped_gemm_amd import mx, synth
    x, w = synth.linear_inputs(seed=0, device=dev)
    qx = mx.quantize(x, "rceil")
    qw = mx.quantize(w, "rceil")
    out = mx.scaled_mm(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        mx.quantize(x, "rceil", out=qx)
        mx.quantize(w, "rceil", out=qw)
        mx.scaled_mm(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"], out=out)
    b.record()
    torch.cuda.synchronize()
    host_loop_us = a.elapsed_time(b) / reps * 1e3
    # the same three launches captured in a HIP graph and replayed; for a
    # graph this small, one replay has cost more than the three direct
    # launches (about 44 against 31 us), so the graph is a capture check
    # here, not a speed-up
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mx.quantize(x, "rceil", out=qx)
        mx.quantize(w, "rceil", out=qw)
        mx.scaled_mm(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"], out=out)
    g.replay()
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    graph_us = a.elapsed_time(b) / reps * 1e3
    return {"us_per_linear_fwd": round(host_loop_us, 2), "us_per_linear_fwd_graph": round(graph_us, 2),
            "shape": "256x256x512, bf16 out",
            "note": "x and W quantized row-wise, then the scaled GEMM: three launches; the first figure is a "
                    "Python loop of calls, the second the same launches replayed from a HIP graph (the replay "
                    "overhead of a three-node graph exceeds that of three direct launches)"}


def _fused_swiglu_component(torch, dev, reps=5):
    """The MoE Scout w13 forward with SwiGLU + dual quantization fused into
    its epilogue, against the grouped forward followed by the standalone
    fused SwiGLU kernel (what the step runs)."""
    import numpy as np
    from quantize_grouped_gemm_amd import mx, synth
    c = synth.MOE_SCOUT
    E, T, D, H = c["E"], c["T"], c["D"], c["H"]
    sizes = synth.zipf_group_sizes(T, E, 14)
    Tcap = synth.capacity(T, E)
    offs = torch.tensor(np.cumsum(-(-sizes // 128) * 128).astype(np.int32), device=dev)
    g = synth.generator(0, dev)
    x = synth.normal_bf16((Tcap, D), 1.0, g, dev)
    w = synth.normal_bf16((E, 2 * H, D), 0.02, g, dev)
    qx, qw = mx.quantize(x, "rceil"), mx.quantize(w, "rceil")
    del x, w
    fo = mx.grouped_mm_swiglu_fwd(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"], offs)
    z = fo["z"]
    so = mx.swiglu_quant_fwd(z[:, :H], z[:, H:], "rceil")

    def timed(f):
        f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            f()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e3

    fused = timed(lambda: mx.grouped_mm_swiglu_fwd(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"], offs,
                                                   out=fo))
    gemm = timed(lambda: mx.grouped_mm_fwd(qx["q_row"], qx["s_row"], qw["q_row"], qw["s_row"], offs, out=z))
    swi = timed(lambda: mx.swiglu_quant_fwd(z[:, :H], z[:, H:], "rceil", out=so))
    return {"fused_us": round(fused, 1), "unfused_gemm_us": round(gemm, 1), "unfused_swiglu_us": round(swi, 1),
            "unfused_total_us": round(gemm + swi, 1)}


def _vendor_gemm_component(torch, dev, reps=10):
    """The dense MXFP8 GEMM beside the vendor library on the same FP8 codes:
    hipBLASLt through torch._scaled_mm with block-32 E8M0 scales, its
    per-tensor-scaled FP8 GEMM and the bf16 matmul. Every scale is 2^0, so
    all four compute the same product; the largest relative difference to
    this library's output is reported."""
    from quantize_grouped_gemm_amd import mx
    g = torch.Generator(device=dev)
    g.manual_seed(0)

    def codes(r, c):
        mag = torch.randint(0, 0x7E, (r, c), generator=g, device=dev, dtype=torch.int32)
        sign = torch.randint(0, 2, (r, c), generator=g, device=dev, dtype=torch.int32) * 0x80
        return (mag | sign).to(torch.uint8)

    def timed(f):
        f()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                f()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / reps / 1e3)
        return sorted(ts)[1]

    res = {}
    # the dense MLP's w13 and w2 forward shapes, a square one and a MoE-sized one
    for M, N, K in ((8192, 28672, 4096), (8192, 4096, 14336), (8192, 8192, 8192), (16384, 16384, 5120)):
        qa, qb = codes(M, K), codes(N, K)
        sa = torch.full((K // 128, M, 4), 127, dtype=torch.uint8, device=dev)
        sb = torch.full((K // 128, N, 4), 127, dtype=torch.uint8, device=dev)
        out = mx.scaled_mm(qa, sa, qb, sb)
        fl = 2.0 * M * N * K
        r = {"this_mxfp8_tflops": round(fl / timed(lambda: mx.scaled_mm(qa, sa, qb, sb, out=out)) / 1e12, 1)}
        A, B = qa.view(torch.float8_e4m3fn), qb.view(torch.float8_e4m3fn)
        try:
            ea = torch.full((M, K // 32), 127, dtype=torch.uint8, device=dev).view(torch.float8_e8m0fnu)
            eb = torch.full((N, K // 32), 127, dtype=torch.uint8, device=dev).view(torch.float8_e8m0fnu)
            ref = torch._scaled_mm(A, B.t(), scale_a=ea, scale_b=eb, out_dtype=torch.bfloat16)
            r["hipblaslt_mxfp8_tflops"] = round(fl / timed(
                lambda: torch._scaled_mm(A, B.t(), scale_a=ea, scale_b=eb, out_dtype=torch.bfloat16)) / 1e12, 1)
            r["max_rel_diff_vs_hipblaslt_mxfp8"] = float(
                ((out.float() - ref.float()).abs().max() / ref.float().abs().max()).item())
            del ea, eb, ref
        except Exception as e:   # MX scales not supported by this torch / library build
            r["hipblaslt_mxfp8_tflops"] = f"unavailable: {type(e).__name__}"
        one = torch.ones((), device=dev)
        r["hipblaslt_fp8_tensorwise_tflops"] = round(fl / timed(
            lambda: torch._scaled_mm(A, B.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)) / 1e12, 1)
        Ab, Bb = A.to(torch.bfloat16), B.to(torch.bfloat16)
        r["torch_bf16_matmul_tflops"] = round(fl / timed(lambda: Ab @ Bb.t()) / 1e12, 1)
        res[f"{M}x{N}x{K}"] = r
        del qa, qb, sa, sb, out, A, B, Ab, Bb
        torch.cuda.empty_cache()
    return res


def _oracle_sqnr(net, sizes, x, w13, w2, dy, per_group=8, ncols=64, seed=0):
    """End-to-end SQNR (dB) of the GPU step's y, dx and weight gradients
    against a chain fed only by the oracle, from the same bf16 inputs
    (padding, quantization, GEMMs, SwiGLU, ...), on a bounded sample: y and
    dx for a few tokens of the largest and the smallest expert group on
    sampled output columns (their chains are row-local), and dW2 / dW13 of
    the smallest group on sampled entries (its whole chain: every one of its
    tokens, quantized along the tokens as the step does). The pages give no
    threshold; reported only. Part of the CPU-baseline leg (it runs the
    oracle)."""
    import numpy as np
    import torch
    from oracle import mx as O
    from quantize_grouped_gemm_amd import synth
    rng = np.random.default_rng(seed)
    H, D = net.H, net.D

    def bits(t):
        return synth.bits(t)

    def f64(t):
        return t.double().cpu().numpy() if t.dtype == torch.float32 else O.bf16_to_f64(bits(t))

    def sq(ref, got):
        ref, got = np.asarray(ref, np.float64), np.asarray(got, np.float64)
        return round(float(10 * np.log10(np.sum(ref * ref) / max(np.sum((got - ref) ** 2), 1e-300))), 2)

    def ix(a):
        return torch.as_tensor(np.asarray(a, np.int64), device=x.device)

    nz = [g for g in range(len(sizes)) if sizes[g] > 0]
    big, small = max(nz, key=lambda g: sizes[g]), min(nz, key=lambda g: sizes[g])
    tok0 = np.concatenate([[0], np.cumsum(sizes)])
    cols = np.sort(rng.choice(D, ncols, replace=False))
    ys, yg, dxs, dxg = [], [], [], []
    out = {}
    for g in (big, small):
        n = int(sizes[g])
        q13 = O.quantize_bf16(bits(w13[g]), "rceil")                               # along D
        q2r = O.quantize_bf16(bits(w2[g][ix(cols)]), "rceil")                      # rows `cols`, along H
        q2c = O.quantize_bf16(bits(w2[g].T.contiguous()), "rceil")                 # along D
        q13c = O.quantize_bf16(bits(w13[g][:, ix(cols)].T.contiguous()), "rceil")  # along 2H
        if g == small:
            # the whole group, padded to 128 rows, so its weight gradients
            # can be formed too
            tg = np.arange(tok0[g], tok0[g + 1])
            P = -(-n // 128) * 128
        else:
            tg = np.sort(rng.choice(np.arange(tok0[g], tok0[g + 1]), min(per_group, n), replace=False))
            P = len(tg)
        xb = np.zeros((P, D), np.uint16)
        dyb = np.zeros((P, D), np.uint16)
        xb[:len(tg)], dyb[:len(tg)] = bits(x[ix(tg)]), bits(dy[ix(tg)])
        qx = O.quantize_bf16(xb, "rceil", True, g == small)
        z = O.f64_to_bf16(O.scaled_mm(qx["q_row"], qx["s_row"], q13["q_row"], q13["s_row"]))
        h = O.swiglu_fwd(z[:, :H], z[:, H:])
        qh = O.quantize_bf16(h, "rceil", True, g == small)
        qdy = O.quantize_bf16(dyb, "rceil", True, g == small)
        dh = O.f64_to_bf16(O.scaled_mm(qdy["q_row"], qdy["s_row"], q2c["q_row"], q2c["s_row"]))
        dz = O.swiglu_bwd(dh, z[:, :H], z[:, H:])
        qdz = O.quantize_bf16(dz, "rceil", True, g == small)
        sel = np.arange(min(per_group, len(tg)))
        ys.append(O.scaled_mm(qh["q_row"][sel], qh["s_row"][sel], q2r["q_row"], q2r["s_row"]))
        dxs.append(O.scaled_mm(qdz["q_row"][sel], qdz["s_row"][sel], q13c["q_row"], q13c["s_row"]))
        yg.append(f64(net.y[ix(tg[sel])][:, ix(cols)]))
        dxg.append(f64(net.dx[ix(tg[sel])][:, ix(cols)]))
        if g == small:
            r_d, r_h, r_2h = (np.sort(rng.choice(m, 32, replace=False)) for m in (D, H, 2 * H))
            dw2 = O.scaled_mm(qdy["q_col"][r_d], qdy["s_col"][r_d], qh["q_col"][r_h], qh["s_col"][r_h])
            dw13 = O.scaled_mm(qdz["q_col"][r_2h], qdz["s_col"][r_2h], qx["q_col"][r_d], qx["s_col"][r_d])
            out["dw2_small_group"] = sq(dw2, f64(net.dw2[g][ix(r_d)][:, ix(r_h)]))
            out["dw13_small_group"] = sq(dw13, f64(net.dw13[g][ix(r_2h)][:, ix(r_d)]))
    out["y"] = sq(np.concatenate(ys), np.concatenate(yg))
    out["dx"] = sq(np.concatenate(dxs), np.concatenate(dxg))
    out["sample"] = (f"y, dx: {per_group} tokens of expert {big} ({int(sizes[big])} tokens) and of expert {small} "
                     f"({int(sizes[small])} tokens) x {ncols} columns; dW2, dW13: expert {small}, 32 x 32 "
                     f"entries, all its tokens")
    return out


def _cpu_baseline():
    """The oracle on a bounded slice of the default workload: one expert with
    4096 of its 8192 hidden units and 2048 tokens (about 15 s on 16 host
    threads). Weight quantization and the
    token-dependent work are timed separately and each scaled to the full
    step (16 experts x 8192 hidden; 16384 tokens x 8192 hidden)."""
    import numpy as np
    from oracle import mx as O
    from quantize_grouped_gemm_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    E, T, D, Hs = 1, 2048, 5120, 4096
    c = synth.MOE_SCOUT
    x, w1, w3, w2, dy = [synth.bits(t) for t in synth.mlp_inputs(T, D, Hs, E=E, seed=0)]
    w13 = np.concatenate([w1, w3], axis=1)
    t0 = time.perf_counter()
    O.quantize_bf16(w13, "rceil", True, True)
    O.quantize_bf16(w2, "rceil", True, True)
    t_w = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.moe_mlp_step(x, np.array([T]), w1, w3, w2, dy, "rceil", T)
    t_all = time.perf_counter() - t0
    t_tok = max(t_all - t_w, 1e-9)
    full = t_w * c["E"] * (c["H"] / Hs) + t_tok * (c["T"] / T) * (c["H"] / Hs)
    return {"value": round(c["T"] / full, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "sample": (f"oracle on 1 expert x {Hs}/{c['H']} hidden x {T} tokens, D={D}: weight dual "
                       f"quantization {t_w:.1f} s and token work {t_tok:.1f} s, scaled to 16 experts x "
                       f"{c['H']} hidden and {c['T']} tokens (estimated full step {full:.0f} s)"),
            "sample_seconds": round(t_all, 2)}


def main():
    args = _args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the MXFP8 path here has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(2)
    _ensure_lib()
    dev = torch.device("cuda:0")
    torch.manual_seed(0)

    name = args.workload
    if name == "copy":
        # reference for scaling the FETCH_SIZE / WRITE_SIZE counters: one plain
        # device copy of exactly 1 GiB (reads 1 GiB, writes 1 GiB)
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"workload": "copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30}))
        return
    if name in ("quant", "linear", "vendor_gemm"):
        comp = {"quant": _quant_component, "linear": _linear_component,
                "vendor_gemm": _vendor_gemm_component}[name](torch, dev)
        print(json.dumps({"workload": name, **comp}))
        return

    net, wargs, stages, tokens, config = _build_workload(name, torch, dev)
    torch.cuda.synchronize()
    wall, per = _time_stages(stages, args.steps, args.warmup, torch)
    sqnr = None
    if not args.no_cpu_baseline and name.startswith("moe") and name != "moe_scout_fp8" and not name.endswith("hp"):
        # the CPU-baseline leg's parity figure: the oracle chain against this
        # step's own outputs (the last timed step's, all steps being equal)
        import numpy as np
        x_, sizes_, w13_, w2_, dy_ = wargs
        sqnr = _oracle_sqnr(net, np.array(config["group_sizes"]), x_, w13_, w2_, dy_)
    kernels, table = _kernel_table(stages, per, net.gemm_bytes())
    gemm_kernel = "k_gemm_grouped" if name.startswith("moe") else "k_gemm_dense"
    gemm_flops = sum(st.flops for st in stages)
    gemm_time = sum(t for st, t in zip(stages, per) if st.flops)
    mem_bytes = sum(st.bytes for st in stages)
    roof_time = gemm_flops / PEAK_MXFP8 + mem_bytes / PEAK_HBM
    result = {
        "metric": "MoE MLP fwd+bwd tokens/s (1 GPU)" if name.startswith("moe") else "MLP fwd+bwd tokens/s (1 GPU)",
        "value": round(tokens / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3, one power-of-two scale per row" if name == "moe_scout_fp8" else "mxfp8",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, routed group sizes)",
        "config": config,
        "roofline": _roofline_gemm(table, gemm_kernel, PEAK_MXFP8,
                                   _measured_traffic() if name == "moe_scout" else None,
                                   _padded_ratio(config), _measured_mfma() if name == "moe_scout" else None),
        "step_roofline": {"gemm_useful_tflops": round(gemm_flops / gemm_time / 1e12, 1),
                          "ideal_ms": round(roof_time * 1e3, 4), "frac": round(roof_time / wall, 4)},
        "kernels": kernels,
    }
    del net, wargs, stages
    torch.cuda.empty_cache()
    if not args.no_components:
        comp = {"quantize_stress_32768x7168": _quant_component(torch, dev),
                "linear_256x256x512": _linear_component(torch, dev)}
        torch.cuda.empty_cache()
        if name == "moe_scout":
            comp["moe_scout_w13_fwd_fused_swiglu"] = _fused_swiglu_component(torch, dev)
        if name.startswith("moe"):
            # an optimizer step of 4 micro-batches: the expert weights are
            # dual-quantized once and their MXFP8 copies reused
            n2, a2, s2, tok2, c2 = _build_workload(name, torch, dev)
            acc = list(s2) + 3 * n2.stages(*a2, quantize_weights=False)
            w2_, p2 = _time_stages(acc, max(3, args.steps // 4), 1, torch)
            comp[f"{name}_4_microbatches"] = {
                "tokens_per_s": round(4 * tok2 / w2_, 1), "ms_per_optimizer_step": round(w2_ * 1e3, 3),
                "workload": c2["workload"] + "; 4 micro-batches per optimizer step, expert weights "
                                              "dual-quantized once and reused"}
            del n2, a2, s2, acc
            torch.cuda.empty_cache()
        if name == "moe_scout":
            # the FP8 row-scaled recipe of the same step
            n2, a2, s2, tok2, c2 = _build_workload("moe_scout_fp8", torch, dev)
            w2_, p2 = _time_stages(s2, max(3, args.steps // 2), 2, torch)
            comp["moe_scout_fp8_rowwise"] = {"tokens_per_s": round(tok2 / w2_, 1), "ms_per_step": round(w2_ * 1e3, 3),
                                             "kernels": _kernel_table(s2, p2, n2.gemm_bytes())[0],
                                             "workload": c2["workload"]}
            del n2, a2, s2
            torch.cuda.empty_cache()
            # the same step with bf16 dW (half the weight gradients' bytes
            # written); the headline keeps float32 dW
            n2, a2, s2, tok2, c2 = _build_workload("moe_scout", torch, dev, wgrad_dtype=torch.bfloat16)
            w2_, p2 = _time_stages(s2, max(3, args.steps // 2), 2, torch)
            comp["moe_scout_bf16_dw"] = {"tokens_per_s": round(tok2 / w2_, 1), "ms_per_step": round(w2_ * 1e3, 3),
                                         "kernels": _kernel_table(s2, p2, n2.gemm_bytes())[0],
                                         "workload": c2["workload"]}
            del n2, a2, s2
            torch.cuda.empty_cache()
        for other in ("dense", "moe_dsv3", "moe_dsv3_hp"):
            n2, a2, s2, tok2, c2 = _build_workload(other, torch, dev)
            w2_, p2 = _time_stages(s2, max(3, args.steps // 2), 2, torch)
            k2, t2 = _kernel_table(s2, p2, n2.gemm_bytes())
            gk = "k_gemm_grouped" if other.startswith("moe") else "k_gemm_dense"
            comp[other] = {"tokens_per_s": round(tok2 / w2_, 1), "ms_per_step": round(w2_ * 1e3, 3),
                           "gemm_roofline": _roofline_gemm(t2, gk, PEAK_MXFP8, padded_ratio=_padded_ratio(c2)), "kernels": k2,
                           "workload": c2["workload"]}
            del n2, a2, s2
            torch.cuda.empty_cache()
        result["components"] = comp
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _cpu_baseline()
        if sqnr is not None:
            result["cpu_baseline"]["sqnr_vs_oracle_db"] = sqnr
    print(json.dumps(result))


if __name__ == "__main__":
    main()
