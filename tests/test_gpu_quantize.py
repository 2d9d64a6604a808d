"""GPU parity of MX quantization and dequantization against the oracle:
bit-exact codes and scales (in both scale layouts; k128 scales are compared
after the inverse permutation), every direction and mode, ragged tiles,
batches, strided rows, every finite bf16 value, the stress tensor's planted
cases, and sampled blocks of the full [32768, 7168] stress tensor."""

import numpy as np
import pytest
import torch

from _helpers import bf16_host, dev, host, k128, plain, to_dev
from oracle import mx as O
from quantize_grouped_gemm_amd import mx, synth

pytestmark = pytest.mark.gpu

MODES = ["rceil", "floor"]


def _check_quant(xb_host, xt, mode, rowwise=True, colwise=True, layout="k128"):
    got = mx.quantize(xt, mode, rowwise, colwise, layout=layout)
    ref = O.quantize_bf16(xb_host, mode, rowwise, colwise)
    for k in ref:
        g = host(got[k])
        if k.startswith("s_") and layout == "k128":
            assert g.shape[-1] == 4 and g.shape[-2] == ref[k].shape[-2]
            g = plain(g)
        np.testing.assert_array_equal(g, ref[k], err_msg=f"{k} {mode} {layout}")
    return got


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", [(32, 32), (64, 96), (160, 224), (256, 512), (384, 128)])
def test_quantize_shapes(gpu, mode, shape):
    xb = synth.bits(synth.stress_tensor(*shape, seed=sum(shape)))
    _check_quant(xb, to_dev(xb.view(np.int16)).view(torch.bfloat16), mode, layout="plain")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", [(128, 128), (256, 512), (384, 128), (640, 384)])
def test_quantize_shapes_k128(gpu, mode, shape):
    xb = synth.bits(synth.stress_tensor(*shape, seed=sum(shape) + 1))
    _check_quant(xb, to_dev(xb.view(np.int16)).view(torch.bfloat16), mode, layout="k128")


@pytest.mark.parametrize("seed", range(10))
def test_quantize_random_shapes(gpu, seed):
    """Seeded random requests: batch of 1..3 matrices, row stride wider than
    the columns, either scale layout, mode and direction set, sizes off the
    128 x 128 tile grid where the layout allows (row-wise: any row count;
    plain scales: columns and column-wise rows in multiples of 32)."""
    rng = np.random.default_rng(4000 + seed)
    layout = ["plain", "k128"][seed % 2]
    mode = MODES[int(rng.integers(0, 2))]
    rowwise, colwise = [(True, False), (False, True), (True, True)][int(rng.integers(0, 3))]
    m = 128 if layout == "k128" else 32
    C = m * int(rng.integers(1, 1 + 640 // m))
    R = (m if colwise else 1) * int(rng.integers(1, 1 + 640 // (m if colwise else 1)))
    batch = int(rng.integers(1, 4))
    ld = C + 8 * int(rng.integers(0, 5))
    print(f"seed {seed}: {layout} {mode} row={rowwise} col={colwise} batch={batch} R={R} C={C} ld={ld}", flush=True)
    xb = synth.bits(synth.normal_bf16((batch, R, ld), 1.0, synth.generator(seed)))
    # a few blocks at large and tiny magnitudes
    xb[:, : R // 2, : min(C, 64)] = synth.bits(
        synth.normal_bf16((batch, R // 2, min(C, 64)), 2.0 ** 12, synth.generator(seed + 50)))
    xt = to_dev(xb.view(np.int16)).view(torch.bfloat16)[..., :C]
    got = mx.quantize(xt, mode, rowwise, colwise, layout=layout)
    for b in range(batch):
        ref = O.quantize_bf16(np.ascontiguousarray(xb[b, :, :C]), mode, rowwise, colwise)
        for k in ref:
            g = host(got[k][b])
            if k.startswith("s_") and layout == "k128":
                g = plain(g)
            np.testing.assert_array_equal(g, ref[k], err_msg=f"{k} matrix {b}")


@pytest.mark.parametrize("mode", MODES)
def test_quantize_rowwise_any_rows_and_separate_directions(gpu, mode):
    xb = synth.bits(synth.normal_bf16((100, 96), 1.0, synth.generator(3)))
    xt = to_dev(xb.view(np.int16)).view(torch.bfloat16)
    _check_quant(xb, xt, mode, True, False, layout="plain")
    xb = xb[:96]
    xt = xt[:96].contiguous()
    _check_quant(xb, xt, mode, False, True, layout="plain")
    # k128: row-wise takes any row count; column-wise needs rows % 128
    xb = synth.bits(synth.normal_bf16((100, 256), 1.0, synth.generator(4)))
    _check_quant(xb, to_dev(xb.view(np.int16)).view(torch.bfloat16), mode, True, False)
    xb = synth.bits(synth.normal_bf16((256, 96), 1.0, synth.generator(5)))
    _check_quant(xb, to_dev(xb.view(np.int16)).view(torch.bfloat16), mode, False, True)


@pytest.mark.parametrize("mode", MODES)
def test_quantize_batched_and_strided(gpu, mode):
    xb = synth.bits(synth.stress_tensor(3 * 64, 96, seed=11)).reshape(3, 64, 96)
    _check_quant(xb, to_dev(xb.view(np.int16)).view(torch.bfloat16), mode, layout="plain")
    xb = synth.bits(synth.stress_tensor(3 * 128, 256, seed=13)).reshape(3, 128, 256)
    _check_quant(xb, to_dev(xb.view(np.int16)).view(torch.bfloat16), mode)
    # rows with a leading dimension larger than the width (a column slice)
    wide = synth.bits(synth.stress_tensor(128, 320, seed=12))
    wt = to_dev(wide.view(np.int16)).view(torch.bfloat16)
    _check_quant(wide[:, 64:256], wt[:, 64:256], mode, layout="plain")
    wide = synth.bits(synth.stress_tensor(256, 640, seed=14))
    wt = to_dev(wide.view(np.int16)).view(torch.bfloat16)
    _check_quant(wide[:, 128:384], wt[:, 128:384], mode)


@pytest.mark.parametrize("mode", MODES)
def test_quantize_every_finite_bf16_value(gpu, mode):
    """Each of the 65280 finite bf16 patterns appears 32 times, in blocks
    whose other members have log-uniform random magnitudes, so each value is
    quantized under many different scales."""
    rng = np.random.default_rng(5)
    allv = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allv[(allv & 0x7F80) != 0x7F80]
    vals = np.tile(finite, 32)
    rng.shuffle(vals)
    n = len(vals)
    cols = 1024
    rows = -(-n // cols // 32) * 32
    pad = rows * cols - n
    filler = (rng.integers(0, 0x7F00, pad) | (rng.integers(0, 2, pad) << 15)).astype(np.uint16)
    xb = np.concatenate([vals, filler]).reshape(rows, cols)
    _check_quant(xb, to_dev(xb.view(np.int16)).view(torch.bfloat16), mode)


def test_quantize_nonfinite_blocks(gpu):
    xb = synth.bits(synth.normal_bf16((64, 64), 1.0, synth.generator(9)))
    xb[3, 5] = 0x7FC0     # NaN
    xb[40, 33] = 0xFF80   # -inf
    xb[10, 62] = 0x7F80   # +inf
    for mode in MODES:
        _check_quant(xb, to_dev(xb.view(np.int16)).view(torch.bfloat16), mode, layout="plain")
    big = synth.bits(synth.normal_bf16((128, 256), 1.0, synth.generator(10)))
    big[3, 5] = 0x7FC0
    big[100, 200] = 0xFF80
    for mode in MODES:
        _check_quant(big, to_dev(big.view(np.int16)).view(torch.bfloat16), mode)


@pytest.mark.parametrize("mode", MODES)
def test_stress_full_size_sampled(gpu, mode):
    """The [32768, 7168] stress tensor, quantized in the launch configuration
    the benchmark uses. The oracle checks 512 random rows plus every row
    holding a zero or all-subnormal row block (row-wise), and 256 random
    columns plus every column holding such a column block (column-wise)."""
    R, C = synth.STRESS_SHAPE
    x = synth.stress_tensor(R, C, seed=0, device=dev())
    got = mx.quantize(x, mode, True, True)
    rng = np.random.default_rng(1)
    tiny = 2.0 ** -126
    a = x.abs().float()
    special_rows = torch.nonzero((a.view(R, C // 32, 32).amax(-1) < tiny).any(-1)).flatten().cpu().numpy()
    special_cols = torch.nonzero((a.view(R // 32, 32, C).amax(1) < tiny).any(0)).flatten().cpu().numpy()
    rows = np.unique(np.concatenate([rng.choice(R, 512, replace=False), special_rows]))
    cols = np.unique(np.concatenate([rng.choice(C, 256, replace=False), special_cols]))
    assert len(special_rows) >= 64 and len(special_cols) >= 64
    ri = torch.as_tensor(rows, device=dev())
    ci = torch.as_tensor(cols, device=dev())
    s_row = plain(host(got["s_row"]))
    s_col = plain(host(got["s_col"]))
    q, s = O.quantize(O.bf16_to_f64(bf16_host(x[ri])), mode)
    np.testing.assert_array_equal(host(got["q_row"][ri]), q)
    np.testing.assert_array_equal(s_row[rows], s)
    q, s = O.quantize(O.bf16_to_f64(bf16_host(x[:, ci])).T, mode)
    np.testing.assert_array_equal(host(got["q_col"][ci]), q)
    np.testing.assert_array_equal(s_col[cols], s)
    # dequantize round trip on the same rows: bit-exact against the oracle
    deq = mx.dequantize(got["q_row"], got["s_row"], torch.float32)
    ref = O.f64_to_f32(O.dequantize(host(got["q_row"][ri]), s_row[rows]))
    np.testing.assert_array_equal(host(deq[ri]).view(np.uint32), ref.view(np.uint32))


def test_quantize_inputs_over_one_gib(gpu):
    """Inputs of 1 GiB and more are read with plain loads, smaller ones with
    non-temporal loads: a [2, 16512, 16384] batch of expert weights (1.01
    GiB, N(0, 0.02) with planted outliers and zero blocks) quantized both
    ways, checked bit-exactly on sampled rows and columns of each matrix,
    and against the same matrices quantized one at a time (0.50 GiB each)."""
    Bt, R, C = 2, 16512, 16384
    assert Bt * R * C * 2 >= 1 << 30 > R * C * 2
    g = synth.generator(21, dev())
    w = synth.normal_bf16((Bt, R, C), 0.02, g, dev())
    rng = np.random.default_rng(21)
    flat = w.view(-1)
    pos = torch.as_tensor(np.unique(rng.integers(0, w.numel(), 4096)), device=dev())
    flat[pos] = torch.as_tensor(rng.choice([-1.0, 1.0], len(pos)) * 2.0 ** rng.integers(-3, 9, len(pos)),
                                dtype=torch.bfloat16, device=dev())
    w[0, 100, 32 * 7:32 * 8] = 0
    w[1, 32 * 9:32 * 10, 5] = 0
    got = mx.quantize(w, "rceil", True, True)
    for b in range(Bt):
        one = mx.quantize(w[b], "rceil", True, True)
        for k in ("q_row", "s_row", "q_col", "s_col"):
            assert torch.equal(got[k][b], one[k]), f"{k} of matrix {b}"
        # row 100 holds matrix 0's zero row block, column 5 matrix 1's zero column block
        rows = np.unique(np.append(rng.choice(R, 64, replace=False), 100))
        cols = np.unique(np.append(rng.choice(C, 64, replace=False), 5))
        ri = torch.as_tensor(rows, device=dev())
        ci = torch.as_tensor(cols, device=dev())
        q, s = O.quantize(O.bf16_to_f64(bf16_host(w[b][ri])), "rceil")
        np.testing.assert_array_equal(host(got["q_row"][b][ri]), q)
        np.testing.assert_array_equal(plain(host(got["s_row"][b]))[rows], s)
        q, s = O.quantize(O.bf16_to_f64(bf16_host(w[b][:, ci])).T, "rceil")
        np.testing.assert_array_equal(host(got["q_col"][b][ci]), q)
        np.testing.assert_array_equal(plain(host(got["s_col"][b]))[cols], s)


@pytest.mark.parametrize("cols,layout", [(128 * 127, "k128"), (128 * 126 + 64, "plain")])
def test_quantize_two_tile_path_odd_and_ragged_columns(gpu, cols, layout):
    """Inputs with at least 48 tiles per CU and no row map are quantized two
    adjacent column tiles per workgroup: here an odd number of column tiles
    (the last pair half out of range) and, in the plain layout, a ragged
    last tile of 64 columns. Sampled rows (row-wise) and columns
    (column-wise), the last 200 columns included, against the oracle."""
    R = 128 * 97
    assert (R // 128) * (-(-cols // 128)) >= 48 * 256
    g = synth.generator(cols, dev())
    x = synth.normal_bf16((R, cols), 1.0, g, dev())
    got = mx.quantize(x, "rceil", True, True, layout=layout)
    rng = np.random.default_rng(cols)
    rows = np.unique(np.append(rng.choice(R, 48, replace=False), [0, R - 1]))
    ccols = np.unique(np.concatenate([rng.choice(cols, 48, replace=False), np.arange(cols - 200, cols)]))
    ri = torch.as_tensor(rows, device=dev())
    ci = torch.as_tensor(ccols, device=dev())
    s_row, s_col = host(got["s_row"]), host(got["s_col"])
    if layout == "k128":
        s_row, s_col = plain(s_row), plain(s_col)
    q, s = O.quantize(O.bf16_to_f64(bf16_host(x[ri])), "rceil")
    np.testing.assert_array_equal(host(got["q_row"][ri]), q)
    np.testing.assert_array_equal(s_row[rows], s)
    q, s = O.quantize(O.bf16_to_f64(bf16_host(x[:, ci])).T, "rceil")
    np.testing.assert_array_equal(host(got["q_col"][ci]), q)
    np.testing.assert_array_equal(s_col[ccols], s)


@pytest.mark.parametrize("layout", ["plain", "k128"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dequantize_all_codes_all_scales(gpu, out_dtype, layout):
    """Every code under every scale byte (0..254 and the NaN scale 0xFF); the
    scale bytes also vary along each row so the layouts differ."""
    codes = np.tile(np.arange(256, dtype=np.uint8), 256 * 4).reshape(256, 1024)   # [scale byte, ...]
    scales = ((np.arange(256)[:, None] + 37 * np.arange(32)[None, :]) % 256).astype(np.uint8)
    s_dev = to_dev(k128(scales) if layout == "k128" else scales)
    got = mx.dequantize(to_dev(codes), s_dev, out_dtype, layout=layout)
    ref = O.dequantize(codes, scales)
    if out_dtype == torch.float32:
        g = host(got).astype(np.float64)
        r = O.f64_to_f32(ref).astype(np.float64)
    else:
        g = O.bf16_to_f64(bf16_host(got))
        r = O.bf16_to_f64(O.f64_to_bf16(ref))
    nan = np.isnan(r)
    np.testing.assert_array_equal(np.isnan(g), nan)
    np.testing.assert_array_equal(g[~nan], r[~nan])
    np.testing.assert_array_equal(np.signbit(g[~nan]), np.signbit(r[~nan]))
