"""The allocation-free FP8 dual quantizer (mx_quantize_fp8_dual_scratch)
against the entry point it is a variant of (mx_quantize_fp8_dual with a
caller-owned work area), bit for bit, through the C ABI: two calls in a row,
the second on a smaller input (so stale work-area contents from the first
would show), plus a request larger than the library's 4 MiB work area, which
is refused before anything runs."""

import numpy as np
import pytest
import torch

from _helpers import dev, to_dev
from quantize_grouped_gemm_amd import mx, synth

pytestmark = pytest.mark.gpu


def _same(a, b, what):
    for k in ("q_row", "s_row", "q_col", "s_col"):
        assert torch.equal(a[k], b[k]), f"{what}: {k}"


def test_scratch_entry_point_matches_workspace_entry_point(gpu):
    g = synth.generator(21, dev())
    # a padded activation with per-group column scales (one empty group)
    x1 = synth.normal_bf16((2048, 512), 1.0, g, dev())
    offs = to_dev(np.array([384, 384, 1280], np.int32))
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    got1 = mx.quantize_fp8_dual_scratch(x1, offs=offs, dev_err=err)
    ref1 = mx.quantize_fp8(x1, True, True, offs=offs)
    torch.cuda.synchronize()
    _same(got1, ref1, "first call")
    assert int(err.item()) == 0
    # second call, smaller, without offsets, batched like expert weights
    x2 = synth.normal_bf16((2, 256, 384), 0.02, g, dev())
    got2 = mx.quantize_fp8_dual_scratch(x2)
    ref2 = mx.quantize_fp8(x2, True, True)
    torch.cuda.synchronize()
    _same(got2, ref2, "second call")
    # bad offsets are still reported
    err.zero_()
    mx.quantize_fp8_dual_scratch(x1, offs=to_dev(np.array([384, 200, 1280], np.int32)), dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 1


def test_scratch_entry_point_rejects_oversized_requests(gpu):
    x = torch.zeros((1, 128), dtype=torch.bfloat16, device=dev()).expand(8192, 128).contiguous()
    big = x.reshape(1, 8192, 128).expand(200, 8192, 128)   # 200 * (128 + 8192) int32 > 1 Mi
    with pytest.raises(mx.MXError, match="work area"):
        mx.quantize_fp8_dual_scratch(big.contiguous())
