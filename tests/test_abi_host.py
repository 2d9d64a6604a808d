"""Host-side checks of libmxfp8.so without a GPU: the library loads, exports
every entry point that include/mxfp8.h declares (and the binding binds all of
them), and argument errors are reported before any device work."""

import ctypes
import os
import re

import pytest

from quantize_grouped_gemm_amd import mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp8.h")


def _lib():
    if not os.path.exists(mx.LIB_PATH):
        from quantize_grouped_gemm_amd import build
        build.build()
    return mx.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported_and_bound():
    L = _lib()
    names = _declared()
    assert len(names) == 22
    for n in names:
        assert hasattr(L, n), n
    assert sorted(mx.EXPORTS) == names
    assert L.mx_abi_version() == 3


def test_argument_errors_are_reported_without_device_work():
    L = _lib()
    p = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    # cols not a multiple of 32
    st = L.mx_quantize(p, 1, 64, 48, 48, 0, 1, 0, p, p, None, None, None)
    assert st == 2 and b"multiple of 32" in L.mx_last_error()
    # K128 scales need the block axis to be a multiple of 128 (row-wise: cols;
    # column-wise: rows)
    st = L.mx_quantize(p, 1, 128, 96, 96, 0, 1, 1, p, p, None, None, None)
    assert st == 2 and b"multiple of 128" in L.mx_last_error()
    assert L.mx_quantize(p, 1, 96, 128, 128, 0, 2, 1, None, None, p, p, None) == 2
    # bad scale mode / direction bits / layout
    assert L.mx_quantize(p, 1, 64, 64, 64, 7, 1, 0, p, p, None, None, None) == 4
    assert L.mx_quantize(p, 1, 64, 64, 64, 0, 8, 0, p, p, None, None, None) == 4
    assert L.mx_quantize(p, 1, 64, 64, 64, 0, 1, 2, p, p, None, None, None) == 4
    # misaligned pointer; K128 scales must be 4-byte aligned
    assert L.mx_quantize(ctypes.c_void_p(18), 1, 64, 64, 64, 0, 1, 0, p, p, None, None, None) == 3
    assert L.mx_quantize(p, 1, 128, 128, 128, 0, 1, 1, p, ctypes.c_void_p(18), None, None, None) == 3
    assert L.mx_dequantize(p, p, 32, 96, 1, 0, p, None) == 2
    assert L.mx_swiglu_quant_fwd(p, p, 192, 64, 96, 0, 1, p, p, p, p, None, None) == 2
    # K not a multiple of 128
    assert L.mx_scaled_mm(p, p, p, p, 32, 32, 96, 0, p, 32, None) == 2
    # grouped: Tcap not a multiple of 128, bad E
    assert L.mx_scaled_grouped_mm_fwd(p, p, p, p, p, 4, 100, 64, 128, 0, p, None, None) == 2
    assert L.mx_scaled_grouped_mm_wgrad(p, p, p, p, p, 0, 128, 64, 64, 1, p, None, None) == 2
    # GEMM operand rows are addressed with 32-bit offsets: K below 2^23 (and
    # (H + 128) x K below 2^31 for the fused w13 + SwiGLU)
    st = L.mx_scaled_mm(p, p, p, p, 256, 256, 1 << 23, 0, p, 256, None)
    assert st == 2 and b"below 2^23" in L.mx_last_error()
    assert L.mx_scaled_grouped_mm_fwd(p, p, p, p, p, 4, 256, 64, 1 << 23, 0, p, None, None) == 2
    st = L.mx_scaled_grouped_mm_swiglu_fwd(p, p, p, p, p, 4, 256, 1 << 16, 1 << 15, 0, p, p, p, p, p, None,
                                           None, None)
    assert st == 2 and b"(H + 128)" in L.mx_last_error()
    # MXFP8 weight gradient: 256 rows of Tcap codes must be addressable with 32-bit offsets
    st = L.mx_scaled_grouped_mm_wgrad(p, p, p, p, p, 4, 1 << 23, 16, 16, 1, p, None, None)
    assert st == 2 and b"below 2^23" in L.mx_last_error()
    # one workgroup per dW tile of every group: the 1-D grid must hold them
    st = L.mx_scaled_grouped_mm_wgrad(p, p, p, p, p, 1024, 128, 1 << 20, 1 << 20, 0, p, None, None)
    assert st == 2 and b"too many tiles" in L.mx_last_error()
    assert L.mx_pad_groups(p, p, 2, 10, 24, 128, 256, p, p, p, None, None) == 2
    assert L.mx_unpad_groups(p, p, 128, 10, 32, None, None) == 1
    # FP8 row-scaled: cols not a multiple of 128; column-wise rows not a
    # multiple of 128; offsets without a group count
    assert L.mx_quantize_fp8_rowwise(p, 1, 64, 96, 96, p, p, None) == 2
    assert L.mx_quantize_fp8_colwise(p, 1, 96, 128, 128, None, 0, p, p, p, None, None) == 2
    assert L.mx_quantize_fp8_colwise(p, 1, 128, 128, 128, p, 0, p, p, p, None, None) == 2
    assert L.mx_quantize_fp8_dual(p, 1, 96, 128, 128, None, 0, p, p, p, p, p, None, None) == 2
    assert L.mx_quantize_fp8_dual(p, 1, 128, 128, 128, p, 0, p, p, p, p, p, None, None) == 2
    assert L.mx_quantize_fp8_dual(p, 1, 128, 128, 128, None, 0, p, p, None, p, p, None, None) == 1
    # fused w13 + SwiGLU: H not a multiple of 128, bad mode
    assert L.mx_scaled_grouped_mm_swiglu_fwd(p, p, p, p, p, 4, 256, 96, 128, 0, p, p, p, p, p, None, None,
                                             None) == 2
    assert L.mx_scaled_grouped_mm_swiglu_fwd(p, p, p, p, p, 4, 256, 128, 128, 5, p, p, p, p, p, None, None,
                                             None) == 4
    # token-order grouped GEMM: T beyond Tcap, missing group sizes
    assert L.mx_scaled_grouped_mm_fwd_unpad(p, p, p, p, p, p, 4, 256, 300, 64, 128, 0, p, None, None) == 2
    assert L.mx_scaled_grouped_mm_dgrad_unpad(p, p, p, p, p, None, 4, 256, 200, 64, 128, 0, p, None, None) == 1
    # fused pad + quantize: cols not a multiple of 32, K128 column-wise needs
    # Tcap % 128, missing row map
    assert L.mx_pad_quantize(p, p, 2, 10, 48, 128, 256, 0, 1, 0, p, p, None, None, p, p, None, None) == 2
    assert L.mx_pad_quantize(p, p, 2, 10, 128, 128, 96, 0, 2, 1, None, None, p, p, p, p, None, None) == 2
    assert L.mx_pad_quantize(p, p, 2, 10, 128, 128, 256, 0, 1, 0, p, p, None, None, p, None, None, None) == 1


def test_valid_call_without_gpu_fails_loudly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; the device path is covered by the gpu tests")
    L = _lib()
    p = ctypes.c_void_p(16)
    st = L.mx_quantize(p, 1, 64, 64, 64, 0, 1, 0, p, p, None, None, None)
    assert st == 5
    assert L.mx_last_error()


def test_k128_scale_layout_permutation():
    """The tests' layout converters follow the header's K128 formula: byte
    ((j/4) * R + r) * 4 + j%4 holds the scale of row r, block j."""
    import numpy as np

    from _helpers import k128, plain
    rng = np.random.default_rng(0)
    for lead, R, nb in (((), 5, 8), ((3,), 7, 4), ((2, 2), 3, 12)):
        s = rng.integers(0, 256, lead + (R, nb)).astype(np.uint8)
        t = k128(s)
        assert t.shape == lead + (nb // 4, R, 4)
        flat = t.reshape(lead + (-1,))
        for idx in np.ndindex(*lead):
            for r in range(R):
                for j in range(nb):
                    assert flat[idx + (((j // 4) * R + r) * 4 + j % 4,)] == s[idx + (r, j)]
        np.testing.assert_array_equal(plain(t), s)
