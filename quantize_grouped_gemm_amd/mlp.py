"""MXFP8 SwiGLU MLP forward + backward composed from the libmxfp8 calls.

Pipeline (the fused-MLP composite of "Add MXFP8 fused-MLP overrides in
torchtitan", Summary: w13 GEMM -> fused SwiGLU + dual MXFP8 quantization ->
w2 GEMM, and its backward; the per-group padding of the routed-experts
variant follows the same page's integration notes and the torchtitan commit
quoted on the TrainingWeightWrapperTensor page):

  forward   quantize x (rows; columns too for the weight gradient)
            quantize w13 = [w1; w3] and w2 (rows and columns)
            z = x w13^T                       (bf16, MXFP8 GEMM)
            h = silu(z[:, :H]) * z[:, H:]     (fused kernel: h quantized both
                                               ways, bf16 h only if asked)
            y = h w2^T
  backward  quantize dy (rows and columns)
            dh   = dy w2                      (w2 quantized along D)
            dW2  = dy^T h                     (both quantized along tokens)
            dZ   = SwiGLU backward            (fused kernel, dual quantized)
            dx   = dZ w13                     (w13 quantized along 2H)
            dW13 = dZ^T x
The grouped variant pads each expert's tokens to a multiple of 128 first
and runs the grouped GEMMs over the padded offsets; the w2 forward and the
w13 input gradient write y and dx straight in token order. With the
MXFP8 weight gradient the padding of x and dy is fused into their
quantization (no bf16 padded copy); the hp recipe keeps the bf16 copies,
which its weight-gradient GEMM reads.

Every buffer is allocated once per shape by the workspace classes, so a
training step only enqueues kernels. The weight-gradient GEMMs run in MXFP8
(float32 dW) or, with wgrad="hp" (the wgrad_with_hp recipe), on the bf16
operands (bf16 dW).
"""

import collections

import torch

from . import mx

# One kernel launch of a step: its name, the HIP kernel it runs, the
# algorithmic work it must do (useful flops for GEMMs, bytes that must move
# for the bandwidth-bound kernels) and the call itself.
Stage = collections.namedtuple("Stage", "name kernel flops bytes fn")


def _qbytes(n, dual):
    """Bytes a quantization of n bf16 values must move: read 2, write 1 code
    + 1/32 scale per direction."""
    return n * (2 + (2 if dual else 1) * (1 + 1 / 32))


_WEIGHT_STAGES = ("quant_w13", "quant_w2", "fp8_w13", "fp8_w2")


def _weights_cached(stages, quantize_weights):
    """Drops the weight quantizations when the cached MXFP8 weights are
    reused: weights change only at the optimizer step, so the micro-batches
    of one step can share one dual quantization of w13 and w2."""
    return stages if quantize_weights else [st for st in stages if st.name not in _WEIGHT_STAGES]


def _pad_qbytes(T, Tcap, D):
    """Bytes of the fused pad + dual quantization: the T real rows are read
    once, the padded [Tcap, D] codes and scales are written both ways, and the
    row map is written."""
    return 2 * T * D + Tcap * D * 2 * (1 + 1 / 32) + 4 * Tcap


def _q_out(lead, R, C, dev, row=True, col=True):
    o = {}
    if row:
        o["q_row"] = torch.empty(lead + (R, C), dtype=torch.uint8, device=dev)
        o["s_row"] = torch.empty(lead + mx.scale_shape(R, C), dtype=torch.uint8, device=dev)
    if col:
        o["q_col"] = torch.empty(lead + (C, R), dtype=torch.uint8, device=dev)
        o["s_col"] = torch.empty(lead + mx.scale_shape(C, R), dtype=torch.uint8, device=dev)
    return o


class DenseMLP:
    """Buffers and step of the dense MXFP8 SwiGLU MLP (T tokens, dim D,
    hidden H)."""

    def __init__(self, T, D, H, device, mode="rceil", wgrad_dtype=torch.float32):
        self.T, self.D, self.H, self.mode = T, D, H, mode
        dev = device
        bf = torch.bfloat16
        self.qx = _q_out((), T, D, dev)
        self.q13 = _q_out((), 2 * H, D, dev)
        self.q2 = _q_out((), D, H, dev)
        self.qdy = _q_out((), T, D, dev)
        self.z = torch.empty((T, 2 * H), dtype=bf, device=dev)
        self.hq = _q_out((), T, H, dev)
        self.y = torch.empty((T, D), dtype=bf, device=dev)
        self.dh = torch.empty((T, H), dtype=bf, device=dev)
        self.dzq = _q_out((), T, 2 * H, dev)
        self.dx = torch.empty((T, D), dtype=bf, device=dev)
        self.dw2 = torch.empty((D, H), dtype=wgrad_dtype, device=dev)
        self.dw13 = torch.empty((2 * H, D), dtype=wgrad_dtype, device=dev)

    def step(self, x, w13, w2, dy, quantize_weights=True):
        """One forward + backward; returns (dx, dW13, dW2). With
        quantize_weights=False the weights' MXFP8 copies from the previous
        step are reused (valid while the weights are unchanged, i.e. between
        optimizer steps)."""
        for st in self.stages(x, w13, w2, dy, quantize_weights):
            st.fn()
        return self.dx, self.dw13, self.dw2

    def stages(self, x, w13, w2, dy, quantize_weights=True):
        """The step as an ordered list of Stage (same calls as step())."""
        return _weights_cached(self._stages(x, w13, w2, dy), quantize_weights)

    def _stages(self, x, w13, w2, dy):
        T, D, H, m = self.T, self.D, self.H, self.mode
        z0, z1 = self.z[:, :H], self.z[:, H:]
        return [
            Stage("quant_x", "k_quant_tile", 0, _qbytes(T * D, True),
                  lambda: mx.quantize(x, m, True, True, out=self.qx)),
            Stage("quant_w13", "k_quant_tile", 0, _qbytes(2 * H * D, True),
                  lambda: mx.quantize(w13, m, True, True, out=self.q13)),
            Stage("quant_w2", "k_quant_tile", 0, _qbytes(D * H, True),
                  lambda: mx.quantize(w2, m, True, True, out=self.q2)),
            Stage("gemm_w13_fwd", "k_gemm_dense", 2 * T * 2 * H * D, 0,
                  lambda: mx.scaled_mm(self.qx["q_row"], self.qx["s_row"], self.q13["q_row"],
                                       self.q13["s_row"], out=self.z)),
            Stage("swiglu_fwd", "k_swiglu_fwd", 0, T * H * (4 + 2 * (1 + 1 / 32)),
                  lambda: mx.swiglu_quant_fwd(z0, z1, m, out=self.hq)),
            Stage("gemm_w2_fwd", "k_gemm_dense", 2 * T * D * H, 0,
                  lambda: mx.scaled_mm(self.hq["q_row"], self.hq["s_row"], self.q2["q_row"],
                                       self.q2["s_row"], out=self.y)),
            Stage("quant_dy", "k_quant_tile", 0, _qbytes(T * D, True),
                  lambda: mx.quantize(dy, m, True, True, out=self.qdy)),
            # backward in the order described at _stages of MoEMLP
            Stage("gemm_w2_dgrad", "k_gemm_dense", 2 * T * D * H, 0,
                  lambda: mx.scaled_mm(self.qdy["q_row"], self.qdy["s_row"], self.q2["q_col"],
                                       self.q2["s_col"], out=self.dh)),
            Stage("swiglu_bwd", "k_swiglu_bwd", 0, T * H * (6 + 4 * (1 + 1 / 32)),
                  lambda: mx.swiglu_quant_bwd(self.dh, z0, z1, m, out=self.dzq)),
            Stage("gemm_w2_wgrad", "k_gemm_dense", 2 * T * D * H, 0,
                  lambda: mx.scaled_mm(self.qdy["q_col"], self.qdy["s_col"], self.hq["q_col"],
                                       self.hq["s_col"], out=self.dw2)),
            Stage("gemm_w13_wgrad", "k_gemm_dense", 2 * T * 2 * H * D, 0,
                  lambda: mx.scaled_mm(self.dzq["q_col"], self.dzq["s_col"], self.qx["q_col"],
                                       self.qx["s_col"], out=self.dw13)),
            Stage("gemm_w13_dgrad", "k_gemm_dense", 2 * T * 2 * H * D, 0,
                  lambda: mx.scaled_mm(self.dzq["q_row"], self.dzq["s_row"], self.q13["q_col"],
                                       self.q13["s_col"], out=self.dx)),
        ]

    def gemm_flops(self):
        return 18 * self.T * self.D * self.H

    def gemm_bytes(self):
        """Algorithmic HBM bytes of each GEMM stage: both MX operands (codes
        and scales) read once and the output written once."""
        T, D, H = self.T, self.D, self.H
        w = self.dw2.element_size()
        return {"gemm_w13_fwd": _mxb(T, D) + _mxb(2 * H, D) + 2 * T * 2 * H,
                "gemm_w2_fwd": _mxb(T, H) + _mxb(D, H) + 2 * T * D,
                "gemm_w2_dgrad": _mxb(T, D) + _mxb(H, D) + 2 * T * H,
                "gemm_w2_wgrad": _mxb(D, T) + _mxb(H, T) + w * D * H,
                "gemm_w13_dgrad": _mxb(T, 2 * H) + _mxb(D, 2 * H) + 2 * T * D,
                "gemm_w13_wgrad": _mxb(2 * H, T) + _mxb(D, T) + w * 2 * H * D}


def _mxb(R, C):
    """Bytes of an MX operand [R, C]: one code per element, one scale per 32."""
    return R * C * (1 + 1 / 32)


class MoEMLP:
    """Buffers and step of the routed-experts MXFP8 SwiGLU MLP: E experts,
    T routed tokens (expert-major), dim D, expert hidden H, groups padded to
    `multiple` rows inside a capacity of Tcap rows."""

    def __init__(self, E, T, D, H, Tcap, device, mode="rceil", wgrad="mx", wgrad_dtype=torch.float32,
                 multiple=128, recipe="mxfp8"):
        self.E, self.T, self.D, self.H, self.Tcap = E, T, D, H, Tcap
        self.mode, self.wgrad, self.multiple, self.recipe = mode, wgrad, multiple, recipe
        dev = device
        bf = torch.bfloat16
        fp8 = recipe == "fp8_rowwise"
        if fp8:
            wgrad = self.wgrad = "mx"   # the FP8 weight gradients run on FP8 operands
        mxw = wgrad == "mx" and not fp8
        # bf16 padded copies exist only for the hp weight gradient; the MXFP8
        # recipe pads while it quantizes
        self.x_pad = None if mxw else torch.empty((Tcap, D), dtype=bf, device=dev)
        self.dy_pad = None if mxw else torch.empty((Tcap, D), dtype=bf, device=dev)
        if fp8:
            # FP8 row-scaled operands of h and dA|dB, quantized from their bf16 values
            self.qh8 = _q_out((), Tcap, H, dev)
            self.qdz8 = _q_out((), Tcap, 2 * H, dev)
        self.offs = torch.empty((E,), dtype=torch.int32, device=dev)
        self.src = torch.empty((Tcap,), dtype=torch.int32, device=dev)
        self.offs2 = torch.empty((E,), dtype=torch.int32, device=dev)
        self.src2 = torch.empty((Tcap,), dtype=torch.int32, device=dev)
        self.err = torch.zeros((1,), dtype=torch.int32, device=dev)
        self.qx = _q_out((), Tcap, D, dev, True, mxw or fp8)
        self.q13 = _q_out((E,), 2 * H, D, dev)
        self.q2 = _q_out((E,), D, H, dev)
        self.qdy = _q_out((), Tcap, D, dev, True, mxw or fp8)
        self.z = torch.empty((Tcap, 2 * H), dtype=bf, device=dev)
        self.hq = _q_out((), Tcap, H, dev)
        if not mxw:
            self.hq["h"] = torch.empty((Tcap, H), dtype=bf, device=dev)
        self.y = torch.empty((T, D), dtype=bf, device=dev)
        self.dh = torch.empty((Tcap, H), dtype=bf, device=dev)
        self.dzq = _q_out((), Tcap, 2 * H, dev)
        if not mxw:
            self.dzq["dab"] = torch.empty((Tcap, 2 * H), dtype=bf, device=dev)
        self.dx = torch.empty((T, D), dtype=bf, device=dev)
        wdt = wgrad_dtype if mxw or fp8 else bf
        self.dw2 = torch.empty((E, D, H), dtype=wdt, device=dev)
        self.dw13 = torch.empty((E, 2 * H, D), dtype=wdt, device=dev)

    def step(self, x, sizes, w13, w2, dy, quantize_weights=True):
        """One forward + backward; returns (dx, dW13, dW2). With
        quantize_weights=False the experts' MXFP8 weight copies from the
        previous step are reused (valid between optimizer steps)."""
        for st in self.stages(x, sizes, w13, w2, dy, quantize_weights):
            st.fn()
        return self.dx, self.dw13, self.dw2

    def stages(self, x, sizes, w13, w2, dy, quantize_weights=True):
        """The step as an ordered list of Stage (same calls as step()).
        GEMM flops count real tokens only; padded rows are executed but not
        counted."""
        return _weights_cached(self._stages(x, sizes, w13, w2, dy), quantize_weights)

    def _stages(self, x, sizes, w13, w2, dy):
        if self.recipe == "fp8_rowwise":
            return self._stages_fp8(x, sizes, w13, w2, dy)
        E, T, D, H, Tc, m = self.E, self.T, self.D, self.H, self.Tcap, self.mode
        mxw = self.wgrad == "mx"
        z0, z1 = self.z[:, :H], self.z[:, H:]
        err = self.err
        if mxw:
            # padding fused into the dual quantization (k_pad_map + k_quant_tile)
            st = [Stage("pad_quant_x", "k_quant_tile", 0, _pad_qbytes(T, Tc, D),
                        lambda: mx.pad_quantize(x, sizes, Tc, m, True, True, multiple=self.multiple,
                                                out=dict(self.qx, offs=self.offs, src_row=self.src),
                                                dev_err=err))]
        else:
            st = [Stage("pad_x", "k_pad", 0, 2 * T * D + 2 * Tc * D,
                        lambda: mx.pad_groups(x, sizes, Tc, self.multiple,
                                              out=dict(x_pad=self.x_pad, offs=self.offs, src_row=self.src),
                                              dev_err=err)),
                  Stage("quant_x", "k_quant_tile", 0, _qbytes(Tc * D, False),
                        lambda: mx.quantize(self.x_pad, m, True, False, out=self.qx))]
        st += [
            Stage("quant_w13", "k_quant_tile", 0, _qbytes(E * 2 * H * D, True),
                  lambda: mx.quantize(w13, m, True, True, out=self.q13)),
            Stage("quant_w2", "k_quant_tile", 0, _qbytes(E * D * H, True),
                  lambda: mx.quantize(w2, m, True, True, out=self.q2)),
            Stage("gemm_w13_fwd", "k_gemm_grouped", 2 * T * 2 * H * D, 0,
                  lambda: mx.grouped_mm_fwd(self.qx["q_row"], self.qx["s_row"], self.q13["q_row"],
                                            self.q13["s_row"], self.offs, out=self.z, dev_err=err)),
            Stage("swiglu_fwd", "k_swiglu_fwd", 0, Tc * H * (4 + 2 * (1 + 1 / 32) + (0 if mxw else 2)),
                  lambda: mx.swiglu_quant_fwd(z0, z1, m, want_h=not mxw, out=self.hq)),
            # y straight in token order: the GEMM drops the pad rows itself
            Stage("gemm_w2_fwd", "k_gemm_grouped", 2 * T * D * H, 0,
                  lambda: mx.grouped_mm_fwd_unpad(self.hq["q_row"], self.hq["s_row"], self.q2["q_row"],
                                                  self.q2["s_row"], self.offs, sizes, T, out=self.y, dev_err=err)),
        ]
        if mxw:
            st.append(Stage("pad_quant_dy", "k_quant_tile", 0, _pad_qbytes(T, Tc, D),
                            lambda: mx.pad_quantize(dy, sizes, Tc, m, True, True, multiple=self.multiple,
                                                    out=dict(self.qdy, offs=self.offs2, src_row=self.src2),
                                                    dev_err=err)))
        else:
            st += [Stage("pad_dy", "k_pad", 0, 2 * T * D + 2 * Tc * D,
                         lambda: mx.pad_groups(dy, sizes, Tc, self.multiple,
                                               out=dict(x_pad=self.dy_pad, offs=self.offs2, src_row=self.src2),
                                               dev_err=err)),
                   Stage("quant_dy", "k_quant_tile", 0, _qbytes(Tc * D, False),
                         lambda: mx.quantize(self.dy_pad, m, True, False, out=self.qdy))]
        # Backward: w2 dgrad, the SwiGLU backward, both weight gradients, and
        # the w13 dgrad last. Each weight gradient writes its whole dW, and the
        # kernel after it pays for writing back those lines from the caches:
        # a GEMM hides that under its arithmetic, a bandwidth-bound kernel (the
        # SwiGLU backward, or the next step's weight quantization) does not.
        st += [
            Stage("gemm_w2_dgrad", "k_gemm_grouped", 2 * T * D * H, 0,
                  lambda: mx.grouped_mm_dgrad(self.qdy["q_row"], self.qdy["s_row"], self.q2["q_col"],
                                              self.q2["s_col"], self.offs, out=self.dh, dev_err=err)),
            Stage("swiglu_bwd", "k_swiglu_bwd", 0, Tc * H * (6 + 4 * (1 + 1 / 32) + (0 if mxw else 4)),
                  lambda: mx.swiglu_quant_bwd(self.dh, z0, z1, m, want_dab=not mxw, out=self.dzq)),
        ]
        if mxw:
            st += [
                Stage("gemm_w2_wgrad", "k_gemm_wgrad", 2 * T * D * H, 0,
                      lambda: mx.grouped_mm_wgrad(self.qdy["q_col"], self.qdy["s_col"], self.hq["q_col"],
                                                  self.hq["s_col"], self.offs, out=self.dw2, dev_err=err)),
                Stage("gemm_w13_wgrad", "k_gemm_wgrad", 2 * T * 2 * H * D, 0,
                      lambda: mx.grouped_mm_wgrad(self.dzq["q_col"], self.dzq["s_col"], self.qx["q_col"],
                                                  self.qx["s_col"], self.offs, out=self.dw13, dev_err=err)),
            ]
        else:
            st += [
                Stage("gemm_w2_wgrad_hp", "k_gemm_wgrad_hp", 2 * T * D * H, 0,
                      lambda: mx.grouped_mm_wgrad_hp(self.dy_pad, self.hq["h"], self.offs, out=self.dw2,
                                                     dev_err=err)),
                Stage("gemm_w13_wgrad_hp", "k_gemm_wgrad_hp", 2 * T * 2 * H * D, 0,
                      lambda: mx.grouped_mm_wgrad_hp(self.dzq["dab"], self.x_pad, self.offs, out=self.dw13,
                                                     dev_err=err)),
            ]
        st.append(Stage("gemm_w13_dgrad", "k_gemm_grouped", 2 * T * 2 * H * D, 0,
                        lambda: mx.grouped_mm_dgrad_unpad(self.dzq["q_row"], self.dzq["s_row"], self.q13["q_col"],
                                                          self.q13["s_col"], self.offs, sizes, T, out=self.dx,
                                                          dev_err=err)))
        return st

    def _stages_fp8(self, x, sizes, w13, w2, dy):
        """The step with FP8 row-scaled operands (one power-of-two scale per
        row; the weight-gradient operands per column and group): the same
        grouped GEMMs, with the quantizations done by the FP8 kernels from
        bf16 tensors (h and dA|dB kept in bf16 for them)."""
        E, T, D, H, Tc, m = self.E, self.T, self.D, self.H, self.Tcap, self.mode
        z0, z1 = self.z[:, :H], self.z[:, H:]
        err = self.err
        fq = mx.quantize_fp8
        return [
            Stage("pad_x", "k_pad", 0, 2 * T * D + 2 * Tc * D,
                  lambda: mx.pad_groups(x, sizes, Tc, self.multiple,
                                        out=dict(x_pad=self.x_pad, offs=self.offs, src_row=self.src),
                                        dev_err=err)),
            Stage("fp8_x", "k_fp8", 0, _qbytes(Tc * D, True) + 2 * Tc * D,
                  lambda: fq(self.x_pad, True, True, offs=self.offs, out=self.qx, dev_err=err)),
            Stage("fp8_w13", "k_fp8", 0, _qbytes(E * 2 * H * D, True) + 2 * E * 2 * H * D,
                  lambda: fq(w13, True, True, out=self.q13)),
            Stage("fp8_w2", "k_fp8", 0, _qbytes(E * D * H, True) + 2 * E * D * H,
                  lambda: fq(w2, True, True, out=self.q2)),
            Stage("gemm_w13_fwd", "k_gemm_grouped", 2 * T * 2 * H * D, 0,
                  lambda: mx.grouped_mm_fwd(self.qx["q_row"], self.qx["s_row"], self.q13["q_row"],
                                            self.q13["s_row"], self.offs, out=self.z, dev_err=err)),
            Stage("swiglu_fwd", "k_swiglu_fwd", 0, Tc * H * (4 + 2 * (1 + 1 / 32) + 2),
                  lambda: mx.swiglu_quant_fwd(z0, z1, m, want_h=True, out=self.hq)),
            Stage("fp8_h", "k_fp8", 0, _qbytes(Tc * H, True) + 2 * Tc * H,
                  lambda: fq(self.hq["h"], True, True, offs=self.offs, out=self.qh8, dev_err=err)),
            Stage("gemm_w2_fwd", "k_gemm_grouped", 2 * T * D * H, 0,
                  lambda: mx.grouped_mm_fwd_unpad(self.qh8["q_row"], self.qh8["s_row"], self.q2["q_row"],
                                                  self.q2["s_row"], self.offs, sizes, T, out=self.y, dev_err=err)),
            Stage("pad_dy", "k_pad", 0, 2 * T * D + 2 * Tc * D,
                  lambda: mx.pad_groups(dy, sizes, Tc, self.multiple,
                                        out=dict(x_pad=self.dy_pad, offs=self.offs2, src_row=self.src2),
                                        dev_err=err)),
            Stage("fp8_dy", "k_fp8", 0, _qbytes(Tc * D, True) + 2 * Tc * D,
                  lambda: fq(self.dy_pad, True, True, offs=self.offs, out=self.qdy, dev_err=err)),
            Stage("gemm_w2_dgrad", "k_gemm_grouped", 2 * T * D * H, 0,
                  lambda: mx.grouped_mm_dgrad(self.qdy["q_row"], self.qdy["s_row"], self.q2["q_col"],
                                              self.q2["s_col"], self.offs, out=self.dh, dev_err=err)),
            # backward in the order described at _stages
            Stage("swiglu_bwd", "k_swiglu_bwd", 0, Tc * H * (6 + 4 * (1 + 1 / 32) + 4),
                  lambda: mx.swiglu_quant_bwd(self.dh, z0, z1, m, want_dab=True, out=self.dzq)),
            Stage("fp8_dz", "k_fp8", 0, _qbytes(Tc * 2 * H, True) + 2 * Tc * 2 * H,
                  lambda: fq(self.dzq["dab"], True, True, offs=self.offs, out=self.qdz8, dev_err=err)),
            Stage("gemm_w2_wgrad", "k_gemm_wgrad", 2 * T * D * H, 0,
                  lambda: mx.grouped_mm_wgrad(self.qdy["q_col"], self.qdy["s_col"], self.qh8["q_col"],
                                              self.qh8["s_col"], self.offs, out=self.dw2, dev_err=err)),
            Stage("gemm_w13_wgrad", "k_gemm_wgrad", 2 * T * 2 * H * D, 0,
                  lambda: mx.grouped_mm_wgrad(self.qdz8["q_col"], self.qdz8["s_col"], self.qx["q_col"],
                                              self.qx["s_col"], self.offs, out=self.dw13, dev_err=err)),
            Stage("gemm_w13_dgrad", "k_gemm_grouped", 2 * T * 2 * H * D, 0,
                  lambda: mx.grouped_mm_dgrad_unpad(self.qdz8["q_row"], self.qdz8["s_row"], self.q13["q_col"],
                                                    self.q13["s_col"], self.offs, sizes, T, out=self.dx,
                                                    dev_err=err)),
        ]

    def gemm_flops(self):
        """Useful GEMM flops of one step (real tokens only)."""
        return 18 * self.T * self.D * self.H

    def gemm_bytes(self):
        """Algorithmic HBM bytes of each GEMM stage: operands read once over
        the padded capacity (the layout the kernels read), all experts'
        weights, outputs written once (y and dx in token order; every
        expert's dW, the empty ones as zeros)."""
        E, T, D, H, Tc = self.E, self.T, self.D, self.H, self.Tcap
        w = self.dw2.element_size()
        b = {"gemm_w13_fwd": _mxb(Tc, D) + E * _mxb(2 * H, D) + 2 * Tc * 2 * H,
             "gemm_w2_fwd": _mxb(Tc, H) + E * _mxb(D, H) + 2 * T * D,
             "gemm_w2_dgrad": _mxb(Tc, D) + E * _mxb(H, D) + 2 * Tc * H,
             "gemm_w13_dgrad": _mxb(Tc, 2 * H) + E * _mxb(D, 2 * H) + 2 * T * D,
             "gemm_w2_wgrad": _mxb(D, Tc) + _mxb(H, Tc) + w * E * D * H,
             "gemm_w13_wgrad": _mxb(2 * H, Tc) + _mxb(D, Tc) + w * E * 2 * H * D,
             "gemm_w2_wgrad_hp": 2 * Tc * D + 2 * Tc * H + w * E * D * H,
             "gemm_w13_wgrad_hp": 2 * Tc * 2 * H + 2 * Tc * D + w * E * 2 * H * D}
        return b
