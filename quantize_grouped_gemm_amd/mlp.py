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
The grouped variant pads each expert's tokens to a multiple of 128 first,
runs the grouped GEMMs over the padded offsets and unpads y and dx.

Every buffer is allocated once per shape by the workspace classes, so a
training step only enqueues kernels. The weight-gradient GEMMs run in MXFP8
(float32 dW) or, with wgrad="hp" (the wgrad_with_hp recipe), on the bf16
operands (bf16 dW).
"""

import torch

from . import mx


def _q_out(lead, R, C, dev, row=True, col=True):
    o = {}
    if row:
        o["q_row"] = torch.empty(lead + (R, C), dtype=torch.uint8, device=dev)
        o["s_row"] = torch.empty(lead + (R, C // 32), dtype=torch.uint8, device=dev)
    if col:
        o["q_col"] = torch.empty(lead + (C, R), dtype=torch.uint8, device=dev)
        o["s_col"] = torch.empty(lead + (C, R // 32), dtype=torch.uint8, device=dev)
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

    def forward(self, x, w13, w2):
        H, m = self.H, self.mode
        mx.quantize(x, m, True, True, out=self.qx)
        mx.quantize(w13, m, True, True, out=self.q13)
        mx.quantize(w2, m, True, True, out=self.q2)
        mx.scaled_mm(self.qx["q_row"], self.qx["s_row"], self.q13["q_row"], self.q13["s_row"], out=self.z)
        mx.swiglu_quant_fwd(self.z[:, :H], self.z[:, H:], m, out=self.hq)
        mx.scaled_mm(self.hq["q_row"], self.hq["s_row"], self.q2["q_row"], self.q2["s_row"], out=self.y)
        return self.y

    def backward(self, dy):
        H, m = self.H, self.mode
        mx.quantize(dy, m, True, True, out=self.qdy)
        mx.scaled_mm(self.qdy["q_row"], self.qdy["s_row"], self.q2["q_col"], self.q2["s_col"], out=self.dh)
        mx.scaled_mm(self.qdy["q_col"], self.qdy["s_col"], self.hq["q_col"], self.hq["s_col"], out=self.dw2)
        mx.swiglu_quant_bwd(self.dh, self.z[:, :H], self.z[:, H:], m, out=self.dzq)
        mx.scaled_mm(self.dzq["q_row"], self.dzq["s_row"], self.q13["q_col"], self.q13["s_col"], out=self.dx)
        mx.scaled_mm(self.dzq["q_col"], self.dzq["s_col"], self.qx["q_col"], self.qx["s_col"], out=self.dw13)
        return self.dx, self.dw13, self.dw2

    def step(self, x, w13, w2, dy):
        self.forward(x, w13, w2)
        return self.backward(dy)

    def gemm_flops(self):
        return 18 * self.T * self.D * self.H


class MoEMLP:
    """Buffers and step of the routed-experts MXFP8 SwiGLU MLP: E experts,
    T routed tokens (expert-major), dim D, expert hidden H, groups padded to
    `multiple` rows inside a capacity of Tcap rows."""

    def __init__(self, E, T, D, H, Tcap, device, mode="rceil", wgrad="mx", wgrad_dtype=torch.float32,
                 multiple=128):
        self.E, self.T, self.D, self.H, self.Tcap = E, T, D, H, Tcap
        self.mode, self.wgrad, self.multiple = mode, wgrad, multiple
        dev = device
        bf = torch.bfloat16
        mxw = wgrad == "mx"
        self.x_pad = torch.empty((Tcap, D), dtype=bf, device=dev)
        self.dy_pad = torch.empty((Tcap, D), dtype=bf, device=dev)
        self.offs = torch.empty((E,), dtype=torch.int32, device=dev)
        self.src = torch.empty((Tcap,), dtype=torch.int32, device=dev)
        self.offs2 = torch.empty((E,), dtype=torch.int32, device=dev)
        self.src2 = torch.empty((Tcap,), dtype=torch.int32, device=dev)
        self.err = torch.zeros((1,), dtype=torch.int32, device=dev)
        self.qx = _q_out((), Tcap, D, dev, True, mxw)
        self.q13 = _q_out((E,), 2 * H, D, dev)
        self.q2 = _q_out((E,), D, H, dev)
        self.qdy = _q_out((), Tcap, D, dev, True, mxw)
        self.z = torch.empty((Tcap, 2 * H), dtype=bf, device=dev)
        self.hq = _q_out((), Tcap, H, dev)
        if not mxw:
            self.hq["h"] = torch.empty((Tcap, H), dtype=bf, device=dev)
        self.y_pad = torch.empty((Tcap, D), dtype=bf, device=dev)
        self.y = torch.empty((T, D), dtype=bf, device=dev)
        self.dh = torch.empty((Tcap, H), dtype=bf, device=dev)
        self.dzq = _q_out((), Tcap, 2 * H, dev)
        if not mxw:
            self.dzq["dab"] = torch.empty((Tcap, 2 * H), dtype=bf, device=dev)
        self.dx_pad = torch.empty((Tcap, D), dtype=bf, device=dev)
        self.dx = torch.empty((T, D), dtype=bf, device=dev)
        wdt = wgrad_dtype if mxw else bf
        self.dw2 = torch.empty((E, D, H), dtype=wdt, device=dev)
        self.dw13 = torch.empty((E, 2 * H, D), dtype=wdt, device=dev)

    def forward(self, x, sizes, w13, w2):
        H, m = self.H, self.mode
        mxw = self.wgrad == "mx"
        mx.pad_groups(x, sizes, self.Tcap, self.multiple,
                      out=dict(x_pad=self.x_pad, offs=self.offs, src_row=self.src), dev_err=self.err)
        mx.quantize(self.x_pad, m, True, mxw, out=self.qx)
        mx.quantize(w13, m, True, True, out=self.q13)
        mx.quantize(w2, m, True, True, out=self.q2)
        mx.grouped_mm_fwd(self.qx["q_row"], self.qx["s_row"], self.q13["q_row"], self.q13["s_row"],
                          self.offs, out=self.z, dev_err=self.err)
        mx.swiglu_quant_fwd(self.z[:, :H], self.z[:, H:], m, want_h=not mxw, out=self.hq)
        mx.grouped_mm_fwd(self.hq["q_row"], self.hq["s_row"], self.q2["q_row"], self.q2["s_row"],
                          self.offs, out=self.y_pad, dev_err=self.err)
        mx.unpad_groups(self.y_pad, self.src, self.T, out=self.y)
        return self.y

    def backward(self, dy, sizes):
        H, m = self.H, self.mode
        mxw = self.wgrad == "mx"
        mx.pad_groups(dy, sizes, self.Tcap, self.multiple,
                      out=dict(x_pad=self.dy_pad, offs=self.offs2, src_row=self.src2), dev_err=self.err)
        mx.quantize(self.dy_pad, m, True, mxw, out=self.qdy)
        mx.grouped_mm_dgrad(self.qdy["q_row"], self.qdy["s_row"], self.q2["q_col"], self.q2["s_col"],
                            self.offs, out=self.dh, dev_err=self.err)
        if mxw:
            mx.grouped_mm_wgrad(self.qdy["q_col"], self.qdy["s_col"], self.hq["q_col"], self.hq["s_col"],
                                self.offs, out=self.dw2, dev_err=self.err)
        else:
            mx.grouped_mm_wgrad_hp(self.dy_pad, self.hq["h"], self.offs, out=self.dw2, dev_err=self.err)
        mx.swiglu_quant_bwd(self.dh, self.z[:, :H], self.z[:, H:], m, want_dab=not mxw, out=self.dzq)
        mx.grouped_mm_dgrad(self.dzq["q_row"], self.dzq["s_row"], self.q13["q_col"], self.q13["s_col"],
                            self.offs, out=self.dx_pad, dev_err=self.err)
        mx.unpad_groups(self.dx_pad, self.src, self.T, out=self.dx)
        if mxw:
            mx.grouped_mm_wgrad(self.dzq["q_col"], self.dzq["s_col"], self.qx["q_col"], self.qx["s_col"],
                                self.offs, out=self.dw13, dev_err=self.err)
        else:
            mx.grouped_mm_wgrad_hp(self.dzq["dab"], self.x_pad, self.offs, out=self.dw13, dev_err=self.err)
        return self.dx, self.dw13, self.dw2

    def step(self, x, sizes, w13, w2, dy):
        self.forward(x, sizes, w13, w2)
        return self.backward(dy, sizes)

    def gemm_flops(self):
        """Useful GEMM flops of one step (real tokens only)."""
        return 18 * self.T * self.D * self.H
