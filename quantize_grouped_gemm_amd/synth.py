"""Seeded synthetic inputs for the MXFP8 training hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so both the GPU path's tests and the CPU oracle's tests
can take their inputs from it.

Workloads (all synthetic; no datasets or trained weights are involved):
  * single MXFP8 linear: x [256, 512] ~ N(0, 1), W [256, 512] ~ N(0, 0.02)
  * dense SwiGLU MLP shaped like Llama-3-8B: T=8192, D=4096, H=14336
  * routed-experts MLP, one GPU's share of a Llama4-Scout-like MoE: E=16,
    D=5120, H=8192, T=16384 top-1 tokens, Zipf(1.1) group sizes over 14 of the
    16 experts (two are empty)
  * fine-grained MoE, one GPU's share of a DeepSeek-V3-like model: E=32,
    D=7168, H=2048, 65536 token slots (8192 tokens x top-8), group sizes
    multinomial over Dirichlet(0.3) expert probabilities
  * quantization stress tensor [32768, 7168]: N(0, 1) with planted outliers,
    zero blocks, subnormals and values exactly at the E4M3 maximum.

bf16 tensors are drawn in float32 and rounded to bf16 by torch's
round-to-nearest-even cast.
"""

import numpy as np
import torch

LINEAR_SHAPE = dict(M=256, N=256, K=512)
DENSE_MLP = dict(T=8192, D=4096, H=14336)
MOE_SCOUT = dict(E=16, D=5120, H=8192, T=16384)
MOE_DSV3 = dict(E=32, D=7168, H=2048, T=65536)
STRESS_SHAPE = (32768, 7168)
PAD_MULTIPLE = 128


def bits(t):
    """bf16 torch tensor (any device) -> numpy uint16 bit patterns on host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def from_bits(b, device="cpu"):
    """numpy uint16 bit patterns -> bf16 torch tensor on ``device``."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(device)


def generator(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_bf16(shape, std=1.0, gen=None, device="cpu"):
    """bf16 tensor ~ N(0, std^2), drawn in float32 on ``device``."""
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def capacity(T, E, multiple=PAD_MULTIPLE):
    """Worst-case row count after padding every group of a T-token, E-group
    batch up to ``multiple`` rows, rounded up to ``multiple``."""
    return -(-(T + E * (multiple - 1)) // multiple) * multiple


def zipf_group_sizes(T, E, n_active, s=1.1, seed=0):
    """Zipf(s) expert probabilities over ranks 1..n_active, multinomial(T)
    counts, assigned to a seeded choice of n_active of the E experts; the
    other E - n_active experts get no tokens."""
    rng = np.random.default_rng(seed)
    p = np.arange(1, n_active + 1, dtype=np.float64) ** (-s)
    counts = rng.multinomial(T, p / p.sum())
    ids = rng.permutation(E)[:n_active]
    sizes = np.zeros(E, np.int64)
    sizes[ids] = counts
    return sizes


def dirichlet_group_sizes(T, E, alpha=0.3, seed=0):
    """Expert probabilities ~ Dirichlet(alpha * 1_E), counts ~ multinomial(T)."""
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(E, alpha))
    return rng.multinomial(T, p).astype(np.int64)


def linear_inputs(seed=0, device="cpu", M=256, N=256, K=512):
    g = generator(seed, device)
    x = normal_bf16((M, K), 1.0, g, device)
    w = normal_bf16((N, K), 0.02, g, device)
    return x, w


def mlp_inputs(T, D, H, E=None, seed=0, device="cpu"):
    """x [T, D] ~ N(0,1); w1, w3 [(E,) H, D] and w2 [(E,) D, H] ~ N(0, 0.02);
    dy [T, D] ~ N(0, 1). Draw order: x, w1, w3, w2, dy."""
    g = generator(seed, device)
    lead = () if E is None else (E,)
    x = normal_bf16((T, D), 1.0, g, device)
    w1 = normal_bf16(lead + (H, D), 0.02, g, device)
    w3 = normal_bf16(lead + (H, D), 0.02, g, device)
    w2 = normal_bf16(lead + (D, H), 0.02, g, device)
    dy = normal_bf16((T, D), 1.0, g, device)
    return x, w1, w3, w2, dy


def stress_tensor(R=STRESS_SHAPE[0], C=STRESS_SHAPE[1], seed=0, device="cpu"):
    """Quantization stress tensor (bf16 [R, C], R and C multiples of 32).

    Base N(0, 1) drawn on ``device``; the planted structure is chosen by a
    numpy generator so it is the same on every device. Planted in this order
    (later writes win):
      1. 0.1% of positions: outliers +-2**u, u uniform in {10..14};
      2. 64 row-blocks, 64 column-blocks and one 32x32 tile set to +0, and one
         row-block set to -0;
      3. 0.01% of positions: random bf16 subnormals (either sign), plus 16
         row-blocks and 16 column-blocks made only of subnormals;
      4. 0.01% of positions exactly +-448;
      5. 64 row-blocks whose maximum magnitude is exactly 448 * 2**k and 64
         whose maximum is one bf16 step above 1.75 * 2**k (k in -20..20).
    A row-block is 32 consecutive elements of a row, a column-block 32
    consecutive elements of a column, both 32-aligned.
    """
    assert R % 32 == 0 and C % 32 == 0
    rng = np.random.default_rng(seed)
    g = generator(seed, device)
    x = torch.randn((R, C), generator=g, device=device, dtype=torch.float32)
    flat = x.view(-1)
    n = R * C

    def last_wins(idx):
        # positions drawn twice keep the later value; a parallel scatter would
        # pick either, so duplicates are resolved here, before it
        _, rev = np.unique(idx[::-1], return_index=True)
        return idx.size - 1 - rev

    def put(idx, vals):
        keep = last_wins(idx)
        flat[torch.as_tensor(idx[keep], device=device)] = torch.as_tensor(
            np.asarray(vals)[keep], dtype=torch.float32, device=device)

    k = max(1, n // 1000)
    idx = rng.integers(0, n, k)
    put(idx, rng.choice([-1.0, 1.0], k) * np.exp2(rng.integers(10, 15, k)))

    def row_blocks(m):
        r = rng.integers(0, R, m)
        b = rng.integers(0, C // 32, m)
        return r, b

    def col_blocks(m):
        c = rng.integers(0, C, m)
        b = rng.integers(0, R // 32, m)
        return c, b

    r, b = row_blocks(64)
    for i in range(64):
        x[r[i], 32 * b[i]:32 * b[i] + 32] = 0.0
    c, b = col_blocks(64)
    for i in range(64):
        x[32 * b[i]:32 * b[i] + 32, c[i]] = 0.0
    tr, tc = rng.integers(0, R // 32), rng.integers(0, C // 32)
    x[32 * tr:32 * tr + 32, 32 * tc:32 * tc + 32] = 0.0
    r, b = row_blocks(1)
    x[r[0], 32 * b[0]:32 * b[0] + 32] = -0.0

    xb = x.to(torch.bfloat16)
    xi = xb.view(torch.int16).view(-1)

    def sub_bits(m):
        mag = rng.integers(1, 0x80, m)
        sign = rng.integers(0, 2, m) << 15
        v = (mag | sign).astype(np.uint16).view(np.int16)
        return torch.as_tensor(v, device=device)

    k2 = max(1, n // 10000)
    idx = rng.integers(0, n, k2)
    keep = last_wins(idx)
    xi[torch.as_tensor(idx[keep], device=device)] = sub_bits(k2)[torch.as_tensor(keep, device=device)]
    xi2 = xi.view(R, C)
    r, b = row_blocks(16)
    for i in range(16):
        xi2[r[i], 32 * b[i]:32 * b[i] + 32] = sub_bits(32)
    c, b = col_blocks(16)
    for i in range(16):
        xi2[32 * b[i]:32 * b[i] + 32, c[i]] = sub_bits(32)

    # exactly +-448 (bf16 0x43E0)
    idx = rng.integers(0, n, k2)
    v448 = np.where(rng.integers(0, 2, k2) == 1, 0xC3E0, 0x43E0).astype(np.uint16).view(np.int16)
    keep = last_wins(idx)
    xi[torch.as_tensor(idx[keep], device=device)] = torch.as_tensor(v448[keep], device=device)

    def exp_bits(kk, mant):
        # bf16 with exponent field 127 + kk and 7-bit mantissa ``mant``
        return ((127 + kk) << 7) | mant

    r, b = row_blocks(128)
    ks = rng.integers(-20, 21, 128)
    for i in range(128):
        kk = int(ks[i])
        # the block maximum: 448 * 2**k (first 64) or 1.7578125 * 2**k, the
        # bf16 value one step above 1.75 * 2**k (last 64)
        top = exp_bits(kk + 8, 0x60) if i < 64 else exp_bits(kk, 0x61)
        # the other 31 elements: random bf16 magnitudes strictly below it
        # (bit patterns of non-negative bf16 values order like the values)
        small = rng.integers(0, top, 32)
        small = small | (rng.integers(0, 2, 32) << 15)
        small[int(rng.integers(0, 32))] = top | (int(rng.integers(0, 2)) << 15)
        blk = torch.as_tensor(small.astype(np.uint16).view(np.int16), device=device)
        xi2[r[i], 32 * b[i]:32 * b[i] + 32] = blk
    return xb
