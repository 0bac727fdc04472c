"""Seeded synthetic workloads for the attention forward.

This module only draws inputs: it holds the workload table (shapes, dtypes,
value distributions, masks, seeds) and a generator. It contains none of the
attention arithmetic, so both the HIP path's tests and the CPU oracle can take
their inputs from here without sharing any computation.

Every tensor is drawn in float32 from a CPU ``torch.Generator`` seeded per
workload, in the order Q, K, V (then the key lengths), and only then rounded
to the workload's input dtype (round-to-nearest-even). The rounded values are
what both sides receive.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
          "e4m3": torch.float8_e4m3fn}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    in_dtype: str            # "f32" | "bf16" | "f16" | "e4m3"
    out_dtype: str           # dtype of O; LSE is always float32
    causal: bool
    q_dist: tuple            # ("normal", sd) or ("uniform", lo, hi)
    k_dist: tuple
    v_dist: tuple
    key_padding: bool = False   # per-batch valid key length ~ U{0..N}
    block_c: Optional[int] = None  # forced key-tile width, None = library default
    seed: int = 0
    # FP8 inputs only: per-tensor descales (real value = stored value * descale)
    descale: tuple = (1.0, 1.0, 1.0)

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to float32: the value the library receives."""
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32))

    def nominal_flops(self) -> float:
        """4*B*H*N^2*d multiply-adds-as-two-flops, halved for a causal mask."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def with_shape(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the attention forward study, in order. Index 0 is the
# small case the oracle finishes in seconds; index 2 is the headline case.
WORKLOADS = [
    Workload("tiny_f32_n256_d64", 1, 1, 256, 64, "f32", "f32", False,
             ("normal", 1.0), ("normal", 1.0), ("normal", 1.0), block_c=64, seed=1000),
    Workload("bf16_noncausal_n2048_d64", 4, 16, 2048, 64, "bf16", "f32", False,
             ("normal", 1.0), ("normal", 1.0), ("normal", 1.0), seed=1001),
    Workload("bf16_causal_n8192_d128", 2, 32, 8192, 128, "bf16", "bf16", True,
             ("normal", 1.0), ("normal", 1.0), ("normal", 1.0), seed=1002),
    # Q variance 4 (sd 2): large logits, so the running max moves often.
    Workload("bf16_causal_long_n32768_d128", 1, 8, 32768, 128, "bf16", "bf16", True,
             ("normal", 2.0), ("normal", 1.0), ("normal", 1.0), seed=1003),
    Workload("f16_keypad_n4096_d64", 8, 16, 4096, 64, "f16", "f16", False,
             ("normal", 3.0), ("normal", 3.0), ("uniform", -1.0, 1.0),
             key_padding=True, seed=1004),
]
BY_NAME = {w.name: w for w in WORKLOADS}

# FP8 (E4M3) forward: the headline shape with per-tensor scaling. Real inputs
# ~ N(0, 1) are stored as value / descale with power-of-two descales (Q, K
# 2^-6, V 2^-5), so the stored values spread over E4M3's normal range (|x| up
# to ~300 < 448) and the dequantized logits match the bf16 headline's.
FP8_WORKLOADS = [
    Workload("fp8_causal_n8192_d128", 2, 32, 8192, 128, "e4m3", "bf16", True,
             ("normal", 64.0), ("normal", 64.0), ("normal", 32.0), seed=3000,
             descale=(2.0 ** -6, 2.0 ** -6, 2.0 ** -5)),
]
FP8_BY_NAME = {w.name: w for w in FP8_WORKLOADS}


def _draw(gen: torch.Generator, shape, dist) -> torch.Tensor:
    if dist[0] == "normal":
        return torch.randn(shape, generator=gen, dtype=torch.float32) * dist[1]
    if dist[0] == "uniform":
        lo, hi = dist[1], dist[2]
        return torch.rand(shape, generator=gen, dtype=torch.float32) * (hi - lo) + lo
    raise ValueError(f"unknown distribution {dist!r}")


def key_lengths(gen: torch.Generator, B: int, N: int) -> torch.Tensor:
    """Per-batch valid key length drawn uniformly from {0..N}; the first batch
    is forced to 0 (every row fully masked) and the last to N (no padding) so
    both extremes are always present."""
    lens = torch.randint(0, N + 1, (B,), generator=gen, dtype=torch.int64)
    lens[0] = 0
    if B > 1:
        lens[B - 1] = N
    return lens


def mask_from_lengths(lens: torch.Tensor, N: int) -> torch.Tensor:
    """[B][N] uint8, 1 where the key is valid (j < len_b), 0 where padded."""
    j = torch.arange(N, dtype=torch.int64)
    return (j[None, :] < lens[:, None]).to(torch.uint8).contiguous()


def generate(w: Workload, seed: Optional[int] = None, lens: Optional[torch.Tensor] = None) -> dict:
    """Draw Q, K, V ([B][H][N][d], contiguous, CPU) and the key mask.

    Returns a dict with q, k, v (in_dtype), mask (uint8 [B][N] or None),
    lens (int64 [B] or None), scale (float32 value as a Python float), causal,
    in_dtype / out_dtype names, descale (q, k, v). For "e4m3" the float32
    draw is rounded to E4M3 by torch's conversion (nearest, ties to even).
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    dt = DTYPES[w.in_dtype]
    q = _draw(gen, shape, w.q_dist).to(dt).contiguous()
    k = _draw(gen, shape, w.k_dist).to(dt).contiguous()
    v = _draw(gen, shape, w.v_dist).to(dt).contiguous()
    mask = None
    if w.key_padding or lens is not None:
        if lens is None:
            lens = key_lengths(gen, w.B, w.N)
        mask = mask_from_lengths(lens, w.N)
    return dict(q=q, k=k, v=v, mask=mask, lens=lens, scale=w.scale, causal=w.causal,
                in_dtype=w.in_dtype, out_dtype=w.out_dtype, descale=w.descale, workload=w)


def generate_dout(w: Workload, seed: Optional[int] = None) -> torch.Tensor:
    """The output gradient dO for the backward of workload `w`: [B][H][N][d]
    i.i.d. N(0, 1) in float32 from a generator seeded with w.seed + 7000 (or
    `seed`), rounded to the input dtype."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed + 7000 if seed is None else seed)
    return _draw(gen, (w.B, w.H, w.N, w.d), ("normal", 1.0)).to(DTYPES[w.in_dtype]).contiguous()


# ---------------------------------------------------------------- row softmax

@dataclasses.dataclass(frozen=True)
class SoftmaxWorkload:
    """A [rows][cols] matrix whose rows are softmaxed independently."""
    name: str
    rows: int
    cols: int
    in_dtype: str
    out_dtype: str
    dist: tuple              # ("normal", sd) or ("uniform", lo, hi), drawn in float32
    masked_frac: float = 0.0  # fraction of entries set to -inf (drawn after the values)
    seed: int = 0

    def algorithmic_bytes(self) -> int:
        """x read once, y and the float32 LSE written once."""
        eb = {"f32": 4, "bf16": 2, "f16": 2}
        return self.rows * self.cols * (eb[self.in_dtype] + eb[self.out_dtype]) + 4 * self.rows

    def with_shape(self, **kw) -> "SoftmaxWorkload":
        return dataclasses.replace(self, **kw)


SOFTMAX_WORKLOADS = [
    # rows of attention-score length (one per query of the headline attention
    # shape's sequence length), logits with standard deviation 2
    SoftmaxWorkload("sm_bf16_r32768_c8192", 32768, 8192, "bf16", "bf16", ("normal", 2.0), seed=2000),
    # vocabulary-sized rows in float32: too long for registers, streamed
    SoftmaxWorkload("sm_f32_r1024_c131072", 1024, 131072, "f32", "f32", ("normal", 4.0), seed=2001),
]
SOFTMAX_BY_NAME = {w.name: w for w in SOFTMAX_WORKLOADS}


def generate_softmax(w: SoftmaxWorkload, seed: Optional[int] = None) -> torch.Tensor:
    """x [rows][cols] (CPU, contiguous, in_dtype). Values are drawn in float32
    from a generator seeded per workload, then a Bernoulli(masked_frac) draw
    per entry replaces some by -inf, then the matrix is rounded to in_dtype."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed if seed is None else seed)
    x = _draw(gen, (w.rows, w.cols), w.dist)
    if w.masked_frac > 0:
        drop = torch.rand((w.rows, w.cols), generator=gen) < w.masked_frac
        x = x.masked_fill(drop, float("-inf"))
    return x.to(DTYPES[w.in_dtype]).contiguous()
