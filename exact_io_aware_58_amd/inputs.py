"""Seeded synthetic inputs shared by the oracle checks and the HIP path.

This module holds none of attention's arithmetic: it only draws i.i.d.
N(0, 1) tensors (the pages' own benchmark draws its Q, K, V with randn at
shape (1, 12, 2048, 64): ijyty.com/news/1153309, "Flash Attention 技术原理让
Transformer 更快更高效", section "性能对比"), rounds them to the storage dtype
with round-to-nearest-even, and picks seeded subsets of rows to check.  The
oracle reads the rounded values upcast to float64, so parity measures the
kernel's error, not input quantisation.

Recipe: workload k uses seed k; tensor t in {Q: 0, K: 1, V: 2, dO: 3} is
numpy.random.default_rng([k, t]).standard_normal(shape, dtype=float32),
times the workload's input multiplier, then rounded to the dtype.

Grid recipe (draw_grid), for sizes where normal variates and their rounding
take tens of seconds per tensor (a 2^23 x 128 head): each element is
(2u - 31) / 16 with u = one byte of numpy.random.default_rng([k, t, 1]).bytes
masked to 0..31, i.e. 32 equally likely levels in [-1.9375, 1.9375], mean 0,
variance 1.33.  Every level is exact in bf16, fp16 and f32, so the values
need no rounding and sums of them are exact in float64.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# q, k, v, do: attention inputs; oa, ob, la, lb: synthetic partial results
# (outputs and log-sum-exps) for checking the merge on its own.
TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3, "oa": 4, "ob": 5, "la": 6, "lb": 7}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    H: int
    N: int
    D: int
    dtype: str          # "f32", "bf16" or "f16"
    causal: bool
    backward: bool
    input_mult: float = 1.0
    check_rows: int = 0  # 0: check every row; else a seeded subset of rows

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.D)

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)


# The five workloads of the attention path (shape, dtype, mask, passes).
WORKLOADS = {
    "c1": Workload("fwd_f32_b1h1n256d64", 1, 1, 1, 256, 64, "f32", False, False),
    "c2": Workload("fwd_bf16_b1h12n2048d64", 2, 1, 12, 2048, 64, "bf16", False, False),
    "c3": Workload("train_causal_bf16_b8h12n1024d64", 3, 8, 12, 1024, 64, "bf16", True, True),
    "c4": Workload("fwd_bf16_b1h16n16384d128_x0.5", 4, 1, 16, 16384, 128, "bf16", False, False,
                   input_mult=0.5, check_rows=256),
    "c5": Workload("train_causal_bf16_b1h16n65536d64", 5, 1, 16, 65536, 64, "bf16", True, True,
                   check_rows=128),
    # Scale test of the linear-memory claim: a 128K-token causal training step.
    "n128k": Workload("train_causal_bf16_b1h8n131072d64", 6, 1, 8, 131072, 64, "bf16", True, True,
                      check_rows=64),
    # D = 128 forwards at the short end of the N >= 4096 range (the N = 16384
    # recipe, inputs x 0.5) and a D = 128 training step.
    "n4k_d128": Workload("fwd_bf16_b1h16n4096d128_x0.5", 8, 1, 16, 4096, 128, "bf16", False,
                         False, input_mult=0.5, check_rows=128),
    "n8k_d128": Workload("fwd_bf16_b1h16n8192d128_x0.5", 9, 1, 16, 8192, 128, "bf16", False,
                         False, input_mult=0.5, check_rows=128),
    "train_d128": Workload("train_bf16_b1h16n16384d128", 10, 1, 16, 16384, 128, "bf16", False,
                           True, check_rows=64),
}


def round_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even.
    Inputs are finite (N(0,1) draws), so no NaN handling is needed."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_to_dtype(x32: np.ndarray, dtype: str):
    """Returns (values as float32, raw storage array for upload)."""
    if dtype == "f32":
        x = np.ascontiguousarray(x32, dtype=np.float32)
        return x, x
    if dtype == "bf16":
        bits = round_bf16_bits(x32)
        return bf16_bits_to_f32(bits), bits
    if dtype == "f16":
        h = x32.astype(np.float16)  # numpy's float32->float16 cast is RNE
        return h.astype(np.float32), h
    raise ValueError(f"unknown dtype {dtype!r}")


def draw(seed: int, tensor: str, shape, dtype: str, mult: float = 1.0):
    """One seeded tensor: (float32 values, raw storage array)."""
    rng = np.random.default_rng([seed, TENSOR_IDS[tensor]])
    x = rng.standard_normal(shape, dtype=np.float32)
    if mult != 1.0:
        x = x * np.float32(mult)
    return round_to_dtype(x, dtype)


def draw_grid(seed: int, tensor: str, shape, dtype: str):
    """One seeded grid-valued tensor (see the module docstring):
    (float32 values, raw storage array)."""
    rng = np.random.default_rng([seed, TENSOR_IDS[tensor], 1])
    u = np.frombuffer(rng.bytes(int(np.prod(shape))), dtype=np.uint8).reshape(shape)
    x = (u & 31).astype(np.float32)
    x *= np.float32(2.0 / 16.0)
    x -= np.float32(31.0 / 16.0)
    if dtype == "bf16":
        return x, (x.view(np.uint32) >> 16).astype(np.uint16)  # exact: low half is zero
    if dtype == "f16":
        return x, x.astype(np.float16)
    if dtype == "f32":
        return x, x
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(w: Workload, with_grad=None):
    """Dict name -> (float32 values, raw storage) for q, k, v (and do)."""
    names = ["q", "k", "v"]
    if with_grad if with_grad is not None else w.backward:
        names.append("do")
    return {n: draw(w.seed, n, w.shape, w.dtype, w.input_mult if n != "do" else 1.0)
            for n in names}


def check_row_subset(w: Workload, count: int = None, seed_offset: int = 1000):
    """Seeded (b, h, i) triples to check at full size.

    Always holds i in {0, 1, 63, 64, 127, 128, N/2, N-1} (tile edges and the
    causal diagonal) in the first and last head of batch 0; the rest are drawn
    uniformly without replacement from default_rng(seed + seed_offset).
    """
    count = count or w.check_rows
    N = w.N
    fixed = sorted({i for i in (0, 1, 63, 64, 127, 128, N // 2, N - 1) if 0 <= i < N})
    picked = []
    for h in sorted({0, w.H - 1}):
        picked += [(0, h, i) for i in fixed]
    seen = set(picked)
    rng = np.random.default_rng(w.seed + seed_offset)
    total = w.B * w.H * N
    while len(picked) < count:
        flat = int(rng.integers(total))
        b, rem = divmod(flat, w.H * N)
        h, i = divmod(rem, N)
        if (b, h, i) not in seen:
            seen.add((b, h, i))
            picked.append((b, h, i))
    return np.array(picked, dtype=np.int64)
