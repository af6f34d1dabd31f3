"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke run.

This module draws random numbers and builds index arrays only; it holds none of
the attention arithmetic, so both the HIP path and the CPU oracle can take their
inputs from it.

Recipe (the same on every machine, independent of the device):
* one CPU ``torch.Generator`` per tensor, seeded ``seed_base + i`` with
  i = 0..5 for Q, K, V, tQ, tK, tV, i = 6 for the jagged lengths, i = 7
  for the backward's dO, i = 8 for an additive bias and i = 9 for a mask;
* values i.i.d. N(0, 1) drawn in fp32 and rounded to the working dtype
  (round-to-nearest-even for bf16) on the CPU;
* jagged lengths uniform in [1, max_len], offsets = exclusive prefix sum (int64).
These match the workloads the pages test and benchmark: i.i.d. normal Q/K/V
(the pages draw N(0, 0.5^2) with seed 20; the workloads here are N(0, 1)),
[B, H, N, D] dense layouts, and a jagged [H, total_len, D] layout addressed by
offsets.
"""

from __future__ import annotations

import dataclasses
import math

import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _normal(shape, seed, dtype, std=1.0):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return (torch.randn(*shape, generator=g, dtype=torch.float32) * std).to(dtype)


def dense_inputs(B, H, Nq, Nkv, D, dtype="bf16", seed_base=0, tangents=False, Dv=None, std=1.0):
    """Q [B,H,Nq,D], K [B,H,Nkv,D], V [B,H,Nkv,Dv] (Dv defaults to D; and
    tQ/tK/tV when tangents) on the CPU, i.i.d. N(0, std^2)."""
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    Dv = D if Dv is None else Dv
    q = _normal((B, H, Nq, D), seed_base + 0, dt, std)
    k = _normal((B, H, Nkv, D), seed_base + 1, dt, std)
    v = _normal((B, H, Nkv, Dv), seed_base + 2, dt, std)
    if not tangents:
        return q, k, v
    tq = _normal((B, H, Nq, D), seed_base + 3, dt, std)
    tk = _normal((B, H, Nkv, D), seed_base + 4, dt, std)
    tv = _normal((B, H, Nkv, Dv), seed_base + 5, dt, std)
    return q, k, v, tq, tk, tv


def grad_output(shape, dtype="bf16", seed_base=0):
    """dO for the backward: i.i.d. N(0, 1), seeded seed_base + 7 (CPU)."""
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    return _normal(shape, seed_base + 7, dt)


def score_bias(shape, dtype="bf16", seed_base=0, scale=1.0):
    """Additive score bias: i.i.d. N(0, scale^2), seeded seed_base + 8 (CPU)."""
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed_base + 8))
    return (torch.randn(*shape, generator=g, dtype=torch.float32) * scale).to(dt)


def score_mask(shape, keep=0.75, seed_base=0):
    """Boolean mask, each entry True (key kept) with probability `keep`,
    seeded seed_base + 9 (CPU)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed_base + 9))
    return torch.rand(*shape, generator=g) < keep


def jagged_lengths(num_seqs, max_len, seed_base=0, min_len=1):
    """Sequence lengths uniform in [min_len, max_len] (int64, CPU)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed_base + 6))
    return torch.randint(min_len, max_len + 1, (num_seqs,), generator=g, dtype=torch.int64)


def offsets_from_lengths(lengths):
    """Exclusive prefix sum with the total appended: [0, l0, l0+l1, ...]."""
    lengths = torch.as_tensor(lengths, dtype=torch.int64)
    return torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(lengths, 0)])


def jagged_inputs(lengths, H, D, dtype="bf16", seed_base=0, tangents=False):
    """Jagged Q/K/V [H, total_len, D] for the given lengths, plus offsets."""
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    offsets = offsets_from_lengths(lengths)
    T = int(offsets[-1])
    tensors = [_normal((H, T, D), seed_base + i, dt) for i in range(6 if tangents else 3)]
    return (*tensors, offsets)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark / parity workload (sizes as the pages' workloads)."""
    name: str
    kind: str            # "dense", "jvp" or "jagged"
    dtype: str
    B: int = 1
    H: int = 1
    N: int = 0           # dense: Nq == Nkv
    D: int = 64
    causal: tuple = (False,)
    num_seqs: int = 0    # jagged
    max_len: int = 0     # jagged: lengths U{1..max_len}; also max_seq_len

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", "dense", "fp32", B=1, H=2, N=128, D=64),
    "causal_d64": Workload("causal_d64", "dense", "bf16", B=4, H=16, N=1024, D=64, causal=(True,)),
    "long_d128": Workload("long_d128", "dense", "bf16", B=4, H=32, N=4096, D=128, causal=(False, True)),
    "jvp_d64": Workload("jvp_d64", "jvp", "bf16", B=4, H=16, N=2048, D=64, causal=(False, True)),
    "jagged_d128": Workload("jagged_d128", "jagged", "bf16", H=8, D=128, num_seqs=256, max_len=1024),
}
