"""Seeded random sweeps of the dense forward and JVP, and of the backward,
over the supported configuration space, each case against the fp64 oracle on
the same seeded inputs.

The hand-picked cases elsewhere cover each edge on its own; this sweep draws
combinations of them from a fixed seed (so every run checks the same cases):
head dims 16..256 and value dims that differ from the query/key dim, bf16,
fp16 and fp32, causal or not (the small causal grids here all take the
paired key-split workgroups), cross-attention with Nq != Nkv, ragged sizes
from 1 to 700 rows, and tensors stored [B, N, H, D] and viewed as
[B, H, N, D] (non-contiguous head and row strides).
"""

import numpy as np
import pytest
import torch

import oracle
import attention_forward_online_attn_amd as attn
from attention_forward_online_attn_amd import workloads as wl
from parity import assert_close, host64
from test_parity_bwd_gpu import check_grads

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def draw_cases(n, seed):
    """(case id, B, H, Nq, Nkv, D, Dv, dtype, causal, jvp, strided) tuples
    inside the documented support: D = 256 on the plain forward with Dv = D;
    no 16-wide value tile under the 16-bit JVP with a 128-wide query/key dim."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        jvp = bool(rng.integers(0, 2))
        dtype = ["bf16", "fp16", "fp32"][int(rng.integers(0, 3))]
        D = int(rng.choice([16, 32, 64, 128, 256]))
        Dv = D if rng.random() < 0.6 else int(rng.choice([16, 32, 64, 128]))
        if D == 256 and (jvp or Dv != D):
            continue
        if jvp and D == 128 and Dv == 16 and dtype != "fp32":
            continue
        causal = bool(rng.integers(0, 2))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        Nq = int(rng.integers(1, 700))
        Nkv = Nq if causal else int(rng.integers(1, 700))
        strided = bool(rng.integers(0, 2))
        out.append((len(out), B, H, Nq, Nkv, D, Dv, dtype, causal, jvp, strided))
    return out


CASES = draw_cases(96, seed=2026)


def to_device(t, strided):
    """On the GPU, either contiguous or stored [B, N, H, D] and viewed as
    [B, H, N, D] (same values)."""
    if not strided:
        return t.cuda()
    return t.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "c{}-B{}H{}-{}x{}-D{}v{}-{}{}{}{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], "-causal" if c[8] else "", "-jvp" if c[9] else "",
    "-strided" if c[10] else ""))
def test_random_configuration(gpu_lib, case):
    i, B, H, Nq, Nkv, D, Dv, dtype, causal, jvp, strided = case
    ts = wl.dense_inputs(B, H, Nq, Nkv, D, dtype, 500 + 10 * i, tangents=jvp, Dv=Dv)
    dev = [to_device(t, strided) for t in ts]
    scale = D ** -0.5
    label = f"random case {case}"
    if jvp:
        o, to, lse = attn.fwd_jvp(*dev, causal=causal, sm_scale=scale)
        ro, rto, rl = oracle.attention_jvp(*ts, oracle.scale_as_passed(scale), causal)
        assert_close(DT[dtype], host64(o), host64(lse), ro, rl, host64(to), rto, label=label)
    else:
        o, lse = attn.fwd(*dev, causal=causal, sm_scale=scale)
        ro, rl = oracle.attention(*ts, oracle.scale_as_passed(scale), causal)
        assert_close(DT[dtype], host64(o), host64(lse), ro, rl, label=label)


def draw_bwd_cases(n, seed):
    """(case id, B, H, Nq, Nkv, D, dtype, causal, strided): the backward's
    support is bf16 and fp16 at head dims 32, 64 and 128."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = ["bf16", "fp16"][int(rng.integers(0, 2))]
        D = int(rng.choice([32, 64, 128]))
        causal = bool(rng.integers(0, 2))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        Nq = int(rng.integers(1, 500))
        Nkv = Nq if causal else int(rng.integers(1, 500))
        out.append((i, B, H, Nq, Nkv, D, dtype, causal, bool(rng.integers(0, 2))))
    return out


BWD_CASES = draw_bwd_cases(32, seed=2027)


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "b{}-B{}H{}-{}x{}-D{}-{}{}{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "-causal" if c[7] else "", "-strided" if c[8] else ""))
def test_random_backward(gpu_lib, case):
    """dQ, dK, dV from the forward's own O and LSE, to the backward's bound
    (3e-2 of max|g| for bf16, 1e-2 for fp16)."""
    i, B, H, Nq, Nkv, D, dtype, causal, strided = case
    q, k, v = wl.dense_inputs(B, H, Nq, Nkv, D, dtype, 700 + 10 * i)
    do = wl.grad_output((B, H, Nq, D), dtype, 700 + 10 * i)
    scale = D ** -0.5
    qc, kc, vc, doc = (to_device(t, strided) for t in (q, k, v, do))
    o, lse = attn.fwd(qc, kc, vc, causal=causal, sm_scale=scale)
    got = attn.bwd(qc, kc, vc, o, doc, lse, causal=causal, sm_scale=scale)
    ref = oracle.attention_bwd(q, k, v, do, oracle.scale_as_passed(scale), causal)
    check_grads(got, ref, f"random backward case {case}", dtype)
