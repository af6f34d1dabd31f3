"""Seeded random sweeps over the supported configuration space -- the dense
forward and JVP, the backward, the jagged forward and backward, and the
biased / masked forward and backward -- each case against the fp64 oracle on
the same seeded inputs.

The hand-picked cases elsewhere cover each edge on its own; this sweep draws
combinations of them from a fixed seed (so every run checks the same cases):
head dims 16..256 and value dims that differ from the query/key dim, bf16,
fp16 and fp32, causal or not (the small causal grids here all take the
paired key-split workgroups), cross-attention with Nq != Nkv, ragged sizes
from 1 to 700 rows, and tensors stored [B, N, H, D] and viewed as
[B, H, N, D] (non-contiguous head and row strides).

ATTN_SWEEP_SEED=k shifts every sweep's seed by k (default 0: the committed
cases), so that a longer stress run can draw further cases.
"""

import os

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


SEED_SHIFT = int(os.environ.get("ATTN_SWEEP_SEED", "0"))


def draw_cases(n, seed):
    """(case id, B, H, Nq, Nkv, D, Dv, dtype, causal, jvp, strided) tuples
    inside the documented support (every pair of head dims, every dtype)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        jvp = bool(rng.integers(0, 2))
        dtype = ["bf16", "fp16", "fp32"][int(rng.integers(0, 3))]
        D = int(rng.choice([16, 32, 64, 128, 256]))
        Dv = D if rng.random() < 0.6 else int(rng.choice([16, 32, 64, 128, 256]))
        causal = bool(rng.integers(0, 2))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        Nq = int(rng.integers(1, 700))
        Nkv = Nq if causal else int(rng.integers(1, 700))
        strided = bool(rng.integers(0, 2))
        out.append((len(out), B, H, Nq, Nkv, D, Dv, dtype, causal, jvp, strided))
    return out


CASES = draw_cases(96, seed=2026 + SEED_SHIFT)


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
    support is bf16 and fp16 at head dims 16, 32, 64, 128 and 256."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = ["bf16", "fp16"][int(rng.integers(0, 2))]
        D = int(rng.choice([16, 32, 64, 128, 256]))
        causal = bool(rng.integers(0, 2))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        Nq = int(rng.integers(1, 500))
        Nkv = Nq if causal else int(rng.integers(1, 500))
        out.append((i, B, H, Nq, Nkv, D, dtype, causal, bool(rng.integers(0, 2))))
    return out


BWD_CASES = draw_bwd_cases(32, seed=2027 + SEED_SHIFT)


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


def draw_jagged_cases(n, seed):
    """(case id, lengths, H, D, dtype, max_seq_len, causal, backward): lengths
    from a mix of distributions (empty sequences included), max_seq_len at or
    below the longest sequence."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        S = int(rng.integers(1, 40))
        kind = int(rng.integers(0, 3))
        if kind == 0:
            lengths = rng.integers(0, 600, S)
        elif kind == 1:
            lengths = rng.integers(0, 70, S)
        else:
            lengths = np.where(rng.random(S) < 0.3, 0, rng.integers(100, 400, S))
        if lengths.sum() == 0:
            lengths[0] = 1
        longest = max(int(lengths.max()), 1)
        msl = longest if rng.random() < 0.5 else int(rng.integers(1, longest + 1))
        backward = bool(rng.integers(0, 2))
        dtype = ["bf16", "fp16"][int(rng.integers(0, 2))] if backward else ["bf16", "fp16", "fp32"][int(rng.integers(0, 3))]
        D = int(rng.choice([16, 32, 64, 128]))
        out.append((i, [int(x) for x in lengths], int(rng.integers(1, 5)), D, dtype, msl, bool(rng.integers(0, 2)),
                    backward))
    return out


JAGGED_CASES = draw_jagged_cases(24, seed=2028 + SEED_SHIFT)


@pytest.mark.parametrize("case", JAGGED_CASES, ids=lambda c: "j{}-S{}-H{}-D{}-{}-msl{}{}{}".format(
    c[0], len(c[1]), c[2], c[3], c[4], c[5], "-causal" if c[6] else "", "-bwd" if c[7] else ""))
def test_random_jagged(gpu_lib, case):
    """Jagged forward (and, for the backward cases, dQ, dK, dV from the
    forward's own O and LSE) against the oracle."""
    i, lengths, H, D, dtype, msl, causal, backward = case
    lengths = torch.as_tensor(lengths, dtype=torch.int64)
    q, k, v, off = wl.jagged_inputs(lengths, H, D, dtype, 900 + 10 * i)
    scale = D ** -0.5
    qc, kc, vc, oc = (t.cuda() for t in (q, k, v, off))
    o, lse = attn.jagged_fwd(qc, kc, vc, oc, max_seq_len=msl, causal=causal, sm_scale=scale)
    ro, rl = oracle.jagged_attention(q, k, v, off.numpy(), msl, oracle.scale_as_passed(scale), causal)
    assert_close(DT[dtype], host64(o), host64(lse), ro, rl, label=f"random jagged case {case}")
    if backward:
        do = wl.grad_output(q.shape, dtype, 900 + 10 * i)
        got = attn.jagged_bwd(qc, kc, vc, o, do.cuda(), lse, oc, msl, causal=causal, sm_scale=scale)
        ref = oracle.jagged_attention_bwd(q, k, v, do, off.numpy(), msl, oracle.scale_as_passed(scale), causal)
        check_grads(got, ref, f"random jagged backward case {case}", dtype)
        # rows past max_seq_len inside a sequence get exactly zero gradients
        offs = off.numpy()
        for g in got:
            g = host64(g)
            for s_ in range(len(lengths)):
                a, b = int(offs[s_]), int(offs[s_ + 1])
                assert np.all(g[:, a + min(b - a, msl):b] == 0), f"rows past max_seq_len in case {case}"


def draw_bias_cases(n, seed):
    """(case id, B, H, Nq, Nkv, D, dtype, causal, kind, operand shape,
    backward): additive bias or boolean mask, each of the batch, head and
    query dims of the operand either full or broadcast (1)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        backward = bool(rng.integers(0, 2))
        kind = ["add", "mask"][int(rng.integers(0, 2))]
        dtype = ["bf16", "fp16"][int(rng.integers(0, 2))] if backward else ["bf16", "fp16", "fp32"][int(rng.integers(0, 3))]
        D = int(rng.choice([16, 32, 64, 128, 256]))
        causal = bool(rng.integers(0, 2))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        Nq = int(rng.integers(1, 400))
        Nkv = Nq if causal else int(rng.integers(1, 400))
        shape = tuple(d if rng.random() < 0.5 else 1 for d in (B, H, Nq)) + (Nkv,)
        out.append((i, B, H, Nq, Nkv, D, dtype, causal, kind, shape, backward))
    return out


BIAS_CASES = draw_bias_cases(24, seed=2029 + SEED_SHIFT)


@pytest.mark.parametrize("case", BIAS_CASES, ids=lambda c: "x{}-B{}H{}-{}x{}-D{}-{}-{}-op{}{}{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[8], "x".join(map(str, c[9])), "-causal" if c[7] else "",
    "-bwd" if c[10] else ""))
def test_random_bias(gpu_lib, case):
    """Biased or masked forward, or backward (with the bias gradient for an
    additive bias), against the oracle."""
    from test_parity_bias_gpu import bias_case
    from test_parity_bias_bwd_gpu import bias_bwd_case
    i, B, H, Nq, Nkv, D, dtype, causal, kind, shape, backward = case
    if backward:
        bias_bwd_case(B, H, Nq, Nkv, D, dtype, causal, kind, bshape=shape, seed=1100 + 10 * i)
    else:
        bias_case(B, H, Nq, Nkv, D, dtype, causal, kind, bshape=shape, seed=1100 + 10 * i)
