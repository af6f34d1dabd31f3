"""GPU parity of the biased / masked forward (attn_fwd_bias through the C ABI)
against the fp64 oracle on the same seeded inputs.

Covers additive bias and boolean mask for every dtype and head dim, causal
and not, ragged key tails (bias rows stored with a padded row stride, which
is how a caller meets the 16-byte row rule for odd Nkv), broadcast operands
(stride 0 over batch, head or query rows), rows left with no key, -inf bias
entries, and sampled rows of the full-size biased workload.
"""

import numpy as np
import pytest
import torch

import oracle
import attention_forward_online_attn_amd as attn
from attention_forward_online_attn_amd import workloads as wl
from parity import TOL, assert_close, host64

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def make_operand(kind, shape, Nkv, dtype, seed, keep=0.75):
    """Bias (N(0, 2^2)) or mask of `shape` (last dim Nkv), stored with the key
    dimension padded to a multiple of 16 so every row starts 16-byte aligned;
    returns (cpu view, device view) with identical strides."""
    pad = (Nkv + 15) // 16 * 16
    full = list(shape[:-1]) + [pad]
    if kind == "add":
        store = wl.score_bias(full, dtype, seed, scale=2.0)
    else:
        store = wl.score_mask(full, keep, seed)
    return store[..., :Nkv], store.cuda()[..., :Nkv]


def bias_case(B, H, Nq, Nkv, D, dtype, causal, kind, bshape=None, seed=0, scale=None, keep=0.75,
              edit=None, label=""):
    q, k, v = wl.dense_inputs(B, H, Nq, Nkv, D, dtype, seed)
    bshape = bshape or (B, H, Nq, Nkv)
    cpu, dev = make_operand(kind, bshape, Nkv, dtype, seed, keep)
    if edit is not None:  # in-place change applied to both copies
        edit(cpu)
        dev.copy_(cpu.cuda())
    scale = D ** -0.5 if scale is None else scale
    kw = {"bias": dev} if kind == "add" else {"mask": dev}
    o, lse = attn.fwd_bias(q.cuda(), k.cuda(), v.cuda(), causal=causal, sm_scale=scale, **kw)
    okw = {"bias": cpu} if kind == "add" else {"mask": cpu}
    ro, rl = oracle.attention(q, k, v, oracle.scale_as_passed(scale), causal, **okw)
    assert_close(DT[dtype], host64(o), host64(lse), ro, rl,
                 label=label or f"{kind} {B,H,Nq,Nkv,D} {dtype} causal={causal} operand {tuple(bshape)}")
    return ro, rl, host64(o), host64(lse)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_additive_bias(gpu_lib, dtype, D, causal):
    bias_case(2, 3, 300, 300, D, dtype, causal, "add", seed=60 + D)
    if not causal:
        bias_case(1, 2, 77, 333, D, dtype, False, "add", seed=61 + D)  # cross attention, ragged key tail


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_boolean_mask(gpu_lib, dtype, D, causal):
    bias_case(2, 3, 300, 300, D, dtype, causal, "mask", seed=62 + D)
    if not causal:
        bias_case(1, 2, 150, 1000, D, dtype, False, "mask", seed=63 + D, keep=0.3)


@pytest.mark.parametrize("kind", ["add", "mask"])
def test_broadcast_operands(gpu_lib, kind):
    B, H, N = 2, 4, 260
    for shape in [(1, H, N, N), (B, 1, N, N), (B, 1, 1, N), (N, N), (1, 1, 1, N)]:
        bias_case(B, H, N, N, 128, "bf16", False, kind, bshape=shape, seed=64)
    bias_case(B, H, N, N, 64, "bf16", True, kind, bshape=(1, H, N, N), seed=65)
    # shared by the batch (the batch is then the fastest work index): odd batch counts, causal
    bias_case(3, 2, 300, 300, 128, "fp16", True, kind, bshape=(1, 2, 300, 300), seed=72)
    bias_case(5, 3, 200, 200, 64, "fp32", False, kind, bshape=(1, 1, 200, 200), seed=73)


def test_mask_rows_without_keys(gpu_lib):
    """Rows whose mask is all False (and, with causal, rows whose only
    visible keys are masked) are empty: O = 0, LSE = -inf."""
    def edit(m):
        m[0, 0, 5] = False
        m[1, 1, 100:140] = False
        m[0, 1, :, :3] = False  # causal rows 0..2 see only keys 0..i
    for dtype in ("bf16", "fp32"):
        ro, rl, go, gl = bias_case(2, 2, 200, 200, 64, dtype, True, "mask", seed=66, edit=edit)
        assert np.all(np.isneginf(rl[0, 0, 5])) and np.all(np.isneginf(rl[0, 1, :3]))
        assert np.all(go[0, 0, 5] == 0) and np.all(np.isneginf(gl[1, 1, 100:140]))


def test_neg_inf_bias_masks(gpu_lib):
    def edit(b):
        b[0, 0, :, 7] = -float("inf")
        b[0, 1, 3] = -float("inf")  # a row with every key removed
        b[1, 0, 10:20, 50:] = -float("inf")
    for dtype in ("bf16", "fp16", "fp32"):
        ro, rl, go, gl = bias_case(2, 2, 128, 128, 64, dtype, False, "add", seed=67, edit=edit)
        assert np.isneginf(gl[0, 1, 3]) and np.all(go[0, 1, 3] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_zero_scale_with_bias_is_softmax_of_the_bias(gpu_lib, dtype):
    bias_case(1, 2, 130, 130, 64, dtype, False, "add", seed=68, scale=0.0)


def test_tile_sweep(gpu_lib):
    """Query and key counts around the 128-row query tile and 64-key tile."""
    for n in (1, 15, 64, 65, 127, 129, 200):
        bias_case(1, 2, n, n, 128, "bf16", False, "add", seed=69 + n)
        bias_case(1, 2, n, n, 64, "bf16", True, "mask", seed=70 + n)


@pytest.mark.parametrize("kind", ["add", "mask"])
def test_full_size_sampled(gpu_lib, kind):
    """B=4 H=32 N=4096 D=128 with a per-head [1, H, N, N] operand, on sampled
    query rows the oracle computes one by one."""
    B, H, N, D = 4, 32, 4096, 128
    q, k, v = wl.dense_inputs(B, H, N, N, D, "bf16", 0)
    if kind == "add":
        op = wl.score_bias((1, H, N, N), "bf16", 0)
        o, lse = attn.fwd_bias(q.cuda(), k.cuda(), v.cuda(), bias=op.cuda())
        okw = {"bias": op}
    else:
        op = wl.score_mask((1, H, N, N), 0.75, 0)
        o, lse = attn.fwd_bias(q.cuda(), k.cuda(), v.cuda(), mask=op.cuda())
        okw = {"mask": op}
    rng = np.random.default_rng(71)
    rows = [(int(rng.integers(0, B)), int(rng.integers(0, H)), int(i))
            for i in sorted({0, 1, 127, 128, N - 1} | set(int(x) for x in rng.integers(0, N, 40)))]
    ro, rl = oracle.attention_sampled(q, k, v, oracle.scale_as_passed(D ** -0.5), False, rows, **okw)
    oc, lc = host64(o), host64(lse)
    go = np.stack([oc[b, h, i] for b, h, i in rows])
    gl = np.array([lc[b, h, i] for b, h, i in rows])
    assert_close(torch.bfloat16, go, gl, ro, rl, label=f"{kind} [4,32,4096,128] operand [1,32,4096,4096], {len(rows)} rows")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    assert TOL[torch.bfloat16]["o"] == 1e-2
