"""GPU parity of the newer paths on non-contiguous layouts, and their
determinism.

* [B, N, H, D] storage and packed QKV [B, N, 3, H, D] (the bias page's
  layouts) reach every dense entry point through strides only: the JVP, the
  biased forward and backward, the value-dim forward and the backward.
* The backward writes each gradient element once (no atomics): two runs
  agree bit for bit, as do two runs of every forward variant.
"""

import numpy as np
import pytest
import torch

import oracle
import attention_forward_online_attn_amd as attn
from attention_forward_online_attn_amd import workloads as wl
from parity import assert_close, host64

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


def bhnd(x):
    """[B, N, H, D] -> a [B, H, N, D] view."""
    return x.permute(0, 2, 1, 3)


def packed(B, N, H, D, seed, dv=None):
    """q, k, v as views of one packed [B, N, 3, H, D] tensor (or, with a
    value dim, q and k packed and v in its own [B, N, H, Dv] tensor)."""
    g = torch.Generator().manual_seed(seed)
    qkv = torch.randn(B, N, 3, H, D, generator=g).bfloat16()
    if dv is None:
        return qkv, [bhnd(qkv[:, :, i]) for i in range(3)]
    v = torch.randn(B, N, H, dv, generator=g).bfloat16()
    return (qkv, v), [bhnd(qkv[:, :, 0]), bhnd(qkv[:, :, 1]), bhnd(v)]


def rel_check(got, ref, rel, label):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        gmax = float(np.max(np.abs(r)))
        diff = float(np.max(np.abs(host64(g) - r)))
        assert diff <= rel * gmax + 1e-5, f"{label}: {name} {diff / gmax:.2e}"


def test_strided_jvp_and_backward(gpu_lib):
    B, N, H, D = 2, 300, 3, 64
    qkv, (q, k, v) = packed(B, N, H, D, 1)
    qkv_d = qkv.cuda()
    qd, kd, vd = (bhnd(qkv_d[:, :, i]) for i in range(3))
    tan = packed(B, N, H, D, 2)[0].cuda()
    tqd, tkd, tvd = (bhnd(tan[:, :, i]) for i in range(3))
    tq, tk, tv = (bhnd(tan.cpu()[:, :, i]) for i in range(3))
    scale = D ** -0.5
    for causal in (False, True):
        o, to, lse = attn.fwd_jvp(qd, kd, vd, tqd, tkd, tvd, causal=causal)
        ro, rto, rl = oracle.attention_jvp(q, k, v, tq, tk, tv, oracle.scale_as_passed(scale), causal)
        assert_close(BF16, host64(o), host64(lse), ro, rl, host64(to), rto, label=f"strided jvp causal={causal}")
        # backward from strided inputs and a strided dO
        do_store = torch.randn(B, N, H, D, generator=torch.Generator().manual_seed(3)).bfloat16()
        o2, lse2 = attn.fwd(qd, kd, vd, causal=causal)
        got = attn.bwd(qd, kd, vd, o2, bhnd(do_store.cuda()), lse2, causal=causal)
        ref = oracle.attention_bwd(q, k, v, bhnd(do_store), oracle.scale_as_passed(scale), causal)
        rel_check(got, ref, 3e-2, f"strided bwd causal={causal}")


def test_strided_bias_paths(gpu_lib):
    B, N, H, D = 2, 260, 4, 64
    qkv, (q, k, v) = packed(B, N, H, D, 4)
    qkv_d = qkv.cuda()
    qd, kd, vd = (bhnd(qkv_d[:, :, i]) for i in range(3))
    bias = wl.score_bias((1, H, N, 264), "bf16", 5)[..., :N]  # padded rows
    bias_d = wl.score_bias((1, H, N, 264), "bf16", 5).cuda()[..., :N]
    scale = D ** -0.5
    o, lse = attn.fwd_bias(qd, kd, vd, bias=bias_d)
    ro, rl = oracle.attention(q, k, v, oracle.scale_as_passed(scale), False, bias=bias)
    assert_close(BF16, host64(o), host64(lse), ro, rl, label="strided biased forward")
    do_store = torch.randn(B, N, H, D, generator=torch.Generator().manual_seed(6)).bfloat16()
    got = attn.bwd_bias(qd, kd, vd, o, bhnd(do_store.cuda()), lse, bias=bias_d, return_dbias=True)
    ref = oracle.attention_bwd(q, k, v, bhnd(do_store), oracle.scale_as_passed(scale), False, bias=bias,
                               with_dbias=True)
    rel_check(got[:3], ref[:3], 3e-2, "strided biased backward")
    db = host64(got[3]).sum(axis=0, keepdims=True)
    rdb = ref[3].sum(axis=0, keepdims=True)
    assert np.max(np.abs(db - rdb)) <= 3e-2 * np.max(np.abs(rdb)) + 1e-5


def test_strided_value_dim(gpu_lib):
    B, N, H, D, Dv = 2, 200, 3, 64, 128
    (qkv, vv), (q, k, v) = packed(B, N, H, D, 7, dv=Dv)
    qkv_d, vv_d = qkv.cuda(), vv.cuda()
    qd, kd, vd = bhnd(qkv_d[:, :, 0]), bhnd(qkv_d[:, :, 1]), bhnd(vv_d)
    o, lse = attn.fwd(qd, kd, vd, causal=True)
    ro, rl = oracle.attention(q, k, v, oracle.scale_as_passed(D ** -0.5), True)
    assert_close(BF16, host64(o), host64(lse), ro, rl, label="strided value dim 128 under qk 64")


def test_backward_and_variants_are_deterministic(gpu_lib):
    q, k, v = (t.cuda() for t in wl.dense_inputs(2, 4, 777, 777, 128, "bf16", 2))
    do = wl.grad_output(q.shape, "bf16", 2).cuda()
    o, lse = attn.fwd(q, k, v, causal=True)
    g1 = attn.bwd(q, k, v, o, do, lse, causal=True)
    g2 = attn.bwd(q, k, v, o, do, lse, causal=True)
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))
    bias = wl.score_bias((1, 4, 777, 784), "bf16", 3).cuda()[..., :777]
    r1 = attn.fwd_bias(q, k, v, bias=bias)
    r2 = attn.fwd_bias(q, k, v, bias=bias)
    assert all(torch.equal(a, b) for a, b in zip(r1, r2))
    b1 = attn.bwd_bias(q, k, v, r1[0], do, r1[1], bias=bias, return_dbias=True)
    b2 = attn.bwd_bias(q, k, v, r1[0], do, r1[1], bias=bias, return_dbias=True)
    assert all(torch.equal(a, b) for a, b in zip(b1, b2))
    ts = [t.cuda() for t in wl.dense_inputs(2, 4, 500, 500, 64, "bf16", 4, tangents=True)]
    j1 = attn.fwd_jvp(*ts, causal=True, return_tlse=True)
    j2 = attn.fwd_jvp(*ts, causal=True, return_tlse=True)
    assert all(torch.equal(a, b) for a, b in zip(j1, j2))
