"""GPU parity of the backward with a score operand (attn_bwd_bias through
the C ABI, fed with attn_fwd_bias's own O and LSE) against the fp64
oracle's gradients, including the bias gradient dS.

Bound per gradient (dq, dk, dv, dbias), as for the plain backward:
max|g - g_ref| <= rel * max|g_ref| + 1e-5 with rel = 3e-2 (bf16) or 1e-2
(fp16).
"""

import numpy as np
import pytest
import torch

import oracle
import attention_forward_online_attn_amd as attn
from attention_forward_online_attn_amd import workloads as wl
from parity import host64
from test_parity_bias_gpu import make_operand

pytestmark = pytest.mark.gpu

REL = {"bf16": 3e-2, "fp16": 1e-2}
ABS = 1e-5


def check(got, ref, names, dtype, label):
    msgs, ok = [], True
    for name, g, r in zip(names, got, ref):
        g = host64(g)
        gmax = float(np.max(np.abs(r), initial=0.0))
        diff = float(np.max(np.abs(g - r), initial=0.0)) if np.all(np.isfinite(g)) else np.inf
        ok = ok and diff <= REL[dtype] * gmax + ABS
        msgs.append(f"{name} {diff / max(gmax, 1e-30):.2e}")
    msg = f"{label}: max|dg|/max|g| " + ", ".join(msgs)
    print(msg, flush=True)
    assert ok, msg


def bias_bwd_case(B, H, Nq, Nkv, D, dtype, causal, kind, bshape=None, seed=0, scale=None, keep=0.75, edit=None,
                  dbias=True):
    q, k, v = wl.dense_inputs(B, H, Nq, Nkv, D, dtype, seed)
    do = wl.grad_output((B, H, Nq, D), dtype, seed)
    bshape = bshape or (B, H, Nq, Nkv)
    cpu, dev = make_operand(kind, bshape, Nkv, dtype, seed, keep)
    if edit is not None:
        edit(cpu)
        dev.copy_(cpu.cuda())
    scale = D ** -0.5 if scale is None else scale
    kw = {"bias": dev} if kind == "add" else {"mask": dev}
    qc, kc, vc, doc = (t.cuda() for t in (q, k, v, do))
    o, lse = attn.fwd_bias(qc, kc, vc, causal=causal, sm_scale=scale, **kw)
    want_db = dbias and kind == "add"
    got = attn.bwd_bias(qc, kc, vc, o, doc, lse, causal=causal, sm_scale=scale, return_dbias=want_db, **kw)
    okw = {"bias": cpu} if kind == "add" else {"mask": cpu}
    ref = oracle.attention_bwd(q, k, v, do, oracle.scale_as_passed(scale), causal, with_dbias=True, **okw)
    names = ["dq", "dk", "dv"]
    if want_db:
        names.append("dbias")
        # the gradient of a broadcast bias is dS summed over its broadcast dims
        r_db = ref[3]
        got_db = got[3].float()
        for ax, n in enumerate(bshape[-4:] if len(bshape) == 4 else (1,) * (4 - len(bshape)) + tuple(bshape)):
            if n == 1:
                r_db = r_db.sum(axis=ax, keepdims=True)
                got_db = got_db.sum(dim=ax, keepdim=True)
        got = list(got[:3]) + [got_db]
        ref = list(ref[:3]) + [r_db]
    else:
        ref = ref[:3]
    check(got, ref, names, dtype, f"{kind} bwd {B, H, Nq, Nkv, D} {dtype} causal={causal} operand {tuple(bshape)}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bias_bwd(gpu_lib, dtype, D, causal):
    bias_bwd_case(2, 3, 300, 300, D, dtype, causal, "add", seed=110 + D)
    bias_bwd_case(2, 3, 300, 300, D, dtype, causal, "mask", seed=111 + D)


def test_bias_bwd_cross_attention_and_padding(gpu_lib):
    bias_bwd_case(1, 2, 77, 333, 128, "bf16", False, "add", seed=112)   # row stride padded to 336
    bias_bwd_case(1, 2, 150, 1000, 64, "bf16", False, "mask", seed=113, keep=0.3)


def test_bias_bwd_broadcast(gpu_lib):
    B, H, N = 2, 4, 260
    for shape in [(1, H, N, N), (B, 1, N, N), (B, 1, 1, N)]:
        bias_bwd_case(B, H, N, N, 64, "bf16", False, "add", bshape=shape, seed=114)
    bias_bwd_case(B, H, N, N, 64, "bf16", True, "mask", bshape=(B, 1, 1, N), seed=115)
    # operands shared by the batch put the batch innermost in the work order
    bias_bwd_case(3, H, N, N, 128, "bf16", True, "add", bshape=(1, H, N, N), seed=116)
    bias_bwd_case(4, 2, N, N, 64, "fp16", False, "mask", bshape=(1, 1, N, N), seed=117)


def test_bias_bwd_empty_rows_and_zero_scale(gpu_lib):
    def edit(m):
        m[0, 0, 5] = False
        m[1, 1, 100:140] = False
    bias_bwd_case(2, 2, 200, 200, 64, "bf16", True, "mask", seed=116, edit=edit)
    bias_bwd_case(1, 2, 130, 130, 64, "bf16", True, "add", seed=117, scale=0.0)


def test_bias_bwd_without_dbias(gpu_lib):
    bias_bwd_case(2, 2, 300, 300, 128, "bf16", True, "add", seed=118, dbias=False)


def test_bias_bwd_full_size_sampled_heads(gpu_lib):
    """The benchmark's biased backward: B=4 H=32 N=4096 D=128 with a per-head
    bias [1, 32, 4096, 4096] shared by the batch (batch-inner work order,
    64-query dK/dV tiles), gradients and the bias gradient dS checked on whole
    sampled (batch, head) slices against the oracle."""
    B, H, N, D = 4, 32, 4096, 128
    q, k, v = wl.dense_inputs(B, H, N, N, D, "bf16", 0)
    do = wl.grad_output((B, H, N, D), "bf16", 0)
    bias = wl.score_bias((1, H, N, N), "bf16", 0)
    qc, kc, vc, doc, bc = (t.cuda() for t in (q, k, v, do, bias))
    o, lse = attn.fwd_bias(qc, kc, vc, bias=bc)
    dq, dk, dv, db = attn.bwd_bias(qc, kc, vc, o, doc, lse, bias=bc, return_dbias=True)
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for b, h in ((0, 5), (3, 30)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.attention_bwd(q[sl], k[sl], v[sl], do[sl], oracle.scale_as_passed(D ** -0.5),
                                   bias=bias[:, h:h + 1], with_dbias=True)
        got_db = db[b:b + 1, h:h + 1].cpu()
        check([dq[sl], dk[sl], dv[sl], got_db], list(ref[:3]) + [ref[3]], ["dq", "dk", "dv", "dbias"], "bf16",
              f"bias bwd [4,32,4096,128] operand [1,32,4096,4096] slice (b={b}, h={h})")
