"""GPU parity of the backward: attn_bwd (through the C ABI, fed with the
forward's own O and LSE) against the fp64 oracle's gradients on the same
seeded inputs.

The oracle computes dQ, dK, dV from q, k, v and dO alone (none of its inputs
or expected values come from the HIP path).  Bound for bf16 inputs, per
gradient: max|g - g_ref| <= 3e-2 * max|g_ref| + 1e-5, the relative bound
used for the JVP's tangent output, whose error has the same sources (P
rounded to bf16, a difference term, fp32 accumulation).  The absolute 1e-5
only matters where a gradient vanishes exactly (one key: dq = dk = 0), where
fp32 rounding of dP - delta leaves about 1e-7; gradients of N(0, 1) data are
of order 0.01 to 1.  fp16 inputs: 1e-2 relative (the tangent bound for fp16),
the same sources at fp16's 11-bit significand.  Each test prints the
achieved relative error.
"""

import numpy as np
import pytest
import torch

import oracle
import attention_forward_online_attn_amd as attn
from attention_forward_online_attn_amd import workloads as wl
from parity import assert_close, host64

pytestmark = pytest.mark.gpu

REL = {"bf16": 3e-2, "fp16": 1e-2}
ABS = 1e-5


def check_grads(got, ref, label, dtype="bf16"):
    rel = REL[dtype]
    msgs, ok = [], True
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = host64(g)
        gmax = float(np.max(np.abs(r), initial=0.0))
        diff = float(np.max(np.abs(g - r), initial=0.0)) if r.size else 0.0
        if not np.all(np.isfinite(g)):
            diff = np.inf
        msgs.append(f"{name} {diff / max(gmax, 1e-30):.2e} (max|g| {gmax:.2e})")
        ok = ok and diff <= rel * gmax + ABS
    msg = f"{label}: max|dg|/max|g| " + ", ".join(msgs) + f" (bound {rel:.0e} relative + {ABS:.0e})"
    print(msg, flush=True)
    assert ok, msg


def bwd_case(B, H, Nq, Nkv, D, causal, seed=0, scale=None, label=None, dtype="bf16"):
    q, k, v = wl.dense_inputs(B, H, Nq, Nkv, D, dtype, seed)
    do = wl.grad_output((B, H, Nq, D), dtype, seed)
    scale = D ** -0.5 if scale is None else scale
    qc, kc, vc, doc = (t.cuda() for t in (q, k, v, do))
    o, lse = attn.fwd(qc, kc, vc, causal=causal, sm_scale=scale)
    got = attn.bwd(qc, kc, vc, o, doc, lse, causal=causal, sm_scale=scale)
    ref = oracle.attention_bwd(q, k, v, do, oracle.scale_as_passed(scale), causal)
    check_grads(got, ref, label or f"bwd {B, H, Nq, Nkv, D} {dtype} causal={causal}", dtype)
    return got


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_tiles_and_ragged_tails(gpu_lib, D, causal):
    bwd_case(2, 3, 300, 300, D, causal, seed=1)     # several 128-row tiles, ragged tail


@pytest.mark.parametrize("D", [64, 128])
def test_bwd_full_size_causal(gpu_lib, D):
    bwd_case(2, 4, 1024, 1024, D, True, seed=2)


@pytest.mark.parametrize("N", [1, 31, 33, 129, 257])
def test_bwd_small_and_odd_lengths(gpu_lib, N):
    bwd_case(1, 2, N, N, 64, True, seed=3)
    bwd_case(1, 2, N, N, 128, False, seed=4)


def test_bwd_cross_attention(gpu_lib):
    bwd_case(1, 2, 100, 333, 128, False, seed=5)
    bwd_case(2, 1, 257, 64, 64, False, seed=6)


def test_bwd_no_keys_and_no_queries(gpu_lib):
    q = torch.randn(1, 2, 40, 64, device="cuda").bfloat16()
    k = torch.empty(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    o, lse = attn.fwd(q, k, k)
    dq, dk, dv = attn.bwd(q, k, k, o, torch.randn_like(q), lse)
    assert torch.all(dq == 0) and dk.numel() == 0 and dv.numel() == 0
    q0 = torch.empty(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    k1 = torch.randn(1, 2, 50, 64, device="cuda").bfloat16()
    dq, dk, dv = attn.bwd(q0, k1, k1, q0, q0, torch.empty(1, 2, 0, device="cuda"))
    assert dq.numel() == 0 and torch.all(dk == 0) and torch.all(dv == 0)


def test_bwd_deterministic(gpu_lib):
    q, k, v = (t.cuda() for t in wl.dense_inputs(2, 2, 500, 500, 128, "bf16", 7))
    do = wl.grad_output(q.shape, "bf16", 7).cuda()
    o, lse = attn.fwd(q, k, v, causal=True)
    a = attn.bwd(q, k, v, o, do, lse, causal=True)
    ws = torch.full((attn.bwd_workspace_bytes(2, 2, 500),), 0x7F, dtype=torch.uint8, device="cuda")
    b = attn.bwd(q, k, v, o, do, lse, causal=True, workspace=ws)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_strided_layouts(gpu_lib):
    """Inputs stored [B, N, H, D] and viewed as [B, H, N, D]."""
    B, H, N, D = 2, 3, 200, 64
    g = torch.Generator().manual_seed(8)
    base = [torch.randn(B, N, H, D, generator=g).bfloat16() for _ in range(4)]
    q, k, v, do = (x.permute(0, 2, 1, 3) for x in base)
    qc, kc, vc, doc = (x.cuda().permute(0, 2, 1, 3) for x in base)
    assert not qc.is_contiguous()
    o, lse = attn.fwd(qc, kc, vc)
    got = attn.bwd(qc, kc, vc, o, doc, lse)
    ref = oracle.attention_bwd(q, k, v, do, oracle.scale_as_passed(D ** -0.5), False)
    check_grads(got, ref, "bwd [B,N,H,D] storage")


def test_bwd_unscaled_logits(gpu_lib):
    """sm_scale = 1 on the N(0, 1) inputs as drawn: raw q.k logits of std 8
    (the SLL jagged page applies no scale), nearly one-hot rows."""
    B, H, N, D = 1, 2, 256, 64
    q, k, v = wl.dense_inputs(B, H, N, N, D, "bf16", 9)
    do = wl.grad_output(q.shape, "bf16", 9)
    qc, kc, vc, doc = (t.cuda() for t in (q, k, v, do))
    o, lse = attn.fwd(qc, kc, vc, causal=True, sm_scale=1.0)
    got = attn.bwd(qc, kc, vc, o, doc, lse, causal=True, sm_scale=1.0)
    check_grads(got, oracle.attention_bwd(q, k, v, do, 1.0, True), "bwd sm_scale=1")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_fp16(gpu_lib, D, causal):
    """fp16 inputs on the same kernels (fp16 MFMA products, P and dS rounded to fp16)."""
    bwd_case(2, 3, 300, 300, D, causal, seed=8, dtype="fp16")
    bwd_case(1, 2, 1024, 1024, D, causal, seed=9, dtype="fp16")


def test_bwd_fp16_odd_shapes(gpu_lib):
    bwd_case(1, 2, 1, 1, 64, True, seed=10, dtype="fp16")
    bwd_case(1, 2, 100, 333, 128, False, seed=11, dtype="fp16")


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_full_size_sampled_heads(gpu_lib, causal):
    """The benchmark's backward, B=4 H=32 N=4096 D=128 (4096 workgroups per
    gradient kernel, XCD-aware order), checked on whole (batch, head) slices:
    heads are independent, so the oracle computes the gradients of a few
    sampled slices exactly."""
    B, H, N, D = 4, 32, 4096, 128
    q, k, v = wl.dense_inputs(B, H, N, N, D, "bf16", 0)
    do = wl.grad_output((B, H, N, D), "bf16", 0)
    qc, kc, vc, doc = (t.cuda() for t in (q, k, v, do))
    o, lse = attn.fwd(qc, kc, vc, causal=causal)
    dq, dk, dv = (g.cpu() for g in attn.bwd(qc, kc, vc, o, doc, lse, causal=causal))
    o, lse = host64(o), host64(lse)
    del qc, kc, vc, doc
    for b, h in ((0, 0), (3, 31), (1, 17)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        # the forward those gradients start from, on the same whole slice
        ro, rl = oracle.attention(q[sl], k[sl], v[sl], oracle.scale_as_passed(D ** -0.5), causal)
        assert_close(torch.bfloat16, o[sl], lse[sl], ro, rl,
                     label=f"fwd [4,32,4096,128] causal={causal} slice (b={b}, h={h})")
        ref = oracle.attention_bwd(q[sl], k[sl], v[sl], do[sl], oracle.scale_as_passed(D ** -0.5), causal)
        check_grads((dq[sl], dk[sl], dv[sl]), ref, f"bwd [4,32,4096,128] causal={causal} slice (b={b}, h={h})")
