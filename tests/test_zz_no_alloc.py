"""jagged_attn_fwd_noalloc (through the C ABI): the tile plan in the
library's static device scratch instead of a caller's workspace.  Checked
against jagged_attn_fwd on the same inputs over two calls in a row, the
second with a smaller input (so the scratch holds the first call's longer
plan when the second starts): the outputs must be bit-identical (the same
kernels compute the same items; only the plan's home differs), and within
the bf16 bounds of the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
import attention_forward_online_attn_amd as attn
from attention_forward_online_attn_amd import workloads as wl
from parity import assert_close, host64

pytestmark = pytest.mark.gpu


def _run(lengths, H, D, max_seq_len, causal, seed):
    lengths = torch.as_tensor(lengths, dtype=torch.int64)
    q, k, v, off = wl.jagged_inputs(lengths, H, D, "bf16", seed)
    qc, kc, vc, offc = (t.cuda() for t in (q, k, v, off))
    o_ws, l_ws = attn.jagged_fwd(qc, kc, vc, offc, max_seq_len, causal=causal)
    # outputs pre-filled with NaN: every element must be written
    o = torch.full_like(qc, float("nan"))
    lse = torch.full((H, q.shape[1]), float("nan"), dtype=torch.float32, device="cuda")
    o_na, l_na = attn.jagged_fwd_noalloc(qc, kc, vc, offc, max_seq_len, causal=causal, out=(o, lse))
    torch.cuda.synchronize()
    assert o_na.data_ptr() == o.data_ptr() and l_na.data_ptr() == lse.data_ptr()
    assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws)
    ro, rl = oracle.jagged_attention(q, k, v, off.numpy(), max_seq_len, oracle.scale_as_passed(D ** -0.5), causal)
    assert_close(torch.bfloat16, host64(o_na), host64(l_na), ro, rl,
                 label=f"noalloc jagged {len(lengths)} sequences H={H} D={D} causal={causal}")


def test_noalloc_matches_workspace_path_twice(gpu_lib):
    # first call: 96 sequences of lengths U[0, 700] (empty ones included),
    # 2 heads, D = 128 -> a plan of several hundred items
    lengths = wl.jagged_lengths(96, 700, 21)
    lengths[[3, 50]] = 0
    _run(lengths, 2, 128, 1024, False, 21)
    # second call on the same GPU, smaller: 5 sequences, one truncated at
    # max_seq_len, causal; the scratch still holds the longer first plan
    _run([130, 0, 1, 257, 64], 3, 64, 200, True, 22)


def test_noalloc_rejects_plans_beyond_the_scratch(gpu_lib):
    # 131071 one-row sequences need 131071 query tiles: one past the 2^20-byte scratch
    S = 131071
    q = torch.zeros((1, S, 64), dtype=torch.bfloat16, device="cuda")
    off = torch.arange(S + 1, dtype=torch.int64, device="cuda")
    with pytest.raises(attn.AttnError) as e:
        attn.jagged_fwd_noalloc(q, q, q, off, 16)
    assert e.value.status == -4 and "static scratch" in str(e.value)
    # one sequence fewer fits
    o, lse = attn.jagged_fwd_noalloc(q[:, :S - 1], q[:, :S - 1], q[:, :S - 1], off[:S], 16)
    torch.cuda.synchronize()
    assert torch.equal(o, torch.zeros_like(o)) and torch.all(lse == 0)
