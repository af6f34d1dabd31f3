"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pins catch every one of them.

Each mutant is the oracle's source with one textual change (a dropped term, a
wrong sign or index, an operand swapped).  The checks below are the same kinds
of pins as tests/test_oracle.py -- independent library, finite differences,
brute-force sums, invariants -- run against the mutated module; at least one
must fail for every mutant, and none may fail for the unmodified source.
"""

import inspect
import math
import types

import numpy as np
import pytest
import torch

import oracle

MUTANTS = {
    "drop_rho": ("tp = p * (ts - rho[:, None])", "tp = p * ts"),
    "drop_p_tv": ("tp @ v + p @ tv", "tp @ v"),
    "causal_off_by_one": ("cols[None, :] <= row_pos[r0:r1, None]", "cols[None, :] < row_pos[r0:r1, None]"),
    "causal_flipped": ("cols[None, :] <= row_pos[r0:r1, None]", "cols[None, :] >= row_pos[r0:r1, None]"),
    "tangent_operand_swapped": ("q[r0:r1] @ tk.T", "tq[r0:r1] @ k.T"),
    "lse_base2": ("m + np.log(safe)", "m + np.log2(safe)"),
    "lse_no_shift": ("m + np.log(safe)", "np.log(safe)"),
    "scale_dropped": ("s = scale * (q[r0:r1] @ k.T)", "s = (q[r0:r1] @ k.T)"),
    "tangent_scale_dropped": ("ts = scale * (tq[r0:r1] @ k.T", "ts = (tq[r0:r1] @ k.T"),
    "unnormalised": ("p = e / safe[:, None]", "p = e"),
    "keys_not_truncated": [("k[h, begin:begin + used], v[h, begin:begin + used]", "k[h, begin:end], v[h, begin:end]"),
                           ("kv_len = np.where(np.arange(n) < used, used, 0)", "kv_len = np.where(np.arange(n) < used, n, 0)")],
    "truncated_rows_attend": ("kv_len = np.where(np.arange(n) < used, used, 0)", "kv_len = np.where(np.arange(n) < used, used, used)"),
    "transposed_value_product": ("p @ v, 0.0)", "(v.T @ p.T).T[:, ::-1], 0.0)"),
    # backward
    "bwd_drop_delta": ("ds = p * (dp - delta[:, None])", "ds = p * dp"),
    "bwd_delta_sign": ("ds = p * (dp - delta[:, None])", "ds = p * (dp + delta[:, None])"),
    "bwd_dk_scale_dropped": ("dk += scale * (ds.T @ q[r0:r1])", "dk += (ds.T @ q[r0:r1])"),
    "bwd_dq_scale_dropped": ("dq[r0:r1] = scale * (ds @ k)", "dq[r0:r1] = (ds @ k)"),
    "bwd_dv_untransposed": ("dv += p.T @ g", "dv += p @ g"),
    "bwd_dk_wrong_operand": ("dk += scale * (ds.T @ q[r0:r1])", "dk += scale * (ds.T @ g)"),
    "bwd_dp_wrong_operand": ("dp = g @ v.T", "dp = g @ k.T"),
    "bwd_causal_dropped": ("allowed &= row_pos[r0:r1, None] >= cols[None, :]", "pass"),
    "bwd_delta_from_wrong_rows": ("delta = (o * g).sum(axis=1)", "delta = (o * g).sum(axis=0).sum() / o.shape[0] + 0 * g[:, 0]"),
    # additive bias and boolean mask
    "bias_sign": ("s = s + bias[r0:r1]", "s = s - bias[r0:r1]"),
    "bias_log2_units": ("s = s + bias[r0:r1]", "s = s + bias[r0:r1] / np.log(2.0)"),
    "bias_times_scale": ("s = s + bias[r0:r1]", "s = s + scale * bias[r0:r1]"),
    "bias_transposed": ("bias=None if bias is None else bias[b, h],\n", "bias=None if bias is None else bias[b, h].T,\n"),
    "mask_inverted": ("allowed &= mask[r0:r1]", "allowed &= ~mask[r0:r1]"),
    "mask_ignored": ("allowed &= mask[r0:r1]", "pass"),
    "neg_inf_bias_not_masked": ("allowed &= bias[r0:r1] != -np.inf  # a -inf bias masks the key", "pass"),
    "bwd_bias_dropped": ("            s = s + bias[r0:r1]\n            allowed &= bias[r0:r1] != -np.inf\n", "            pass\n"),
    "dbias_is_p": ("dbias[r0:r1] = ds", "dbias[r0:r1] = p"),
}


def _module(src):
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, scale, causal):
    t = torch.from_numpy
    with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
        return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal, scale=scale).numpy()


def _pins_hold(m) -> bool:
    """True when the module passes every pin used here."""
    try:
        q, k, v = rnd((1, 2, 6, 4), 1), rnd((1, 2, 6, 4), 2), rnd((1, 2, 6, 4), 3)
        tq, tk, tv = rnd(q.shape, 4), rnd(k.shape, 5), rnd(v.shape, 6)
        for causal in (False, True):
            o, lse = m.attention(q, k, v, 0.6, causal)
            if not np.allclose(o, _sdpa(q, k, v, 0.6, causal), atol=1e-12, rtol=0):
                return False
            # LSE by direct summation
            for h in range(2):
                for i in range(6):
                    js = range(i + 1) if causal else range(6)
                    ref = math.log(math.fsum(math.exp(0.6 * float(q[0, h, i] @ k[0, h, j])) for j in js))
                    if abs(lse[0, h, i] - ref) > 1e-12:
                        return False
            # JVP by central differences
            _, to, _ = m.attention_jvp(q, k, v, tq, tk, tv, 0.6, causal)
            e = 1e-6
            op, _ = m.attention(q + e * tq, k + e * tk, v + e * tv, 0.6, causal)
            om, _ = m.attention(q - e * tq, k - e * tk, v - e * tv, 0.6, causal)
            if not np.allclose(to, (op - om) / (2 * e), atol=1e-8, rtol=0):
                return False
        # backward: torch's fp64 reverse-mode autodiff of its own attention
        for causal in (False, True):
            qq, kk, vv, dd = rnd((1, 2, 7, 4), 11), rnd((1, 2, 7, 4), 12), rnd((1, 2, 7, 4), 13), rnd((1, 2, 7, 4), 14)
            tt = [torch.from_numpy(x).requires_grad_(True) for x in (qq, kk, vv)]
            with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
                oo = torch.nn.functional.scaled_dot_product_attention(*tt, is_causal=causal, scale=0.6)
            oo.backward(torch.from_numpy(dd))
            for got, ref in zip(m.attention_bwd(qq, kk, vv, dd, 0.6, causal), tt):
                if not np.allclose(got, ref.grad.numpy(), atol=1e-12, rtol=0):
                    return False
        # jagged with truncation equals dense attention on each sequence's leading rows
        lengths, M = [5, 2, 7], 4
        off = np.concatenate([[0], np.cumsum(lengths)])
        jq, jk, jv = rnd((2, 14, 4), 7), rnd((2, 14, 4), 8), rnd((2, 14, 4), 9)
        o, lse = m.jagged_attention(jq, jk, jv, off, M, 0.5, False)
        for s in range(3):
            a, b = off[s], off[s + 1]
            u = min(b - a, M)
            od = _sdpa(jq[None, :, a:a + u], jk[None, :, a:a + u], jv[None, :, a:a + u], 0.5, False)[0]
            if not np.allclose(o[:, a:a + u], od, atol=1e-12, rtol=0):
                return False
            if not (np.all(o[:, a + u:b] == 0) and np.all(np.isneginf(lse[:, a + u:b]))):
                return False
        # bias and mask: torch's attention with the same attn_mask, a fully
        # masked row, a -inf bias row, and the gradients (bias included)
        bq, bk, bv = rnd((1, 2, 5, 4), 21), rnd((1, 2, 7, 4), 22), rnd((1, 2, 7, 4), 23)
        bias, msk = rnd((1, 2, 5, 7), 24), np.random.default_rng(25).random((1, 2, 5, 7)) < 0.6
        msk[..., 1] = True
        o, _ = m.attention(bq, bk, bv, 0.6, bias=bias, mask=msk)
        tt = [torch.from_numpy(x) for x in (bq, bk, bv)]
        with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
            ref = torch.nn.functional.scaled_dot_product_attention(
                *tt, attn_mask=torch.from_numpy(np.where(msk, bias, -np.inf)), scale=0.6).numpy()
        if not np.allclose(o, ref, atol=1e-12, rtol=0):
            return False
        sq, sk, sv = rnd((1, 1, 6, 4), 26), rnd((1, 1, 6, 4), 27), rnd((1, 1, 6, 4), 28)
        ob, lb = m.attention(sq, sk, sv, 0.5, bias=rnd((1, 1, 6, 6), 29))
        ot, lt = m.attention(sq, sk, sv, 0.5, bias=rnd((1, 1, 6, 6), 29).transpose(0, 1, 3, 2))
        sb = rnd((1, 1, 6, 6), 29)
        with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
            rb = torch.nn.functional.scaled_dot_product_attention(
                *[torch.from_numpy(x) for x in (sq, sk, sv)], attn_mask=torch.from_numpy(sb), scale=0.5).numpy()
        if not np.allclose(ob, rb, atol=1e-12, rtol=0):
            return False
        em = np.ones((1, 1, 6, 6), bool)
        em[0, 0, 2] = False
        oe, le = m.attention(sq, sk, sv, 0.5, mask=em)
        oi, li = m.attention(sq, sk, sv, 0.5, bias=np.where(em, 0.0, -np.inf))
        for oo_, ll_ in ((oe, le), (oi, li)):
            if not (np.all(oo_[0, 0, 2] == 0) and np.isneginf(ll_[0, 0, 2]) and np.all(np.isfinite(oo_))):
                return False
        bd = rnd((1, 2, 5, 4), 30)
        tb = [torch.from_numpy(x).requires_grad_(True) for x in (bq, bk, bv, bias)]
        sc = (0.6 * tb[0] @ tb[1].transpose(-1, -2) + tb[3]).masked_fill(torch.from_numpy(~msk), float("-inf"))
        (torch.softmax(sc, dim=-1) @ tb[2]).backward(torch.from_numpy(bd))
        got = m.attention_bwd(bq, bk, bv, bd, 0.6, bias=bias, mask=msk, with_dbias=True)
        for g, r in zip(got, tb):
            if not np.allclose(g, r.grad.numpy(), atol=1e-12, rtol=0):
                return False
        return True
    except Exception:
        return False


SOURCE = inspect.getsource(oracle)


def test_unmodified_oracle_passes_the_pins():
    assert _pins_hold(_module(SOURCE))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    edits = MUTANTS[name]
    mutated = SOURCE
    for old, new in (edits if isinstance(edits, list) else [edits]):
        assert mutated.count(old) >= 1, f"mutation site for {name} not found in the oracle source"
        mutated = mutated.replace(old, new, 1)
    assert not _pins_hold(_module(mutated)), f"pins did not catch mutant {name}"
