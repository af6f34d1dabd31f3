"""Pins of the fp64 oracle's additive bias and boolean mask (CPU only).

The bias page adds a float bias to the scores and masks with a boolean
tensor (flash attention with bias page, ``_attn_fwd_inner`` and
``_flash_attn_fwd``).  The oracle is fixed here to things other than its own
formulas: torch's scaled_dot_product_attention (math backend, fp64, whose
attn_mask has the same meaning), structural identities that hold for exact
attention (duplicating a key is a bias of ln 2; masking a key is removing it;
a per-row constant bias only shifts the LSE), finite differences and torch's
reverse-mode autodiff for the gradients, including the bias gradient.
"""

import math

import numpy as np
import pytest
import torch

import oracle


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def sdpa(q, k, v, scale, attn_mask=None, causal=False):
    t = torch.from_numpy
    m = None if attn_mask is None else (t(attn_mask) if not isinstance(attn_mask, torch.Tensor) else attn_mask)
    with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
        return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, is_causal=causal,
                                                                scale=scale).numpy()


def direct_lse(q, k, scale, bias_row, keep_row):
    """log sum_j exp(scale q.k_j + bias_j) over the kept keys, by fsum."""
    terms = [scale * float(q @ k[j]) + float(bias_row[j]) for j in range(k.shape[0]) if keep_row[j]]
    if not terms:
        return -math.inf
    m = max(terms)
    return m + math.log(math.fsum(math.exp(x - m) for x in terms))


@pytest.mark.parametrize("Nq,Nkv", [(6, 6), (5, 9), (1, 4)])
def test_bias_matches_torch_sdpa(Nq, Nkv):
    scale = 0.7
    q, k, v = rnd((2, 3, Nq, 8), 1), rnd((2, 3, Nkv, 8), 2), rnd((2, 3, Nkv, 8), 3)
    bias = rnd((2, 3, Nq, Nkv), 4, 2.0)
    o, lse = oracle.attention(q, k, v, scale, bias=bias)
    np.testing.assert_allclose(o, sdpa(q, k, v, scale, bias), rtol=0, atol=1e-12)
    keep = np.ones((Nq, Nkv), bool)
    for b, h, i in [(0, 0, 0), (1, 2, Nq - 1), (1, 0, Nq // 2)]:
        assert abs(lse[b, h, i] - direct_lse(q[b, h, i], k[b, h], scale, bias[b, h, i], keep[i])) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_mask_matches_torch_sdpa(causal):
    scale, N = 0.5, 7
    q, k, v = rnd((1, 2, N, 4), 5), rnd((1, 2, N, 4), 6), rnd((1, 2, N, 4), 7)
    mask = np.random.default_rng(8).random((1, 2, N, N)) < 0.6
    mask[..., 0] = True  # every row keeps key 0, so no row is empty and torch is defined
    o, lse = oracle.attention(q, k, v, scale, causal=causal, mask=mask)
    keep = mask & (np.tril(np.ones((N, N), bool)) if causal else True)
    np.testing.assert_allclose(o, sdpa(q, k, v, scale, keep), rtol=0, atol=1e-12)
    for h in range(2):
        for i in range(N):
            assert abs(lse[0, h, i] - direct_lse(q[0, h, i], k[0, h], scale, np.zeros(N), keep[0, h, i])) < 1e-12


def test_bias_and_mask_together_match_torch():
    scale = 0.9
    q, k, v = rnd((1, 2, 5, 4), 9), rnd((1, 2, 8, 4), 10), rnd((1, 2, 8, 4), 11)
    bias = rnd((1, 2, 5, 8), 12)
    mask = np.random.default_rng(13).random((1, 2, 5, 8)) < 0.5
    mask[..., 3] = True
    o, _ = oracle.attention(q, k, v, scale, bias=bias, mask=mask)
    np.testing.assert_allclose(o, sdpa(q, k, v, scale, np.where(mask, bias, -np.inf)), rtol=0, atol=1e-12)


def test_duplicated_key_is_a_bias_of_ln2():
    """Attention over keys (k_0..k_{N-1}, k_j) equals attention over k_0..k_{N-1}
    with a bias of ln 2 on key j: the bias is in natural-log units."""
    scale, N, j = 0.6, 6, 2
    q, k, v = rnd((1, 1, 4, 8), 14), rnd((1, 1, N, 8), 15), rnd((1, 1, N, 8), 16)
    k2 = np.concatenate([k, k[:, :, j:j + 1]], axis=2)
    v2 = np.concatenate([v, v[:, :, j:j + 1]], axis=2)
    o_dup, lse_dup = oracle.attention(q, k2, v2, scale)
    bias = np.zeros((1, 1, 4, N))
    bias[..., j] = math.log(2.0)
    o_b, lse_b = oracle.attention(q, k, v, scale, bias=bias)
    np.testing.assert_allclose(o_b, o_dup, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_b, lse_dup, rtol=0, atol=1e-13)


def test_masked_key_is_a_removed_key():
    scale, N, j = 0.6, 7, 4
    q, k, v = rnd((1, 2, 3, 8), 17), rnd((1, 2, N, 8), 18), rnd((1, 2, N, 8), 19)
    mask = np.ones((1, 2, 3, N), bool)
    mask[..., j] = False
    keep = [i for i in range(N) if i != j]
    o_m, lse_m = oracle.attention(q, k, v, scale, mask=mask)
    o_r, lse_r = oracle.attention(q, k[:, :, keep], v[:, :, keep], scale)
    np.testing.assert_allclose(o_m, o_r, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_m, lse_r, rtol=0, atol=1e-13)


def test_row_constant_bias_shifts_only_the_lse():
    scale = 0.8
    q, k, v = rnd((1, 2, 5, 4), 20), rnd((1, 2, 6, 4), 21), rnd((1, 2, 6, 4), 22)
    c = rnd((1, 2, 5, 1), 23, 3.0)
    o0, lse0 = oracle.attention(q, k, v, scale)
    o1, lse1 = oracle.attention(q, k, v, scale, bias=np.broadcast_to(c, (1, 2, 5, 6)))
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse1, lse0 + c[..., 0], rtol=0, atol=1e-13)


def test_lower_triangular_mask_is_causal():
    N = 9
    q, k, v = rnd((2, 2, N, 4), 24), rnd((2, 2, N, 4), 25), rnd((2, 2, N, 4), 26)
    o_c, lse_c = oracle.attention(q, k, v, 0.5, causal=True)
    o_m, lse_m = oracle.attention(q, k, v, 0.5, mask=np.tril(np.ones((N, N), bool)))
    np.testing.assert_array_equal(o_m, o_c)
    np.testing.assert_array_equal(lse_m, lse_c)


def test_fully_masked_rows_are_empty_and_neg_inf_bias_masks():
    N = 5
    q, k, v = rnd((1, 1, 4, 4), 27), rnd((1, 1, N, 4), 28), rnd((1, 1, N, 4), 29)
    mask = np.ones((1, 1, 4, N), bool)
    mask[0, 0, 1] = False
    mask[0, 0, 3, :2] = False
    o, lse = oracle.attention(q, k, v, 0.5, mask=mask)
    assert np.all(o[0, 0, 1] == 0) and np.isneginf(lse[0, 0, 1])
    assert np.all(np.isfinite(o)) and np.isfinite(lse[0, 0, [0, 2, 3]]).all()
    # a -inf bias is the same as a False mask entry
    bias = np.where(mask, 0.0, -np.inf)
    o2, lse2 = oracle.attention(q, k, v, 0.5, bias=bias)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(lse2, lse)


def test_broadcast_bias_equals_expanded_bias():
    q, k, v = rnd((2, 3, 4, 4), 30), rnd((2, 3, 6, 4), 31), rnd((2, 3, 6, 4), 32)
    small = rnd((1, 3, 1, 6), 33)
    o1, l1 = oracle.attention(q, k, v, 0.5, bias=small)
    o2, l2 = oracle.attention(q, k, v, 0.5, bias=np.ascontiguousarray(np.broadcast_to(small, (2, 3, 4, 6))))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_jvp_with_bias_matches_central_difference(causal):
    """The bias is a constant of the JVP: tO is the derivative of the
    (separately pinned) biased forward along (tq, tk, tv)."""
    N, scale = 7, 0.6
    q, k, v = rnd((1, 2, N, 4), 34), rnd((1, 2, N, 4), 35), rnd((1, 2, N, 4), 36)
    tq, tk, tv = rnd(q.shape, 37), rnd(k.shape, 38), rnd(v.shape, 39)
    bias = rnd((1, 2, N, N), 40)
    mask = np.random.default_rng(41).random((1, 2, N, N)) < 0.7
    mask[..., 0] = True
    _, to, _, tlse = oracle.attention_jvp(q, k, v, tq, tk, tv, scale, causal, with_tlse=True, bias=bias, mask=mask)
    e = 1e-6
    op, lp = oracle.attention(q + e * tq, k + e * tk, v + e * tv, scale, causal, bias=bias, mask=mask)
    om, lm = oracle.attention(q - e * tq, k - e * tk, v - e * tv, scale, causal, bias=bias, mask=mask)
    np.testing.assert_allclose(to, (op - om) / (2 * e), rtol=0, atol=1e-8)
    np.testing.assert_allclose(tlse, (lp - lm) / (2 * e), rtol=0, atol=1e-8)


def test_bwd_with_bias_matches_torch_autodiff():
    """dq, dk, dv and dbias against torch's fp64 reverse-mode autodiff of the
    plain definition softmax(scale q k^T + bias, masked) v."""
    scale, Nq, Nkv = 0.7, 6, 9
    q, k, v = rnd((1, 2, Nq, 4), 42), rnd((1, 2, Nkv, 4), 43), rnd((1, 2, Nkv, 4), 44)
    do, bias = rnd((1, 2, Nq, 4), 45), rnd((1, 2, Nq, Nkv), 46)
    mask = np.random.default_rng(47).random((1, 2, Nq, Nkv)) < 0.6
    mask[..., 2] = True
    t = [torch.from_numpy(x).requires_grad_(True) for x in (q, k, v, bias)]
    s = scale * t[0] @ t[1].transpose(-1, -2) + t[3]
    s = s.masked_fill(torch.from_numpy(~mask), float("-inf"))
    (torch.softmax(s, dim=-1) @ t[2]).backward(torch.from_numpy(do))
    got = oracle.attention_bwd(q, k, v, do, scale, bias=bias, mask=mask, with_dbias=True)
    for g, ref in zip(got, t):
        np.testing.assert_allclose(g, ref.grad.numpy(), rtol=0, atol=1e-12)


def test_dbias_matches_central_difference():
    scale, N = 0.5, 6
    q, k, v, do = rnd((1, 1, N, 4), 48), rnd((1, 1, N, 4), 49), rnd((1, 1, N, 4), 50), rnd((1, 1, N, 4), 51)
    bias, t = rnd((1, 1, N, N), 52), rnd((1, 1, N, N), 53)
    *_, dbias = oracle.attention_bwd(q, k, v, do, scale, causal=True, bias=bias, with_dbias=True)
    e = 1e-6
    lp = float(np.sum(oracle.attention(q, k, v, scale, True, bias=bias + e * t)[0] * do))
    lm = float(np.sum(oracle.attention(q, k, v, scale, True, bias=bias - e * t)[0] * do))
    assert abs((lp - lm) / (2 * e) - float(np.sum(dbias * t))) < 1e-8
    # masked (above-diagonal) entries carry no gradient
    assert np.all(dbias[0, 0][np.triu_indices(N, 1)] == 0)


def test_sampled_rows_with_bias_match_dense():
    q, k, v = rnd((2, 2, 9, 4), 54), rnd((2, 2, 9, 4), 55), rnd((2, 2, 9, 4), 56)
    bias = rnd((1, 2, 9, 9), 57)
    mask = np.random.default_rng(58).random((2, 1, 1, 9)) < 0.7
    mask[..., 0] = True
    o, lse = oracle.attention(q, k, v, 0.4, True, bias=bias, mask=mask)
    rows = [(0, 0, 0), (1, 1, 8), (0, 1, 4), (1, 0, 5)]
    so, sl = oracle.attention_sampled(q, k, v, 0.4, True, rows, bias=bias, mask=mask)
    for n, (b, h, i) in enumerate(rows):  # one row at a time: matmul rounding order differs
        np.testing.assert_allclose(so[n], o[b, h, i], rtol=0, atol=1e-13)
        assert abs(sl[n] - lse[b, h, i]) < 1e-13
