"""Pins of the fp64 oracle's backward (CPU only).

The backward is fixed to things other than its own formulas: central finite
differences of the (separately pinned) forward, torch's fp64 reverse-mode
autodiff through its own attention, the adjoint identity with the (separately
pinned) forward-mode JVP, and closed-form invariants of the gradient.
"""

import numpy as np
import pytest
import torch

import oracle


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def loss(q, k, v, do, scale, causal):
    """L = <dO, O>: its gradient is what the backward computes."""
    o, _ = oracle.attention(q, k, v, scale, causal)
    return float(np.sum(o * do))


SHAPES = [  # Nq, Nkv, D, causal
    (5, 7, 4, False),
    (6, 6, 8, True),
    (1, 3, 4, False),
    (9, 9, 4, True),
]


@pytest.mark.parametrize("Nq,Nkv,D,causal", SHAPES)
def test_bwd_matches_central_difference(Nq, Nkv, D, causal):
    scale = 0.7
    q, k, v = rnd((1, 2, Nq, D), 1), rnd((1, 2, Nkv, D), 2), rnd((1, 2, Nkv, D), 3)
    do = rnd((1, 2, Nq, D), 4)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, causal)
    h = 1e-6
    for i, (x, g) in enumerate(((q, dq), (k, dk), (v, dv))):
        d = rnd(x.shape, 10 + i)
        args_p = [q, k, v]
        args_m = [q, k, v]
        args_p[i] = x + h * d
        args_m[i] = x - h * d
        fd = (loss(*args_p, do, scale, causal) - loss(*args_m, do, scale, causal)) / (2 * h)
        assert abs(fd - float(np.sum(g * d))) < 1e-7 * max(1.0, abs(fd)), (i, fd, float(np.sum(g * d)))


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_matches_torch_reverse_autodiff(causal):
    N, D, scale = 11, 8, 8 ** -0.5
    q, k, v = rnd((2, 2, N, D), 5), rnd((2, 2, N, D), 6), rnd((2, 2, N, D), 7)
    do = rnd((2, 2, N, D), 8)
    t = [torch.from_numpy(x).requires_grad_(True) for x in (q, k, v)]
    with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
        o = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal, scale=scale)
    o.backward(torch.from_numpy(do))
    for got, ref in zip(oracle.attention_bwd(q, k, v, do, scale, causal), t):
        np.testing.assert_allclose(got, ref.grad.numpy(), rtol=0, atol=1e-12)


def test_bwd_cross_attention_matches_torch():
    scale = 0.4
    q, k, v = rnd((1, 3, 4, 8), 9), rnd((1, 3, 13, 8), 10), rnd((1, 3, 13, 8), 11)
    do = rnd((1, 3, 4, 8), 12)
    t = [torch.from_numpy(x).requires_grad_(True) for x in (q, k, v)]
    o = torch.softmax(scale * t[0] @ t[1].transpose(-1, -2), dim=-1) @ t[2]  # plain definition, autodiff
    o.backward(torch.from_numpy(do))
    for got, ref in zip(oracle.attention_bwd(q, k, v, do, scale, False), t):
        np.testing.assert_allclose(got, ref.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_is_adjoint_of_jvp(causal):
    """<dO, J t> = <J^T dO, t> for every tangent t: the backward is the
    transpose of the (separately pinned) forward-mode JVP."""
    N, D, scale = 10, 4, 0.9
    q, k, v = rnd((1, 2, N, D), 13), rnd((1, 2, N, D), 14), rnd((1, 2, N, D), 15)
    do = rnd((1, 2, N, D), 16)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, causal)
    for seed in range(3):
        tq, tk, tv = rnd(q.shape, 20 + seed), rnd(k.shape, 30 + seed), rnd(v.shape, 40 + seed)
        _, to, _ = oracle.attention_jvp(q, k, v, tq, tk, tv, scale, causal)
        lhs = float(np.sum(do * to))
        rhs = float(np.sum(dq * tq) + np.sum(dk * tk) + np.sum(dv * tv))
        assert abs(lhs - rhs) < 1e-10 * max(1.0, abs(lhs))


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_invariants(causal):
    N, D, scale = 12, 8, 0.5
    q, k, v = rnd((1, 1, N, D), 17), rnd((1, 1, N, D), 18), rnd((1, 1, N, D), 19)
    do = rnd((1, 1, N, D), 20)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, causal)
    # each row of P sums to one: the value gradients add up to the output gradients
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=0, atol=1e-12)
    # each row of dS sums to zero (softmax is shift invariant): sum_j dK_j = 0
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, rtol=0, atol=1e-12)
    # identical keys: the weights do not depend on q, so dQ = 0
    kk = np.repeat(k[:, :, :1], N, axis=2)
    dq2, _, _ = oracle.attention_bwd(q, kk, v, do, scale, causal)
    np.testing.assert_allclose(dq2, 0.0, rtol=0, atol=1e-12)
    # linear in dO
    a = oracle.attention_bwd(q, k, v, 2.0 * do, scale, causal)
    for x, y in zip(a, (dq, dk, dv)):
        np.testing.assert_allclose(x, 2.0 * y, rtol=1e-13, atol=1e-14)


def test_bwd_causal_key_gradient_comes_from_later_queries():
    """With the causal mask, key j only sees queries i >= j: the gradients of
    the last key and value come from the last query alone."""
    N, D, scale = 7, 4, 0.8
    q, k, v = rnd((1, 1, N, D), 21), rnd((1, 1, N, D), 22), rnd((1, 1, N, D), 23)
    do = rnd((1, 1, N, D), 24)
    _, dk, dv = oracle.attention_bwd(q, k, v, do, scale, True)
    do_last = np.zeros_like(do)
    do_last[:, :, -1] = do[:, :, -1]
    _, dk_l, dv_l = oracle.attention_bwd(q, k, v, do_last, scale, True)
    np.testing.assert_allclose(dv[:, :, -1], dv_l[:, :, -1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk[:, :, -1], dk_l[:, :, -1], rtol=0, atol=1e-14)


def test_bwd_empty_and_degenerate():
    q, do = rnd((1, 1, 3, 4), 25), rnd((1, 1, 3, 4), 26)
    k = v = np.zeros((1, 1, 0, 4))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.5, False)
    assert np.all(dq == 0) and dk.shape == (1, 1, 0, 4) and dv.shape == (1, 1, 0, 4)
    # one key: O = v, so dV = sum of dO over rows and dQ = dK = 0
    k1, v1 = rnd((1, 1, 1, 4), 27), rnd((1, 1, 1, 4), 28)
    dq, dk, dv = oracle.attention_bwd(q, k1, v1, do, 0.5, False)
    np.testing.assert_allclose(dv[0, 0, 0], do[0, 0].sum(axis=0), atol=1e-14)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)


def test_jagged_bwd_is_dense_bwd_per_sequence():
    lengths, M, H, D, scale = [5, 0, 9, 3], 6, 2, 4, 0.6
    off = np.concatenate([[0], np.cumsum(lengths)])
    T = int(off[-1])
    q, k, v, do = (rnd((H, T, D), 30 + i) for i in range(4))
    for causal in (False, True):
        dq, dk, dv = oracle.jagged_attention_bwd(q, k, v, do, off, M, scale, causal)
        for s in range(len(lengths)):
            a, b = int(off[s]), int(off[s + 1])
            u = min(b - a, M)
            if u:
                ref = oracle.attention_bwd(q[None, :, a:a + u], k[None, :, a:a + u], v[None, :, a:a + u],
                                           do[None, :, a:a + u], scale, causal)
                for got, r in zip((dq, dk, dv), ref):
                    np.testing.assert_allclose(got[:, a:a + u], r[0], rtol=0, atol=1e-13)
            # rows and keys past max_seq_len take no part
            for g in (dq, dk, dv):
                assert np.all(g[:, a + u:b] == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_tlse_is_derivative_of_lse(causal):
    """tLSE = d/de LSE(q + e tq, k + e tk): central differences of the
    (separately pinned) forward oracle's LSE, and torch forward-mode autodiff of
    logsumexp over the masked scores."""
    N, D, scale = 9, 8, 0.6
    q, k, v = rnd((1, 2, N, D), 40), rnd((1, 2, N, D), 41), rnd((1, 2, N, D), 42)
    tq, tk, tv = rnd(q.shape, 43), rnd(k.shape, 44), rnd(v.shape, 45)
    _, _, _, tlse = oracle.attention_jvp(q, k, v, tq, tk, tv, scale, causal, with_tlse=True)
    h = 1e-6
    _, lp = oracle.attention(q + h * tq, k + h * tk, v, scale, causal)
    _, lm = oracle.attention(q - h * tq, k - h * tk, v, scale, causal)
    np.testing.assert_allclose(tlse, (lp - lm) / (2 * h), rtol=0, atol=1e-8)

    def lse_fn(a, b):
        s = scale * a @ b.transpose(-1, -2)
        if causal:
            s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        return torch.logsumexp(s, dim=-1)
    t = torch.from_numpy
    _, ref = torch.func.jvp(lse_fn, (t(q), t(k)), (t(tq), t(tk)))
    np.testing.assert_allclose(tlse, ref.numpy(), rtol=0, atol=1e-12)
    # the value tangent does not move the LSE
    _, _, _, tlse2 = oracle.attention_jvp(q, k, v, tq, tk, 5.0 * tv, scale, causal, with_tlse=True)
    np.testing.assert_array_equal(tlse, tlse2)
