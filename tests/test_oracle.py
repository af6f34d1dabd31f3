"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test fixes the oracle to something the mathematics or an independent
library determines: torch's own fp64 attention and forward-mode autodiff,
central finite differences, brute-force sums on tiny inputs, closed forms and
invariants.  Together they are chosen so that a dropped term, a wrong sign or
index, or a transposed operand in the oracle fails at least one of them
(tests/test_oracle_mutants.py plants such mistakes and checks exactly that).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def sdpa64(q, k, v, scale, causal):
    """torch's fp64 CPU attention (math path), an independent implementation."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
        return torch.nn.functional.scaled_dot_product_attention(
            t(q), t(k), t(v), is_causal=causal, scale=scale).numpy()


SHAPES = [  # B, H, Nq, Nkv, D, causal, scale
    (1, 1, 1, 1, 4, False, 0.5),
    (2, 3, 5, 7, 8, False, 0.37),
    (1, 2, 17, 17, 16, True, 0.25),
    (2, 1, 33, 33, 8, True, 1.0),
    (1, 2, 9, 31, 16, False, 16 ** -0.5),
]


@pytest.mark.parametrize("B,H,Nq,Nkv,D,causal,scale", SHAPES)
def test_output_matches_torch_attention(B, H, Nq, Nkv, D, causal, scale):
    q, k, v = rnd((B, H, Nq, D), 1), rnd((B, H, Nkv, D), 2), rnd((B, H, Nkv, D), 3)
    o, _ = oracle.attention(q, k, v, scale, causal)
    np.testing.assert_allclose(o, sdpa64(q, k, v, scale, causal), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_is_log_of_direct_sum(causal):
    """LSE_i = log sum_j exp(S_ij), summed without any max shift (small inputs)."""
    N, D, scale = 6, 3, 0.7
    q, k, v = rnd((1, 1, N, D), 4, 0.5), rnd((1, 1, N, D), 5, 0.5), rnd((1, 1, N, D), 6)
    _, lse = oracle.attention(q, k, v, scale, causal)
    for i in range(N):
        terms = []
        for j in range(N):
            if causal and j > i:
                continue
            s = scale * math.fsum(q[0, 0, i, d] * k[0, 0, j, d] for d in range(D))
            terms.append(math.exp(s))
        assert abs(lse[0, 0, i] - math.log(math.fsum(terms))) < 1e-13


def test_output_brute_force_loops():
    """O_i = sum_j exp(S_ij) v_j / sum_j exp(S_ij), in plain loops."""
    Nq, Nkv, D, scale = 4, 5, 3, 0.9
    q, k, v = rnd((1, 1, Nq, D), 7), rnd((1, 1, Nkv, D), 8), rnd((1, 1, Nkv, D), 9)
    o, _ = oracle.attention(q, k, v, scale, False)
    for i in range(Nq):
        w = [math.exp(scale * sum(q[0, 0, i, d] * k[0, 0, j, d] for d in range(D))) for j in range(Nkv)]
        for d in range(D):
            ref = sum(w[j] * v[0, 0, j, d] for j in range(Nkv)) / sum(w)
            assert abs(o[0, 0, i, d] - ref) < 1e-13


JVP_SHAPES = [(1, 1, 1, 1), (2, 3, 2, False), (4, 4, 4, True), (5, 7, 3, False), (6, 6, 5, True)]


@pytest.mark.parametrize("shape", JVP_SHAPES)
def test_jvp_matches_central_difference(shape):
    Nq, Nkv, D, causal = shape[0], shape[1], shape[2], (shape[3] if len(shape) > 3 else False)
    causal = bool(causal) and Nq == Nkv
    scale = 0.8
    q, k, v = rnd((1, 2, Nq, D), 10), rnd((1, 2, Nkv, D), 11), rnd((1, 2, Nkv, D), 12)
    tq, tk, tv = rnd(q.shape, 13), rnd(k.shape, 14), rnd(v.shape, 15)
    o, to, lse = oracle.attention_jvp(q, k, v, tq, tk, tv, scale, causal)
    h = 1e-6
    op, _ = oracle.attention(q + h * tq, k + h * tk, v + h * tv, scale, causal)
    om, _ = oracle.attention(q - h * tq, k - h * tk, v - h * tv, scale, causal)
    np.testing.assert_allclose(to, (op - om) / (2 * h), rtol=0, atol=1e-8)
    o2, lse2 = oracle.attention(q, k, v, scale, causal)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


@pytest.mark.parametrize("causal", [False, True])
def test_jvp_matches_torch_forward_autodiff(causal):
    N, D, scale = 9, 8, 8 ** -0.5
    q, k, v = rnd((2, 2, N, D), 16), rnd((2, 2, N, D), 17), rnd((2, 2, N, D), 18)
    tq, tk, tv = rnd(q.shape, 19), rnd(k.shape, 20), rnd(v.shape, 21)
    t = torch.from_numpy

    def f(a, b, c):
        with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
            return torch.nn.functional.scaled_dot_product_attention(a, b, c, is_causal=causal, scale=scale)

    _, ref = torch.func.jvp(f, (t(q), t(k), t(v)), (t(tq), t(tk), t(tv)))
    _, to, _ = oracle.attention_jvp(q, k, v, tq, tk, tv, scale, causal)
    np.testing.assert_allclose(to, ref.numpy(), rtol=0, atol=1e-12)


def test_identical_keys_average_values():
    """All keys equal: O_i = mean of the attended V rows, LSE_i = s_i + log n_i,
    and with tK = 0 the tangent is the mean of the attended tV rows."""
    N, D, scale = 7, 4, 0.6
    q, v, tq, tv = rnd((1, 1, N, D), 22), rnd((1, 1, N, D), 23), rnd((1, 1, N, D), 24), rnd((1, 1, N, D), 25)
    krow = rnd((D,), 26)
    k = np.broadcast_to(krow, (1, 1, N, D)).copy()
    for causal in (False, True):
        o, to, lse = oracle.attention_jvp(q, k, v, tq, np.zeros_like(k), tv, scale, causal)
        for i in range(N):
            n = i + 1 if causal else N
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n].mean(axis=0), atol=1e-13)
            np.testing.assert_allclose(to[0, 0, i], tv[0, 0, :n].mean(axis=0), atol=1e-13)
            assert abs(lse[0, 0, i] - (scale * q[0, 0, i] @ krow + math.log(n))) < 1e-13


def test_single_key():
    """One key: O = V_0, LSE = scale q.k_0, tO = tV_0 for any tQ, tK."""
    D, scale = 5, 0.45
    q, k, v = rnd((1, 2, 3, D), 27), rnd((1, 2, 1, D), 28), rnd((1, 2, 1, D), 29)
    tq, tk, tv = rnd(q.shape, 30), rnd(k.shape, 31), rnd(v.shape, 32)
    o, to, lse = oracle.attention_jvp(q, k, v, tq, tk, tv, scale, False)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), atol=1e-14)
    np.testing.assert_allclose(to, np.broadcast_to(tv, to.shape), atol=1e-13)
    np.testing.assert_allclose(lse, scale * np.einsum("bhid,bhd->bhi", q, k[:, :, 0]), atol=1e-14)


def test_causal_row_equals_prefix_attention():
    N, D, scale = 11, 6, 0.5
    q, k, v = rnd((1, 1, N, D), 33), rnd((1, 1, N, D), 34), rnd((1, 1, N, D), 35)
    tq, tk, tv = rnd(q.shape, 36), rnd(k.shape, 37), rnd(v.shape, 38)
    o, to, lse = oracle.attention_jvp(q, k, v, tq, tk, tv, scale, True)
    for i in range(N):
        sl = slice(0, i + 1)
        o1, to1, l1 = oracle.attention_jvp(q[:, :, i:i + 1], k[:, :, sl], v[:, :, sl],
                                           tq[:, :, i:i + 1], tk[:, :, sl], tv[:, :, sl], scale, False)
        np.testing.assert_allclose(o[:, :, i], o1[:, :, 0], atol=1e-14)
        np.testing.assert_allclose(to[:, :, i], to1[:, :, 0], atol=1e-13)
        np.testing.assert_allclose(lse[:, :, i], l1[:, :, 0], atol=1e-14)
    # row 0 attends only key 0
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-15)


def test_key_shift_and_value_shift():
    """k_j + u for every j leaves O unchanged and adds scale q_i.u to LSE_i;
    v_j + c for every j adds c to O (softmax rows sum to one)."""
    Nq, Nkv, D, scale = 6, 9, 4, 0.7
    q, k, v = rnd((1, 1, Nq, D), 39), rnd((1, 1, Nkv, D), 40), rnd((1, 1, Nkv, D), 41)
    u, c = rnd((D,), 42), rnd((D,), 43)
    o, lse = oracle.attention(q, k, v, scale, False)
    o2, lse2 = oracle.attention(q, k + u, v + c, scale, False)
    np.testing.assert_allclose(o2, o + c, atol=1e-13)
    np.testing.assert_allclose(lse2, lse + scale * (q @ u), atol=1e-12)


def test_jvp_special_cases_and_linearity():
    N, D, scale = 8, 4, 0.5
    q, k, v = rnd((1, 1, N, D), 44), rnd((1, 1, N, D), 45), rnd((1, 1, N, D), 46)
    z = np.zeros_like(q)
    tv = rnd(v.shape, 47)
    for causal in (False, True):
        # only tV: tO = attention(Q, K, tV)
        _, to, _ = oracle.attention_jvp(q, k, v, z, z, tv, scale, causal)
        o_tv, _ = oracle.attention(q, k, tv, scale, causal)
        np.testing.assert_allclose(to, o_tv, atol=1e-14)
        # tV = V: tO = O
        o, to, _ = oracle.attention_jvp(q, k, v, z, z, v, scale, causal)
        np.testing.assert_allclose(to, o, atol=1e-14)
        # linear in the tangents
        t1 = [rnd(q.shape, 48 + i) for i in range(3)]
        t2 = [rnd(q.shape, 52 + i) for i in range(3)]
        a, b = 0.7, -1.3
        _, r1, _ = oracle.attention_jvp(q, k, v, *t1, scale, causal)
        _, r2, _ = oracle.attention_jvp(q, k, v, *t2, scale, causal)
        _, r12, _ = oracle.attention_jvp(q, k, v, *[a * x + b * y for x, y in zip(t1, t2)], scale, causal)
        np.testing.assert_allclose(r12, a * r1 + b * r2, atol=1e-12)


def test_no_keys_gives_empty_rows():
    q = rnd((1, 2, 3, 4), 56)
    e = np.zeros((1, 2, 0, 4))
    o, to, lse = oracle.attention_jvp(q, e, e, q, e, e, 0.5, False)
    assert np.all(o == 0) and np.all(to == 0) and np.all(np.isneginf(lse))


def test_causal_needs_square():
    q = rnd((1, 1, 3, 4), 57)
    with pytest.raises(ValueError):
        oracle.attention(q, q[:, :, :2], q[:, :, :2], 0.5, True)


def test_sampled_rows_equal_full():
    B, H, N, D, scale = 2, 2, 40, 8, 0.35
    q, k, v = rnd((B, H, N, D), 58), rnd((B, H, N, D), 59), rnd((B, H, N, D), 60)
    tq, tk, tv = rnd(q.shape, 61), rnd(k.shape, 62), rnd(v.shape, 63)
    rows = [(0, 0, 0), (1, 1, 39), (0, 1, 17), (1, 0, 5)]
    for causal in (False, True):
        o, to, lse = oracle.attention_jvp(q, k, v, tq, tk, tv, scale, causal)
        so, sto, slse = oracle.attention_sampled(q, k, v, scale, causal, rows, tangents=(tq, tk, tv))
        for idx, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(so[idx], o[b, h, i], atol=1e-14)
            np.testing.assert_allclose(sto[idx], to[b, h, i], atol=1e-13)
            assert abs(slse[idx] - lse[b, h, i]) < 1e-14


# ---------------------------------------------------------------- jagged


def _jagged_case(lengths, H=2, D=4, seed=70):
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(offsets[-1])
    q, k, v = rnd((H, T, D), seed), rnd((H, T, D), seed + 1), rnd((H, T, D), seed + 2)
    return q, k, v, offsets


@pytest.mark.parametrize("causal", [False, True])
def test_jagged_is_dense_per_sequence(causal):
    lengths = [3, 0, 7, 1, 5]
    q, k, v, off = _jagged_case(lengths)
    o, lse = oracle.jagged_attention(q, k, v, off, 64, 0.6, causal)
    for s in range(len(lengths)):
        a, b = off[s], off[s + 1]
        if a == b:
            continue
        od, ld = oracle.attention(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], 0.6, causal)
        np.testing.assert_allclose(o[:, a:b], od[0], atol=1e-14)
        np.testing.assert_allclose(lse[:, a:b], ld[0], atol=1e-14)


def test_jagged_equal_lengths_is_dense_batch():
    S, L, H, D = 3, 6, 2, 4
    q, k, v, off = _jagged_case([L] * S, H=H, D=D, seed=80)
    o, lse = oracle.jagged_attention(q, k, v, off, L, 0.5, False)
    dense = lambda x: x.reshape(H, S, L, D).transpose(1, 0, 2, 3)  # [H, S*L, D] -> [S, H, L, D]
    od, ld = oracle.attention(dense(q), dense(k), dense(v), 0.5, False)
    np.testing.assert_allclose(dense(o), od, atol=1e-14)
    np.testing.assert_allclose(lse.reshape(H, S, L).transpose(1, 0, 2), ld, atol=1e-14)


def test_jagged_truncation_at_max_seq_len():
    """Only the first max_seq_len rows of a sequence take part, as queries and
    keys; later rows get O = 0 and LSE = -inf."""
    lengths, M = [9, 4], 5
    q, k, v, off = _jagged_case(lengths, seed=90)
    for causal in (False, True):
        o, lse = oracle.jagged_attention(q, k, v, off, M, 0.5, causal)
        # sequence 0: rows 0..4 attend keys 0..4 only
        od, ld = oracle.attention(q[None, :, 0:5], k[None, :, 0:5], v[None, :, 0:5], 0.5, causal)
        np.testing.assert_allclose(o[:, 0:5], od[0], atol=1e-14)
        np.testing.assert_allclose(lse[:, 0:5], ld[0], atol=1e-14)
        assert np.all(o[:, 5:9] == 0) and np.all(np.isneginf(lse[:, 5:9]))
        # sequence 1 is shorter than max_seq_len: untouched by truncation
        od, ld = oracle.attention(q[None, :, 9:13], k[None, :, 9:13], v[None, :, 9:13], 0.5, causal)
        np.testing.assert_allclose(o[:, 9:13], od[0], atol=1e-14)


def test_jagged_no_cross_sequence_attention():
    lengths = [4, 6, 3]
    q, k, v, off = _jagged_case(lengths, seed=100)
    o, lse = oracle.jagged_attention(q, k, v, off, 16, 0.5, False)
    k2, v2 = k.copy(), v.copy()
    k2[:, 4:10] += 5.0
    v2[:, 4:10] -= 3.0
    o2, lse2 = oracle.jagged_attention(q, k2, v2, off, 16, 0.5, False)
    np.testing.assert_array_equal(o[:, :4], o2[:, :4])
    np.testing.assert_array_equal(o[:, 10:], o2[:, 10:])
    np.testing.assert_array_equal(lse[:, :4], lse2[:, :4])
    assert not np.allclose(o[:, 4:10], o2[:, 4:10])


def test_jagged_jvp_is_dense_jvp_per_sequence():
    lengths = [5, 2, 6]
    q, k, v, off = _jagged_case(lengths, seed=110)
    tq, tk, tv = rnd(q.shape, 120), rnd(k.shape, 121), rnd(v.shape, 122)
    o, to, lse = oracle.jagged_attention_jvp(q, k, v, tq, tk, tv, off, 4, 0.5, False)
    for s in range(3):
        a, b = off[s], off[s + 1]
        u = min(b - a, 4)
        sl = slice(a, a + u)
        od, tod, ld = oracle.attention_jvp(q[None, :, sl], k[None, :, sl], v[None, :, sl],
                                           tq[None, :, sl], tk[None, :, sl], tv[None, :, sl], 0.5, False)
        np.testing.assert_allclose(to[:, sl], tod[0], atol=1e-13)
        assert np.all(to[:, a + u:b] == 0)


def test_jagged_rejects_bad_offsets():
    q = rnd((1, 5, 4), 130)
    with pytest.raises(ValueError):
        oracle.jagged_attention(q, q, q, np.array([0, 3, 2, 5]), 8, 0.5)
    with pytest.raises(ValueError):
        oracle.jagged_attention(q, q, q, np.array([0, 3, 4]), 8, 0.5)


# ---------------------------------------------------------------- closed forms


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_golden_two_key_closed_form():
    g = _load("two_key_closed_form.json")
    x = math.log(3.0) / 2.0
    q = np.array([[[[x, 0.0]]]])
    k = np.array([[[[1.0, 0.0], [-1.0, 0.0]]]])
    v = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    tq = np.array([[[[1.0, 0.0]]]])
    o, to, lse = oracle.attention_jvp(q, k, v, tq, np.zeros_like(k), np.zeros_like(v), 1.0, False)
    np.testing.assert_allclose(o[0, 0, 0], g["O"], atol=1e-15)
    np.testing.assert_allclose(to[0, 0, 0], g["tO"], atol=1e-15)
    assert abs(lse[0, 0, 0] - (2 * math.log(2.0) - 0.5 * math.log(3.0))) < 1e-15
    assert abs(g["LSE"] - (2 * math.log(2.0) - 0.5 * math.log(3.0))) < 1e-15


def test_golden_causal_equal_scores():
    g = _load("causal_equal_scores.json")
    N = len(g["O"])
    q = np.zeros((1, 1, N, 2))
    k = np.zeros((1, 1, N, 2))
    v = np.array(g["V"], dtype=np.float64).reshape(1, 1, N, 2)
    o, lse = oracle.attention(q, k, v, 0.125, True)
    np.testing.assert_allclose(o[0, 0], g["O"], atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], [math.log(i + 1) for i in range(N)], atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], g["LSE"], atol=1e-12)


@pytest.mark.parametrize("Dqk,Dv,causal", [(8, 16, False), (16, 4, True), (4, 12, True)])
def test_value_head_dim_differs(Dqk, Dv, causal):
    """JVP page, _attention.forward and _test_jvp_ca: v (and tv, o, to) carry
    their own head dim.  O against torch's attention (math backend, fp64) and
    tO against torch forward-mode autodiff of the plain definition."""
    N, scale = 9, Dqk ** -0.5
    q, k = rnd((2, 2, N, Dqk), 60), rnd((2, 2, N, Dqk), 61)
    v = rnd((2, 2, N, Dv), 62)
    tq, tk, tv = rnd(q.shape, 63), rnd(k.shape, 64), rnd(v.shape, 65)
    o, to, lse = oracle.attention_jvp(q, k, v, tq, tk, tv, scale, causal)
    assert o.shape == (2, 2, N, Dv) and to.shape == (2, 2, N, Dv) and lse.shape == (2, 2, N)
    t = torch.from_numpy
    with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
        ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal, scale=scale)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)

    def f(a, b, c):
        s = scale * a @ b.transpose(-1, -2)
        if causal:
            s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        return torch.softmax(s, dim=-1) @ c
    _, rto = torch.func.jvp(f, (t(q), t(k), t(v)), (t(tq), t(tk), t(tv)))
    np.testing.assert_allclose(to, rto.numpy(), rtol=0, atol=1e-12)


def _decode16(bits, exp_bits, man_bits):
    """IEEE-style binary16 layouts decoded from their definition: sign bit,
    exp_bits of biased exponent, man_bits of fraction; exponent 0 is
    subnormal (fraction * 2^(1 - bias - man_bits)), all ones is inf / NaN."""
    b = bits.astype(np.int64)
    sign = np.where((b >> (exp_bits + man_bits)) & 1, -1.0, 1.0)
    e = (b >> man_bits) & ((1 << exp_bits) - 1)
    f = (b & ((1 << man_bits) - 1)).astype(np.float64)
    bias = (1 << (exp_bits - 1)) - 1
    top = (1 << exp_bits) - 1
    normal = np.ldexp(f + (1 << man_bits), (e - bias - man_bits).astype(np.int64))
    sub = np.ldexp(f, np.full(e.shape, 1 - bias - man_bits, np.int64))
    val = np.where(e == 0, sub, normal)
    val = np.where(e == top, np.where(f == 0, np.inf, np.nan), val)
    return sign * val


@pytest.mark.parametrize("dtype,exp_bits,man_bits", [(torch.bfloat16, 8, 7), (torch.float16, 5, 10)])
def test_as_f64_widens_16bit_tensors_exactly(dtype, exp_bits, man_bits):
    """The widening every GPU parity test feeds through the oracle: all 65536
    bit patterns of the format (zeros, subnormals, the largest finite values,
    infinities, NaNs) as a CPU tensor become exactly the decoded value."""
    bits = np.arange(1 << 16, dtype=np.uint16)
    x = torch.from_numpy(bits.view(np.int16).copy()).view(dtype)
    got = oracle.as_f64(x)
    want = _decode16(bits, exp_bits, man_bits)
    assert got.dtype == np.float64 and got.shape == want.shape
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))  # -0.0 stays -0.0
    # spot values of the format's range
    tiny = 2.0 ** (2 - (1 << (exp_bits - 1)) - man_bits)  # smallest subnormal
    assert got[1] == tiny and got[0x8001] == -tiny
    top = (1 << exp_bits) - 2
    largest = (2.0 - 2.0 ** -man_bits) * 2.0 ** (top - ((1 << (exp_bits - 1)) - 1))
    assert got[(top << man_bits) | ((1 << man_bits) - 1)] == largest
