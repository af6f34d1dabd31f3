"""fp64 CPU oracle for fused attention forward, its forward-mode JVP and the
jagged multi-head variant.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` call it.  It shares no code with the HIP library.

What it computes is the plain, materialised definition that the online-softmax
kernels reach up to rounding order (the rescaling by ``exp(m_old - m_new)`` in
those kernels is an exact identity, so the streamed result equals this one):

* Dense forward -- Triton fused attention tutorial with JVP
  (``_06_fused_attention_blockptr_jvp.py``), ``_attn_fwd`` / ``_attn_fwd_inner``
  and ``JVPAttn.forward``; the same operation on the "Flash Attention v2 with
  JVP" page (``flm/utils/jvp.py``), ``_attn_fwd``:
      S = sm_scale * Q K^T,  P = softmax_rows(S),  O = P V,
      LSE_i = log sum_j exp(S_ij)          (natural log, as that page stores)
* Causal mask -- both pages, the on-band stage of ``_attn_fwd_inner``:
  query i attends to key j only when j <= i (top-left aligned).
* Forward-mode JVP -- ``_attn_fwd_inner`` (tangent scores and the two extra
  accumulators) and the epilogue of ``_attn_fwd`` on both JVP pages; the
  closed form is the derivative of the definition above:
      tS = sm_scale * (tQ K^T + Q tK^T)   (0 where masked)
      rho_i = sum_j P_ij tS_ij
      tP = P * (tS - rho 1^T)
      tO = tP V + P tV
* Jagged multi-head layout -- FBGEMM SLL
  ``triton_multi_head_jagged_flash_attention.py``,
  ``_multi_head_jagged_flash_attention_fwd_kernel`` and the public wrapper's
  docstring: values are [H, total_len, D], sequence s owns rows
  [offsets[s], offsets[s+1]); only its first min(len_s, max_seq_len) rows take
  part, as queries and as keys; there is no attention across sequences.

* Additive bias and boolean mask -- flash attention with bias page
  (``flash_attention.py``), ``_attn_fwd_inner`` and ``_flash_attn_fwd``: a
  float bias [B, H, Nq, Nkv] is added to the scores in natural-log units (the
  wrapper divides it by ln 2 before the kernel's base-2 add, so the two
  agree), a boolean mask keeps key j for query i only where it is True:
      S = sm_scale * Q K^T + bias,   S_ij = -inf where mask_ij is False
  Both combine with the causal mask.  The bias has no tangent (it is not an
  input of the JVP), so tS is unchanged; its gradient is dS.

* Backward (the gradient of the forward above for a loss L with dL/dO = dO) --
  Triton fused attention tutorial with JVP, ``_attn_bwd_preprocess``,
  ``_attn_bwd_dkdv``, ``_attn_bwd_dq`` (the steps, in that page's order):
      delta_i = sum_d O_id dO_id                 (preprocess)
      dV = P^T dO,  dP = dO V^T,  dS = P * (dP - delta 1^T)
      dQ = sm_scale * dS K,  dK = sm_scale * dS^T Q
  P is the forward's softmax (0 where masked); rows without keys give dQ = 0
  and contribute nothing to dK, dV.

Readings where the pages are silent or differ (each is also listed in the
design notes):
* LSE is the natural log, fp32 on the GPU side (the JVP page stores
  ``m * ln2`` in fp32; the tutorial stores the base-2 value).
* A query row with no key to attend (Nkv = 0, or a jagged row at position
  >= max_seq_len inside its sequence) gives O = 0, tO = 0, LSE = -inf (the JVP
  page's empty-row epilogue).
* The jagged page divides p by max_seq_len before the PV product; that
  normalisation is not applied here: O = softmax(S) V like every other page.
* The jagged page applies no sm_scale; here the caller passes one (1.0
  reproduces that page's raw logits).
* The bias page masks with an additive -1e6, so a row whose mask is all
  False would attend every key; here masked scores are exactly -inf and such
  a row is empty (O = 0, LSE = -inf) like every other row without keys.  A
  bias of -inf masks its key the same way.

Everything is computed in float64 from the exact values the GPU receives
(bf16 -> fp64 and fp32 -> fp64 are exact); ``sm_scale`` is taken as the fp32
value that crosses the C ABI, widened to fp64.  Library primitives used as
steps: ``numpy.matmul`` (the products), ``numpy.exp``/``log``/``max``/``sum``.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "as_f64",
    "scale_as_passed",
    "attend_rows",
    "attention",
    "attention_jvp",
    "attention_sampled",
    "jagged_attention",
    "jagged_attention_jvp",
    "attend_rows_bwd",
    "attention_bwd",
    "jagged_attention_bwd",
    "dense_bias",
    "dense_mask",
]

# Rows of S materialised at a time.  Only bounds memory: every row is still
# computed from the whole materialised row of scores.
_ROW_BLOCK = 1024


def as_f64(x) -> np.ndarray:
    """Exact widening to float64 (accepts numpy arrays or CPU torch tensors)."""
    if hasattr(x, "detach"):  # torch tensor: bf16 has no numpy dtype, widen via fp32 (exact)
        x = x.detach().cpu()
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def scale_as_passed(sm_scale: float) -> float:
    """The softmax scale exactly as the fp32 value the GPU path receives."""
    return float(np.float32(sm_scale))


def attend_rows(q, k, v, sm_scale, causal=False, row_pos=None,
                tq=None, tk=None, tv=None, kv_len=None, with_tlse=False,
                bias=None, mask=None):
    """Attention of some query rows of one (batch, head) over all its keys.

    q:  [M, D] query rows;  k: [N, D];  v: [N, Dv].
    row_pos: [M] absolute position of each query row (for the causal mask);
             defaults to 0..M-1.
    kv_len:  [M] optional per-row number of leading keys the row may attend
             (the jagged truncation); keys j >= kv_len[i] are masked.
    tq/tk/tv: optional tangents shaped like q/k/v; when given the JVP output
             tO is returned as well.
    with_tlse: with tangents, also return the tangent of LSE,
             rho_i = sum_j P_ij tS_ij (0 for a row without keys).
    bias:    [M, N] optional float bias added to the scaled scores.
    mask:    [M, N] optional bool; False masks the key for that row.
    Returns (o [M, Dv], lse [M]), (o, to, lse) or (o, to, lse, tlse).
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    if bias is not None:
        bias = as_f64(bias)
    if mask is not None:
        mask = np.asarray(mask, dtype=bool)
    M, N = q.shape[0], k.shape[0]
    scale = float(sm_scale)
    jvp = tq is not None
    if jvp:
        tq, tk, tv = as_f64(tq), as_f64(tk), as_f64(tv)
    if row_pos is None:
        row_pos = np.arange(M)
    row_pos = np.asarray(row_pos, dtype=np.int64)

    o = np.zeros((M, v.shape[1]))
    lse = np.full(M, -np.inf)
    to = np.zeros((M, v.shape[1])) if jvp else None
    tlse = np.zeros(M) if jvp else None

    def result():
        if not jvp:
            return o, lse
        return (o, to, lse, tlse) if with_tlse else (o, to, lse)

    if N == 0 or M == 0:
        return result()

    cols = np.arange(N)
    for r0 in range(0, M, _ROW_BLOCK):
        r1 = min(M, r0 + _ROW_BLOCK)
        # scores S = sm_scale * Q K^T (+ bias) for this block of rows
        s = scale * (q[r0:r1] @ k.T)
        allowed = np.ones_like(s, dtype=bool)
        if bias is not None:
            s = s + bias[r0:r1]
            allowed &= bias[r0:r1] != -np.inf  # a -inf bias masks the key
        if mask is not None:
            allowed &= mask[r0:r1]
        if causal:  # query i attends key j only for j <= i
            allowed &= cols[None, :] <= row_pos[r0:r1, None]
        if kv_len is not None:
            allowed &= cols[None, :] < np.asarray(kv_len)[r0:r1, None]
        s = np.where(allowed, s, -np.inf)
        has_key = allowed.any(axis=1)

        # softmax over each row; the max shift only keeps exp in range
        m = np.where(has_key, s.max(axis=1, initial=-np.inf), 0.0)
        e = np.where(allowed, np.exp(s - m[:, None]), 0.0)
        denom = e.sum(axis=1)
        safe = np.where(has_key, denom, 1.0)
        p = e / safe[:, None]
        o[r0:r1] = np.where(has_key[:, None], p @ v, 0.0)
        lse[r0:r1] = np.where(has_key, m + np.log(safe), -np.inf)

        if jvp:
            # tangent of the scores, zero where masked
            ts = scale * (tq[r0:r1] @ k.T + q[r0:r1] @ tk.T)
            ts = np.where(allowed, ts, 0.0)
            rho = (p * ts).sum(axis=1)            # = tangent of LSE
            tp = p * (ts - rho[:, None])          # tangent of the softmax
            to[r0:r1] = np.where(has_key[:, None], tp @ v + p @ tv, 0.0)
            tlse[r0:r1] = np.where(has_key, rho, 0.0)
    return result()


def _check_dense(q, k, v, causal):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("dense tensors are [B, H, N, D]")
    if causal and q.shape[2] != k.shape[2]:
        raise ValueError("causal attention needs Nq == Nkv (top-left aligned mask)")


def dense_bias(bias, B, H, Nq, Nkv):
    """A float bias broadcast to [B, H, Nq, Nkv] (float64), or None."""
    return None if bias is None else np.broadcast_to(as_f64(bias), (B, H, Nq, Nkv))


def dense_mask(mask, B, H, Nq, Nkv):
    """A boolean mask (any nonzero value keeps the key) broadcast to
    [B, H, Nq, Nkv], or None."""
    if mask is None:
        return None
    if hasattr(mask, "detach"):
        mask = mask.detach().cpu().numpy()
    return np.broadcast_to(np.asarray(mask) != 0, (B, H, Nq, Nkv))


def attention(q, k, v, sm_scale, causal=False, bias=None, mask=None):
    """Dense attention forward.  q: [B,H,Nq,D], k/v: [B,H,Nkv,D]; optional
    bias / mask broadcastable to [B,H,Nq,Nkv].
    Returns (o [B,H,Nq,Dv], lse [B,H,Nq]) in float64."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    _check_dense(q, k, v, causal)
    B, H, Nq, _ = q.shape
    Nkv = k.shape[2]
    bias, mask = dense_bias(bias, B, H, Nq, Nkv), dense_mask(mask, B, H, Nq, Nkv)
    o = np.zeros((B, H, Nq, v.shape[3]))
    lse = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = attend_rows(q[b, h], k[b, h], v[b, h], sm_scale, causal,
                                             bias=None if bias is None else bias[b, h],
                                             mask=None if mask is None else mask[b, h])
    return o, lse


def attention_jvp(q, k, v, tq, tk, tv, sm_scale, causal=False, with_tlse=False, bias=None, mask=None):
    """Dense attention forward with its forward-mode JVP (bias and mask as in
    ``attention``; the bias has no tangent).
    Returns (o, to, lse), or (o, to, lse, tlse) with with_tlse, in float64."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    tq, tk, tv = as_f64(tq), as_f64(tk), as_f64(tv)
    _check_dense(q, k, v, causal)
    B, H, Nq, _ = q.shape
    Nkv = k.shape[2]
    bias, mask = dense_bias(bias, B, H, Nq, Nkv), dense_mask(mask, B, H, Nq, Nkv)
    o = np.zeros((B, H, Nq, v.shape[3]))
    to = np.zeros_like(o)
    lse = np.zeros((B, H, Nq))
    tlse = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            o[b, h], to[b, h], lse[b, h], tlse[b, h] = attend_rows(
                q[b, h], k[b, h], v[b, h], sm_scale, causal,
                tq=tq[b, h], tk=tk[b, h], tv=tv[b, h], with_tlse=True,
                bias=None if bias is None else bias[b, h], mask=None if mask is None else mask[b, h])
    return (o, to, lse, tlse) if with_tlse else (o, to, lse)


def attention_sampled(q, k, v, sm_scale, causal, rows, tangents=None, bias=None, mask=None):
    """Dense attention evaluated only at sampled outputs.

    rows: iterable of (b, h, i) query coordinates.  Each one is computed from
    its own full row of scores, so large problems can be checked row by row.
    bias / mask as in ``attention``.
    Returns (o [R, Dv], lse [R]) or, with tangents=(tq, tk, tv), (o, to, lse).
    """
    rows = list(rows)
    B, H, Nq, Nkv = q.shape[0], q.shape[1], q.shape[2], k.shape[2]
    bias, mask = dense_bias(bias, B, H, Nq, Nkv), dense_mask(mask, B, H, Nq, Nkv)
    R = len(rows)
    o = np.zeros((R, v.shape[3]))
    lse = np.zeros(R)
    to = np.zeros((R, v.shape[3])) if tangents is not None else None
    for idx, (b, h, i) in enumerate(rows):
        kw = {}
        if tangents is not None:
            tq, tk, tv = tangents
            kw = dict(tq=as_f64(tq[b, h, i:i + 1]), tk=as_f64(tk[b, h]), tv=as_f64(tv[b, h]))
        if bias is not None:
            kw["bias"] = bias[b, h, i:i + 1]
        if mask is not None:
            kw["mask"] = mask[b, h, i:i + 1]
        res = attend_rows(as_f64(q[b, h, i:i + 1]), as_f64(k[b, h]), as_f64(v[b, h]),
                          sm_scale, causal, row_pos=[i], **kw)
        if tangents is not None:
            o[idx], to[idx], lse[idx] = res[0][0], res[1][0], res[2][0]
        else:
            o[idx], lse[idx] = res[0][0], res[1][0]
    return (o, to, lse) if tangents is not None else (o, lse)


def _jagged(q, k, v, offsets, max_seq_len, sm_scale, causal, tangents):
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    offsets = np.asarray(offsets, dtype=np.int64)
    if q.ndim != 3:
        raise ValueError("jagged tensors are [H, total_len, D]")
    if max_seq_len < 1:
        raise ValueError("max_seq_len must be >= 1")
    H, T, _ = q.shape
    if offsets[0] != 0 or offsets[-1] != T or np.any(np.diff(offsets) < 0):
        raise ValueError("offsets must start at 0, be non-decreasing and end at total_len")
    jvp = tangents is not None
    if jvp:
        tq, tk, tv = (as_f64(t) for t in tangents)
    o = np.zeros((H, T, v.shape[2]))
    to = np.zeros_like(o) if jvp else None
    lse = np.full((H, T), -np.inf)
    for s in range(len(offsets) - 1):
        begin, end = int(offsets[s]), int(offsets[s + 1])
        n = end - begin
        if n == 0:
            continue
        used = min(n, int(max_seq_len))   # rows (and keys) that take part
        # rows at positions >= max_seq_len attend nothing: O = 0, LSE = -inf
        kv_len = np.where(np.arange(n) < used, used, 0)
        for h in range(H):
            kw = {}
            if jvp:
                kw = dict(tq=tq[h, begin:end], tk=tk[h, begin:begin + used], tv=tv[h, begin:begin + used])
            res = attend_rows(q[h, begin:end], k[h, begin:begin + used], v[h, begin:begin + used],
                              sm_scale, causal, kv_len=kv_len, **kw)
            if jvp:
                o[h, begin:end], to[h, begin:end], lse[h, begin:end] = res
            else:
                o[h, begin:end], lse[h, begin:end] = res
    return (o, to, lse) if jvp else (o, lse)


def jagged_attention(q, k, v, offsets, max_seq_len, sm_scale, causal=False):
    """Jagged multi-head attention forward.  q/k/v: [H, total_len, D];
    offsets: [num_seqs + 1] exclusive prefix sum of the lengths.
    Returns (o [H, total_len, Dv], lse [H, total_len]) in float64."""
    return _jagged(q, k, v, offsets, max_seq_len, sm_scale, causal, None)


def jagged_attention_jvp(q, k, v, tq, tk, tv, offsets, max_seq_len, sm_scale, causal=False):
    """Jagged attention with the forward-mode JVP.  Returns (o, to, lse)."""
    return _jagged(q, k, v, offsets, max_seq_len, sm_scale, causal, (tq, tk, tv))


def attend_rows_bwd(q, k, v, do, sm_scale, causal=False, row_pos=None, kv_len=None,
                    bias=None, mask=None, with_dbias=False):
    """Backward of ``attend_rows`` for some query rows of one (batch, head).

    q: [M, D], k: [N, D], v: [N, Dv], do: [M, Dv] (the gradient of the loss
    with respect to those rows of O).  row_pos / kv_len as in attend_rows.
    bias / mask as in attend_rows; with_dbias also returns dbias [M, N] = dS,
    the gradient with respect to the bias (0 where masked).
    Returns (dq [M, D], dk [N, D], dv [N, Dv]) (+ dbias); dk and dv collect
    the contributions of the given rows only.
    """
    q, k, v, do = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    if bias is not None:
        bias = as_f64(bias)
    if mask is not None:
        mask = np.asarray(mask, dtype=bool)
    M, N = q.shape[0], k.shape[0]
    scale = float(sm_scale)
    if row_pos is None:
        row_pos = np.arange(M)
    row_pos = np.asarray(row_pos, dtype=np.int64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dbias = np.zeros((M, N))

    def result():
        return (dq, dk, dv, dbias) if with_dbias else (dq, dk, dv)

    if N == 0 or M == 0:
        return result()

    cols = np.arange(N)
    for r0 in range(0, M, _ROW_BLOCK):
        r1 = min(M, r0 + _ROW_BLOCK)
        # forward of these rows: S, the mask and P = softmax(S)
        s = scale * (q[r0:r1] @ k.T)
        allowed = np.ones_like(s, dtype=bool)
        if bias is not None:
            s = s + bias[r0:r1]
            allowed &= bias[r0:r1] != -np.inf
        if mask is not None:
            allowed &= mask[r0:r1]
        if causal:  # key j is seen by query i only for i >= j
            allowed &= row_pos[r0:r1, None] >= cols[None, :]
        if kv_len is not None:
            allowed &= cols[None, :] < np.asarray(kv_len)[r0:r1, None]
        s = np.where(allowed, s, -np.inf)
        has_key = allowed.any(axis=1)
        m = np.where(has_key, s.max(axis=1, initial=-np.inf), 0.0)
        e = np.where(allowed, np.exp(s - m[:, None]), 0.0)
        denom = np.where(has_key, e.sum(axis=1), 1.0)
        p = e / denom[:, None]
        o = p @ v
        g = do[r0:r1]
        # preprocess: delta_i = sum_d O_id dO_id
        delta = (o * g).sum(axis=1)
        # dV = P^T dO; dP = dO V^T; dS = P (dP - delta); dQ, dK through S = scale Q K^T
        dv += p.T @ g
        dp = g @ v.T
        ds = p * (dp - delta[:, None])
        dq[r0:r1] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r0:r1])
        dbias[r0:r1] = ds
    return result()


def attention_bwd(q, k, v, do, sm_scale, causal=False, bias=None, mask=None, with_dbias=False):
    """Dense attention backward.  q: [B,H,Nq,D], k/v: [B,H,Nkv,D], do: [B,H,Nq,Dv];
    bias / mask as in ``attention``.
    Returns (dq, dk, dv) in float64, shaped like q, k, v, and with with_dbias
    also dbias [B,H,Nq,Nkv] = dS (sum it over broadcast dimensions for the
    gradient of a broadcast bias)."""
    q, k, v, do = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    _check_dense(q, k, v, causal)
    B, H, Nq = q.shape[:3]
    Nkv = k.shape[2]
    bias, mask = dense_bias(bias, B, H, Nq, Nkv), dense_mask(mask, B, H, Nq, Nkv)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dbias = np.zeros((B, H, Nq, Nkv))
    for b in range(B):
        for h in range(H):
            res = attend_rows_bwd(q[b, h], k[b, h], v[b, h], do[b, h], sm_scale, causal,
                                  bias=None if bias is None else bias[b, h],
                                  mask=None if mask is None else mask[b, h], with_dbias=True)
            dq[b, h], dk[b, h], dv[b, h], dbias[b, h] = res
    return (dq, dk, dv, dbias) if with_dbias else (dq, dk, dv)


def jagged_attention_bwd(q, k, v, do, offsets, max_seq_len, sm_scale, causal=False):
    """Jagged attention backward.  q/k/v/do: [H, total_len, D]; rows and keys
    at positions >= max_seq_len inside their sequence take no part (their
    gradients are 0).  Returns (dq, dk, dv) in float64."""
    q, k, v, do = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    offsets = np.asarray(offsets, dtype=np.int64)
    if q.ndim != 3:
        raise ValueError("jagged tensors are [H, total_len, D]")
    if max_seq_len < 1:
        raise ValueError("max_seq_len must be >= 1")
    H, T, _ = q.shape
    if offsets[0] != 0 or offsets[-1] != T or np.any(np.diff(offsets) < 0):
        raise ValueError("offsets must start at 0, be non-decreasing and end at total_len")
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for s in range(len(offsets) - 1):
        begin, end = int(offsets[s]), int(offsets[s + 1])
        used = min(end - begin, int(max_seq_len))
        if used == 0:
            continue
        for h in range(H):
            a, b_, c = attend_rows_bwd(q[h, begin:begin + used], k[h, begin:begin + used], v[h, begin:begin + used],
                                       do[h, begin:begin + used], sm_scale, causal)
            dq[h, begin:begin + used], dk[h, begin:begin + used], dv[h, begin:begin + used] = a, b_, c
    return dq, dk, dv
