"""Oracle: gradients of chunked causal attention from the final LSE (float64).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The pages train the 2M-token model without gradient checkpointing ("LongVILA
- ... (Jason's Study)", section "What it is"; the Chinese news page makes the
same statement), so the backward consumes the forward's saved output ``O`` and
log-sum-exp rather than recomputing the layer.  The gradients themselves are
the plain calculus of the forward definition in :mod:`oracle.attention`,
evaluated per chunk with the *final* (all-chunk) LSE:

    P_ij  = exp(s_ij - LSE_i)        for visible j, else 0
    dV_j  = sum_i P_ij dO_i
    dP_ij = dO_i . v_j
    D_i   = dO_i . O_i               (O = final merged output)
    dS_ij = P_ij (dP_ij - D_i)
    dQ_i  = scale * sum_j dS_ij k_j
    dK_j  = scale * sum_i dS_ij q_i

For grouped-query attention dK and dV of a KV head are summed over the query
heads mapped to it (``h // G``).  Summing the per-chunk ``dQ`` over all chunks
gives the gradient of the full attention.
"""

from __future__ import annotations

import numpy as np

_ROWS = 256


def bwd_delta(o, do):
    """``D[h, i] = sum_c dO[i, h, c] * O[i, h, c]`` as ``[Hq, Sq]``."""
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    return np.einsum("ihc,ihc->hi", do, o)


def attention_backward(q, k, v, do, lse, delta, q_pos, k_pos, scale=None, q_start=None):
    """Return ``(dq, dk, dv)`` of one chunk.

    ``q, do``: ``[Sq, Hq, d]``; ``k, v``: ``[Sk, Hkv, d]``; ``lse, delta``:
    ``[Hq, Sq]`` (final LSE over all chunks, and ``D`` from :func:`bwd_delta`).
    ``dq`` is this chunk's contribution ``[Sq, Hq, d]``; ``dk, dv`` are
    ``[Sk, Hkv, d]``.  ``q_start`` as in :func:`oracle.attention.attention_forward`.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    delta = np.asarray(delta, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    sq, hq, d = q.shape
    sk, hkv, _ = k.shape
    q_start = (np.full(sq, np.iinfo(np.int64).min, dtype=np.int64) if q_start is None
               else np.asarray(q_start, dtype=np.int64))
    group = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(hq):
        kv = h // group
        kh = k[:, kv, :]
        vh = v[:, kv, :]
        for b0 in range(0, sq, _ROWS):
            r = slice(b0, min(b0 + _ROWS, sq))
            qp = q_pos[r]
            qs = q_start[r]
            cols = np.nonzero((k_pos <= qp.max()) & (k_pos >= qs.min()))[0]
            if cols.size == 0:
                continue
            kc = k_pos[cols][None, :]
            vis = (kc <= qp[:, None]) & (kc >= qs[:, None])
            l_r = lse[h, r]
            live = np.isfinite(l_r)
            s = (q[r, h, :] @ kh[cols].T) * scale
            p = np.where(vis & live[:, None],
                         np.exp(s - np.where(live, l_r, 0.0)[:, None]), 0.0)
            dv[cols, kv, :] += p.T @ do[r, h, :]
            dp = do[r, h, :] @ vh[cols].T
            ds = p * (dp - delta[h, r][:, None])
            dq[r, h, :] += scale * (ds @ kh[cols])
            dk[cols, kv, :] += scale * (ds.T @ q[r, h, :])
    return dq, dk, dv


def attention_abs_dp(q, k, v, do, lse, q_pos, k_pos, scale=None, q_start=None):
    """``C[h, i] = sum_j P_ij |dO_i . v_j|`` over this chunk's visible keys (``[Hq, Sq]``).

    Summed over all chunks it bounds how far ``D_i = dO_i . O_i`` moves when
    ``O`` is computed with every weight ``P_ij`` off by a relative error of at
    most ``u`` (weights rounded to bf16 before the ``P V`` contraction): that
    moves ``O_i`` by ``sum_j e_ij P_ij v_j``, hence ``D_i`` by
    ``sum_j e_ij P_ij dP_ij``, at most ``u * C_i``.  Inputs as in
    :func:`attention_backward`.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    sq, hq, d = q.shape
    sk, hkv, _ = k.shape
    q_start = (np.full(sq, np.iinfo(np.int64).min, dtype=np.int64) if q_start is None
               else np.asarray(q_start, dtype=np.int64))
    group = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((hq, sq))
    for h in range(hq):
        kv = h // group
        for b0 in range(0, sq, _ROWS):
            r = slice(b0, min(b0 + _ROWS, sq))
            qp = q_pos[r]
            qs = q_start[r]
            cols = np.nonzero((k_pos <= qp.max()) & (k_pos >= qs.min()))[0]
            if cols.size == 0:
                continue
            kc = k_pos[cols][None, :]
            vis = (kc <= qp[:, None]) & (kc >= qs[:, None])
            l_r = lse[h, r]
            live = np.isfinite(l_r)
            s = (q[r, h, :] @ k[cols, kv, :].T) * scale
            p = np.where(vis & live[:, None],
                         np.exp(s - np.where(live, l_r, 0.0)[:, None]), 0.0)
            out[h, r] += (p * np.abs(do[r, h, :] @ v[cols, kv, :].T)).sum(axis=1)
    return out


def attention_backward_magnitudes(q, k, v, do, o, lse, q_pos, k_pos, scale=None, q_start=None,
                                  dp_abs=None):
    """Sums of absolute terms of each gradient element of one chunk.

    A backward that rounds ``P`` and ``dS`` to a format with unit roundoff
    ``u``, and takes ``D`` from the same format's rounding of an ``O`` that
    was itself computed with weights rounded that way, errs on each element
    by at most about ``u`` times these sums:

        Mv_j  = sum_i P_ij |dO_i|
        Mq_i  = scale * sum_j (|dS_ij| + P_ij A_i) |k_j|
        Mk_j  = scale * sum_i (|dS_ij| + P_ij A_i) |q_i|
        A_i   = sum_c |dO_ic O_ic| + C_i

    (elementwise absolute values; same layouts as :func:`attention_backward`).
    ``u * A_i`` bounds the error of ``D_i``: ``sum_c |dO_ic O_ic|`` covers
    rounding ``O`` itself, ``C_i = sum_j P_ij |dO_i . v_j|`` over *all* chunks
    (:func:`attention_abs_dp`) covers the rounded weights of the forward.
    ``dp_abs`` is that all-chunk ``C`` (``[Hq, Sq]``); when omitted, this
    chunk's own sum is used, which is the whole of it for a single chunk.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    sq, hq, d = q.shape
    sk, hkv, _ = k.shape
    q_start = (np.full(sq, np.iinfo(np.int64).min, dtype=np.int64) if q_start is None
               else np.asarray(q_start, dtype=np.int64))
    group = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    delta = bwd_delta(o, do)
    absd = np.einsum("ihc,ihc->hi", np.abs(do), np.abs(o))
    if dp_abs is not None:
        dp_abs = np.asarray(dp_abs, dtype=np.float64)
    mq = np.zeros_like(q)
    mk = np.zeros_like(k)
    mv = np.zeros_like(v)
    for h in range(hq):
        kv = h // group
        kh = k[:, kv, :]
        vh = v[:, kv, :]
        for b0 in range(0, sq, _ROWS):
            r = slice(b0, min(b0 + _ROWS, sq))
            qp = q_pos[r]
            qs = q_start[r]
            cols = np.nonzero((k_pos <= qp.max()) & (k_pos >= qs.min()))[0]
            if cols.size == 0:
                continue
            kc = k_pos[cols][None, :]
            vis = (kc <= qp[:, None]) & (kc >= qs[:, None])
            l_r = lse[h, r]
            live = np.isfinite(l_r)
            s = (q[r, h, :] @ kh[cols].T) * scale
            p = np.where(vis & live[:, None],
                         np.exp(s - np.where(live, l_r, 0.0)[:, None]), 0.0)
            dp = do[r, h, :] @ vh[cols].T
            c_abs = (p * np.abs(dp)).sum(axis=1) if dp_abs is None else dp_abs[h, r]
            a_row = absd[h, r] + c_abs
            w = np.abs(p * (dp - delta[h, r][:, None])) + p * a_row[:, None]
            mv[cols, kv, :] += p.T @ np.abs(do[r, h, :])
            mq[r, h, :] += scale * (w @ np.abs(kh[cols]))
            mk[cols, kv, :] += scale * (w.T @ np.abs(q[r, h, :]))
    return mq, mk, mv
