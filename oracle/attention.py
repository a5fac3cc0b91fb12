"""Oracle: causal attention of a query shard against one KV chunk (float64).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Definition followed ("LongVILA Guide: 2M Context Multi-Modal AI Model",
section "Implementation: PyTorch Distributed Pipeline and Token Routing",
the per-ring-step body of ``LongVILAMultiModalAttention.forward``): the
scores are the dot products of query and key rows divided by the square root
of the head dimension, turned into weights by a softmax over the keys, and the
output is the weighted sum of the value rows.

Readings added where that page is silent (each is listed in the design notes):

* causal visibility by global token position, diagonal included: key ``j`` is
  visible to query ``i`` iff ``k_pos[j] <= q_pos[i]`` (the model is a causal
  LM; the page's sample has no mask);
* the softmax runs over the visible keys of *this chunk only* and the
  function also returns ``LSE_i = ln sum_{j visible} exp(s_ij)`` (natural log),
  so that chunk results can be merged exactly (see :mod:`oracle.merge`);
* a row with no visible key has ``O_i = 0`` and ``LSE_i = -inf``;
* grouped-query attention maps query head ``h`` to KV head ``h // G`` with
  ``G = Hq / Hkv`` (contiguous groups).

Packed samples (same page, sections "Three-Stage Long-Context Alignment
Curriculum", stage 3 -- variable-length videos packed into one 2M-token
buffer -- and "Critical Operational Best Practices" -- packing with reset
attention masks): a query attends only to keys of its own sample.  Samples
occupy contiguous position ranges, so "same sample and ``k_pos <= q_pos``"
is exactly ``q_start[i] <= k_pos[j] <= q_pos[i]``, with ``q_start[i]`` the
first position of query ``i``'s sample; ``q_start`` is that optional argument.

Layouts: ``q[Sq, Hq, d]``, ``k, v[Sk, Hkv, d]`` (token-major), outputs
``o[Sq, Hq, d]`` and ``lse[Hq, Sq]``.  All arithmetic is float64.
"""

from __future__ import annotations

import numpy as np

_ROWS = 256  # query rows per block; blocking does not change the result


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def attention_forward(q, k, v, q_pos, k_pos, scale=None, rows=None, q_start=None):
    """Return ``(o, lse)`` of causal attention of ``q`` against ``(k, v)``.

    ``q``: ``[Sq, Hq, d]``; ``k``, ``v``: ``[Sk, Hkv, d]``; ``q_pos``: ``[Sq]``
    and ``k_pos``: ``[Sk]`` integer global positions.  ``scale`` defaults to
    ``1/sqrt(d)``.  ``rows`` optionally restricts the computation to a subset of
    query rows (the outputs then have ``len(rows)`` rows, in that order).
    ``q_start`` (``[Sq]``, optional): first position of each query's packed
    sample; keys before it are not visible.
    """
    q = _as64(q)
    k = _as64(k)
    v = _as64(v)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    sq, hq, d = q.shape
    sk, hkv, dk = k.shape
    q_start = (np.full(sq, np.iinfo(np.int64).min, dtype=np.int64) if q_start is None
               else np.asarray(q_start, dtype=np.int64))
    assert q_start.shape == (sq,)
    assert dk == d and v.shape == (sk, hkv, d)
    assert q_pos.shape == (sq,) and k_pos.shape == (sk,)
    assert hq % hkv == 0
    group = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if rows is None:
        rows = np.arange(sq)
    rows = np.asarray(rows, dtype=np.int64)
    n = rows.shape[0]
    o = np.zeros((n, hq, d), dtype=np.float64)
    lse = np.full((hq, n), -np.inf, dtype=np.float64)
    for h in range(hq):
        kv = h // group
        kh = k[:, kv, :]
        vh = v[:, kv, :]
        for b0 in range(0, n, _ROWS):
            r = rows[b0:b0 + _ROWS]
            qp = q_pos[r]
            qs = q_start[r]
            # keys visible to at least one row of the block; the others carry
            # zero weight for every row and are dropped before the product
            cols = np.nonzero((k_pos <= qp.max()) & (k_pos >= qs.min()))[0]
            if cols.size == 0:
                continue
            s = (q[r, h, :] @ kh[cols].T) * scale
            kc = k_pos[cols][None, :]
            vis = (kc <= qp[:, None]) & (kc >= qs[:, None])
            s = np.where(vis, s, -np.inf)
            has = vis.any(axis=1)
            m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
            e = np.where(vis, np.exp(s - m[:, None]), 0.0)
            tot = e.sum(axis=1)
            with np.errstate(divide="ignore"):
                l_blk = np.where(has, m + np.log(np.where(has, tot, 1.0)), -np.inf)
            w = np.where(has[:, None], e / np.where(has, tot, 1.0)[:, None], 0.0)
            o[b0:b0 + r.size, h, :] = w @ vh[cols]
            lse[h, b0:b0 + r.size] = l_blk
    return o, lse


def visible_pairs(q_pos, k_pos, q_start=None):
    """Number of ``(i, j)`` with ``q_start[i] <= k_pos[j] <= q_pos[i]`` (per head;
    no lower bound without ``q_start``).

    Counted with a sort and a search, independent of the attention above;
    used for the algorithmic FLOP count (4*d*pairs*Hq forward).
    """
    ks = np.sort(np.asarray(k_pos, dtype=np.int64))
    n = np.searchsorted(ks, np.asarray(q_pos, dtype=np.int64), side="right")
    if q_start is not None:
        n = n - np.searchsorted(ks, np.asarray(q_start, dtype=np.int64), side="left")
    return int(np.maximum(n, 0).sum())
