"""Oracle: log-sum-exp merge of chunk results and the ring-order driver.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The ring loop on "LongVILA Guide: 2M Context Multi-Modal AI Model", section
"Implementation: PyTorch Distributed Pipeline and Token Routing", visits one
KV chunk per ring step (the chunk received from the previous ring rank) and
folds each step's attention output into an accumulator.  That page adds the
separately-normalised outputs, which does not equal attention over the union
of the chunks.  The reading used here is the one under which chunking is
exact: each chunk result ``(O_c, LSE_c)`` is normalised over its own keys, and
two results over disjoint key sets combine as

    L = ln(exp(L_a) + exp(L_b))
    O = exp(L_a - L) * O_a + exp(L_b - L) * O_b,

which is the softmax over the union of the key sets.  ``(0, -inf)`` (no
visible key) is the identity of this operation, and merging two empty results
gives ``(0, -inf)`` rather than NaN.  Float64 throughout.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_forward


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Merge two chunk results over disjoint key sets.

    ``o_*``: ``[Sq, Hq, d]``; ``lse_*``: ``[Hq, Sq]``.  Returns ``(o, lse)``.
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    lse = np.logaddexp(lse_a, lse_b)  # -inf only where both are -inf
    live = np.isfinite(lse)
    safe = np.where(live, lse, 0.0)
    w_a = np.where(live, np.exp(lse_a - safe), 0.0)  # [Hq, Sq]
    w_b = np.where(live, np.exp(lse_b - safe), 0.0)
    o = w_a.T[:, :, None] * o_a + w_b.T[:, :, None] * o_b
    return o, lse


def ring_forward(q, k_chunks, v_chunks, q_pos, k_pos_chunks, scale=None, order=None, rows=None,
                 q_start=None):
    """Attention of ``q`` against a list of KV chunks, merged chunk by chunk.

    ``order`` is the visiting order of the chunk indices (ring order by
    default: chunk ``(r - t) mod P`` at step ``t`` when this is rank ``r`` --
    the caller passes it; the result does not depend on it up to rounding).
    """
    n_chunks = len(k_chunks)
    if order is None:
        order = list(range(n_chunks))
    o = None
    lse = None
    for c in order:
        o_c, l_c = attention_forward(q, k_chunks[c], v_chunks[c], q_pos, k_pos_chunks[c],
                                     scale=scale, rows=rows, q_start=q_start)
        if o is None:
            o, lse = o_c, l_c
        else:
            o, lse = lse_merge(o, lse, o_c, l_c)
    return o, lse
