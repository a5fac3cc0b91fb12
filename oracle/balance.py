"""Oracle: shard permutations that give every rank equal causal work.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The pages state the problem, not an algorithm: modality-switching boundaries
leave one rank with pure text and another with dense visual patches, which
stalls the collective steps ("LongVILA Guide: 2M Context Multi-Modal AI
Model", section "Problem", item 2), and a load-aware dispatch by the token
density of each modality is the remedy ("Ultra-Large Multimodal LLM
Inference ...", section 4, "Load Balancing for Tensor Parallelism").  Under a
causal mask, query position ``p`` attends to ``p + 1`` keys, so equal token
counts are not equal work.  The two permutations below are this project's
definitions (listed with the other readings in the design notes):

ZIGZAG(N, P)
    Requires ``N % 2P == 0``; ``L = N / 2P``.  Rank ``r`` owns global
    positions ``[r L, (r+1) L)`` followed by ``[(2P-1-r) L, (2P-r) L)``.

MODALITY(labels, P, g)
    Requires ``N % (2 P g) == 0``.  The stream is cut into blocks of ``g``
    tokens; block ``b``'s visual count is ``vis[b]``.  Rounds ``j = 0, 1, ...``
    each hold ``2P`` consecutive blocks, paired outside-in: pair ``a`` is
    blocks ``(2jP + a, 2jP + 2P - 1 - a)`` with visual count ``pv[a]``.  Within
    a round the pairs are taken in order of decreasing ``pv`` (ties: smaller
    ``a`` first) and handed to the ranks in order of increasing running visual
    total ``cum`` (ties: smaller rank first); the k-th pair goes to the k-th
    rank.  Each rank then lists its blocks in ascending order.

ZIGZAG_PACKED(starts, P)
    Packed samples (variable-length videos packed into one buffer with reset
    attention masks: same page, "Three-Stage Long-Context Alignment
    Curriculum", stage 3, and "Critical Operational Best Practices").  A query
    sees only its own sample, so the causal work of a sample is that of a
    stream of its own length, and a single zigzag over the whole buffer no
    longer balances it.  Each sample ``s`` (positions ``[starts[s],
    starts[s+1])``, length a multiple of ``2P``, ``L_s = len / 2P``) is
    zigzagged on its own: rank ``r`` takes its blocks ``r`` and ``2P-1-r``.
    Rank ``r`` lists, sample by sample, its low block then its high block;
    every rank gets ``2 L_s`` tokens and exactly equal work of every sample.
    Also returned: ``token_start[i]``, the first position of the sample of the
    token in slot ``i`` (the ``q_start`` of the attention with packed samples).

Output layout (all modes): ``perm`` is rank-major, rank ``r``'s
``N / P`` global positions are ``perm[r N/P : (r+1) N/P]`` in ascending order.

Why the work is exactly equal: the causal work of block ``b`` is
``g^2 b + g (g+1) / 2``, and both blocks of every pair in a round have the same
index sum, so any assignment of pairs to ranks gives equal work.  Integer
arithmetic and fixed tie-breaks make the result unique.

Parity of MODALITY's particular assignment is pinned by its definition and
invariants (bijection, equal counts, exactly equal work, ascending order, the
visual-spread bound, reduction to ZIGZAG-at-granularity-g for constant
labels), not by a number printed on the pages, which print none.
"""

from __future__ import annotations

import numpy as np


def zigzag_perm(n: int, p: int) -> np.ndarray:
    """ZIGZAG permutation (int64, rank-major)."""
    if n % (2 * p) != 0:
        raise ValueError("zigzag needs n % (2p) == 0")
    half = n // (2 * p)
    out = []
    for r in range(p):
        out.append(np.arange(r * half, (r + 1) * half))
        out.append(np.arange((2 * p - 1 - r) * half, (2 * p - r) * half))
    return np.concatenate(out).astype(np.int64)


def modality_perm(labels, p: int, g: int) -> np.ndarray:
    """MODALITY permutation (int64, rank-major); ``labels`` is 0 text / 1 visual."""
    labels = np.asarray(labels).astype(np.int64)
    n = labels.shape[0]
    if n % (2 * p * g) != 0:
        raise ValueError("modality balance needs n % (2 p g) == 0")
    n_blocks = n // g
    rounds = n_blocks // (2 * p)
    vis = [int(labels[b * g:(b + 1) * g].sum()) for b in range(n_blocks)]
    cum = [0] * p
    owned = [[] for _ in range(p)]
    for j in range(rounds):
        base = 2 * j * p
        pairs = []
        for a in range(p):
            b_lo = base + a
            b_hi = base + 2 * p - 1 - a
            pairs.append((-(vis[b_lo] + vis[b_hi]), a, b_lo, b_hi))
        pairs.sort()
        ranks = sorted(range(p), key=lambda r: (cum[r], r))
        for (neg_pv, _a, b_lo, b_hi), r in zip(pairs, ranks):
            owned[r].extend([b_lo, b_hi])
            cum[r] += -neg_pv
    out = []
    for r in range(p):
        for b in sorted(owned[r]):
            out.append(np.arange(b * g, (b + 1) * g))
    return np.concatenate(out).astype(np.int64)


def zigzag_packed_perm(starts, p: int):
    """ZIGZAG_PACKED permutation: ``(perm, token_start)``, both int64, rank-major.

    ``starts``: ``n_samples + 1`` ascending positions, ``starts[0] == 0`` and
    the last equal to ``N``; every sample length a multiple of ``2p``.
    """
    starts = [int(x) for x in starts]
    if starts[0] != 0 or any(b - a <= 0 or (b - a) % (2 * p) for a, b in zip(starts, starts[1:])):
        raise ValueError("packed zigzag needs samples of positive length divisible by 2p")
    perm = [[] for _ in range(p)]
    first = [[] for _ in range(p)]
    for a, b in zip(starts, starts[1:]):
        half = (b - a) // (2 * p)
        for r in range(p):
            for blk in (r, 2 * p - 1 - r):
                perm[r].extend(range(a + blk * half, a + (blk + 1) * half))
                first[r].extend([a] * half)
    return (np.concatenate([np.asarray(x, dtype=np.int64) for x in perm]),
            np.concatenate([np.asarray(x, dtype=np.int64) for x in first]))


def inverse_perm(perm) -> np.ndarray:
    """``inv[perm[i]] = i``."""
    perm = np.asarray(perm, dtype=np.int64)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.shape[0])
    return inv


def causal_work_per_rank(perm, p: int) -> np.ndarray:
    """Sum over each rank's positions of ``pos + 1`` (visible keys per query)."""
    perm = np.asarray(perm, dtype=np.int64)
    return (perm + 1).reshape(p, -1).sum(axis=1)


def visual_per_rank(perm, labels, p: int) -> np.ndarray:
    """Visual-token count of each rank's shard."""
    labels = np.asarray(labels).astype(np.int64)
    return labels[np.asarray(perm, dtype=np.int64)].reshape(p, -1).sum(axis=1)


def gather_rows(x, rows) -> np.ndarray:
    """A rank's rows in shard order: ``out[i] = x[rows[i]]``, a zero row where
    ``rows[i]`` does not index ``x`` (the unplaced ``-1`` slots).  The plain
    definition of moving a token-major tensor into the balanced shard order."""
    x = np.asarray(x)
    out = np.zeros((len(rows),) + x.shape[1:], dtype=x.dtype)
    for i, r in enumerate(np.asarray(rows).tolist()):
        if 0 <= r < x.shape[0]:
            out[i] = x[r]
    return out


def scatter_rows(x, rows, out) -> np.ndarray:
    """The inverse move: ``out[rows[i]] = x[i]`` (indices outside ``out`` are
    skipped); ``rows`` distinct.  Returns ``out``, written in place."""
    x = np.asarray(x)
    for i, r in enumerate(np.asarray(rows).tolist()):
        if 0 <= r < out.shape[0]:
            out[r] = x[i]
    return out
