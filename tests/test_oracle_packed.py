"""Pins of the oracle's packed-sample path: the per-sample zigzag permutation and
attention / gradients with a per-query sample start (``q_start``).

What fixes them (none of it is the oracle's own code re-run):
* a hand-worked permutation example and the closed-form causal work per
  sample and rank;
* a pure-Python brute force that applies the definition with explicit sample
  ids ("same sample and k_pos <= q_pos"), not the q_start bound;
* block-diagonal decomposition: packed attention over a stream equals plain
  causal attention run on each sample alone;
* central finite differences of the packed forward.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import (attention_backward, attention_forward, bwd_delta, ring_forward,
                    visible_pairs, zigzag_packed_perm, zigzag_perm)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "packed_zigzag_example.json")


def test_packed_zigzag_worked_example():
    gold = json.load(open(GOLDEN))
    perm, first = zigzag_packed_perm(gold["starts"], gold["n_ranks"])
    assert perm.tolist() == gold["perm"]
    assert first.tolist() == gold["token_start"]


@pytest.mark.parametrize("lens,p", [([16], 2), ([8, 24, 40], 4), ([6, 6, 12, 30], 3),
                                    ([64, 128, 256, 512], 8)])
def test_packed_zigzag_invariants(lens, p):
    starts = np.concatenate([[0], np.cumsum(lens)])
    n = int(starts[-1])
    perm, first = zigzag_packed_perm(starts, p)
    assert sorted(perm.tolist()) == list(range(n))  # bijection
    per = perm.reshape(p, -1)
    assert np.all(np.diff(per, axis=1) > 0)  # ascending within each rank
    sample = np.searchsorted(starts, perm, side="right") - 1
    assert np.array_equal(first, starts[sample])
    for s, ln in enumerate(lens):
        L = ln // (2 * p)
        for r in range(p):
            mine = per[r][sample.reshape(p, -1)[r] == s]
            assert mine.size == 2 * L
            # causal work inside the sample: keys from its start up to the query
            work = int((mine - starts[s] + 1).sum())
            assert work == L * L * (2 * p - 1) + L * (L + 1)


def test_packed_zigzag_single_sample_is_zigzag():
    perm, first = zigzag_packed_perm([0, 96], 6)
    assert np.array_equal(perm, zigzag_perm(96, 6))
    assert not first.any()


def test_packed_zigzag_rejects_bad_lengths():
    with pytest.raises(ValueError):
        zigzag_packed_perm([0, 10, 20], 2)  # 10 is not a multiple of 4
    with pytest.raises(ValueError):
        zigzag_packed_perm([0, 8, 8], 2)  # empty sample


def _packed_case(rng, lens, p, rank, hq, hkv, d):
    starts = np.concatenate([[0], np.cumsum(lens)])
    perm, first = zigzag_packed_perm(starts, p)
    shard = perm.size // p
    qp = perm[rank * shard:(rank + 1) * shard]
    qs = first[rank * shard:(rank + 1) * shard]
    kps = [perm[c * shard:(c + 1) * shard] for c in range(p)]
    q = rng.standard_normal((shard, hq, d))
    ks = [rng.standard_normal((shard, hkv, d)) for _ in range(p)]
    vs = [rng.standard_normal((shard, hkv, d)) for _ in range(p)]
    return starts, qp, qs, kps, q, ks, vs


def test_packed_attention_brute_force(rng):
    """Definition with explicit sample ids, pure Python, on a tiny case."""
    lens, p, hq, hkv, d = [8, 16, 8], 2, 2, 1, 3
    starts, qp, qs, kps, q, ks, vs = _packed_case(rng, lens, p, 1, hq, hkv, d)
    sid = lambda pos: int(np.searchsorted(starts, pos, side="right") - 1)
    o, lse = ring_forward(q, ks, vs, qp, kps, q_start=qs)
    keys = [(int(kp), c, j) for c in range(p) for j, kp in enumerate(kps[c])]
    for i in range(len(qp)):
        for h in range(hq):
            num = [0.0] * d
            den = 0.0
            for kpos, c, j in keys:
                if sid(kpos) != sid(qp[i]) or kpos > qp[i]:
                    continue
                w = math.exp(sum(q[i, h, t] * ks[c][j, 0, t] for t in range(d)) / math.sqrt(d))
                den += w
                for t in range(d):
                    num[t] += w * vs[c][j, 0, t]
            assert abs(lse[h, i] - math.log(den)) < 1e-12
            for t in range(d):
                assert abs(o[i, h, t] - num[t] / den) < 1e-12


def test_packed_attention_is_block_diagonal(rng):
    """Packed attention over a stream equals plain causal attention per sample."""
    lens, hq, hkv, d = [40, 24, 64], 4, 2, 8
    starts = np.concatenate([[0], np.cumsum(lens)])
    n = int(starts[-1])
    pos = np.arange(n)
    first = starts[np.searchsorted(starts, pos, side="right") - 1]
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((n, hkv, d))
    v = rng.standard_normal((n, hkv, d))
    o, lse = attention_forward(q, k, v, pos, pos, q_start=first)
    for a, b in zip(starts, starts[1:]):
        o_s, l_s = attention_forward(q[a:b], k[a:b], v[a:b], pos[a:b] - a, pos[a:b] - a)
        np.testing.assert_allclose(o[a:b], o_s, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, a:b], l_s, rtol=0, atol=1e-13)
    # the gradients decompose the same way
    do = rng.standard_normal((n, hq, d))
    delta = bwd_delta(o, do)
    dq, dk, dv = attention_backward(q, k, v, do, lse, delta, pos, pos, q_start=first)
    for a, b in zip(starts, starts[1:]):
        o_s, l_s = attention_forward(q[a:b], k[a:b], v[a:b], pos[a:b], pos[a:b])
        g = attention_backward(q[a:b], k[a:b], v[a:b], do[a:b], l_s, bwd_delta(o_s, do[a:b]),
                               pos[a:b], pos[a:b])
        for got, want in zip((dq[a:b], dk[a:b], dv[a:b]), g):
            np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_packed_gradients_finite_differences(rng):
    lens, p, hq, hkv, d, h = [8, 16], 2, 2, 1, 4, 1e-6
    _, qp, qs, kps, q, ks, vs = _packed_case(rng, lens, p, 0, hq, hkv, d)
    do = rng.standard_normal(q.shape)

    def loss():
        o, _ = ring_forward(q, ks, vs, qp, kps, q_start=qs)
        return float((o * do).sum())

    o, lse = ring_forward(q, ks, vs, qp, kps, q_start=qs)
    delta = bwd_delta(o, do)
    grads = [attention_backward(q, ks[c], vs[c], do, lse, delta, qp, kps[c], q_start=qs)
             for c in range(p)]
    dq = sum(g[0] for g in grads)

    def fd(arr, idx):
        old = arr[idx]
        arr[idx] = old + h
        lp = loss()
        arr[idx] = old - h
        lm = loss()
        arr[idx] = old
        return (lp - lm) / (2 * h)

    for idx in [(0, 0, 0), (5, 1, 3), (11, 0, 2)]:
        assert abs(fd(q, idx) - dq[idx]) <= 1e-6 * max(1.0, abs(dq[idx]))
    for c in range(p):
        for idx in [(0, 0, 1), (7, 0, 2), (11, 0, 0)]:
            assert abs(fd(ks[c], idx) - grads[c][1][idx]) <= 1e-6 * max(1.0, abs(grads[c][1][idx]))
            assert abs(fd(vs[c], idx) - grads[c][2][idx]) <= 1e-6 * max(1.0, abs(grads[c][2][idx]))


def test_visible_pairs_with_sample_start(rng):
    qp = np.sort(rng.choice(200, 50, replace=False))
    kp = np.sort(rng.choice(200, 70, replace=False))
    qs = np.minimum(qp, (qp // 40) * 40)
    brute = sum(int(((kp >= s) & (kp <= p)).sum()) for p, s in zip(qp, qs))
    assert visible_pairs(qp, kp, qs) == brute
    assert visible_pairs(qp, kp) == sum(int((kp <= p).sum()) for p in qp)
