"""Pins of the chunk merge: split-then-merge equals unsplit, and its algebra."""

import math

import numpy as np
import pytest

from oracle import attention_forward, lse_merge, ring_forward


def _case(rng, n=120, h=3, d=8):
    q = rng.standard_normal((n, h, d))
    k = rng.standard_normal((n, h, d))
    v = rng.standard_normal((n, h, d))
    return q, k, v, np.arange(n)


@pytest.mark.parametrize("cut", [1, 17, 60, 119])
def test_split_then_merge_equals_unsplit(rng, cut):
    q, k, v, pos = _case(rng)
    o_full, l_full = attention_forward(q, k, v, pos, pos)
    o_a, l_a = attention_forward(q, k[:cut], v[:cut], pos, pos[:cut])
    o_b, l_b = attention_forward(q, k[cut:], v[cut:], pos, pos[cut:])
    o, lse = lse_merge(o_a, l_a, o_b, l_b)
    np.testing.assert_allclose(o, o_full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, l_full, rtol=1e-13, atol=1e-13)


def test_many_chunks_any_order(rng):
    q, k, v, pos = _case(rng, n=128)
    o_full, l_full = attention_forward(q, k, v, pos, pos)
    ks = [k[i:i + 32] for i in range(0, 128, 32)]
    vs = [v[i:i + 32] for i in range(0, 128, 32)]
    ps = [pos[i:i + 32] for i in range(0, 128, 32)]
    for order in ([0, 1, 2, 3], [0, 3, 2, 1], [2, 0, 3, 1]):
        o, lse = ring_forward(q, ks, vs, pos, ps, order=order)
        np.testing.assert_allclose(o, o_full, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, l_full, rtol=1e-13, atol=1e-13)


def test_merge_commutative_and_associative(rng):
    sh = (10, 2, 4)
    parts = []
    for _ in range(3):
        parts.append((rng.standard_normal(sh), rng.standard_normal((2, 10)) * 3))
    ab = lse_merge(*parts[0], *parts[1])
    ba = lse_merge(*parts[1], *parts[0])
    np.testing.assert_allclose(ab[0], ba[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ab[1], ba[1], rtol=1e-12, atol=1e-12)
    left = lse_merge(*ab, *parts[2])
    bc = lse_merge(*parts[1], *parts[2])
    right = lse_merge(*parts[0], *bc)
    np.testing.assert_allclose(left[0], right[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(left[1], right[1], rtol=1e-12, atol=1e-12)


def test_minus_inf_is_identity_and_two_empties_stay_empty(rng):
    o = rng.standard_normal((5, 2, 4))
    l = rng.standard_normal((2, 5))
    z = np.zeros_like(o)
    ninf = np.full_like(l, -np.inf)
    m = lse_merge(o, l, z, ninf)
    np.testing.assert_array_equal(m[0], o)
    np.testing.assert_array_equal(m[1], l)
    m2 = lse_merge(z, ninf, z, ninf)
    assert not np.isnan(m2[0]).any()
    assert np.all(m2[0] == 0) and np.all(np.isneginf(m2[1]))


def test_chunk_merged_twice_raises_lse_by_ln2(rng):
    # failure analogue: a ring step replayed twice is detectable from LSE
    q, k, v, pos = _case(rng, n=64)
    o_a, l_a = attention_forward(q, k[:32], v[:32], pos, pos[:32])
    o_b, l_b = attention_forward(q, k[32:], v[32:], pos, pos[32:])
    good = lse_merge(o_a, l_a, o_b, l_b)
    twice = lse_merge(*good, o_b, l_b)
    only_a = pos < 32  # rows that see nothing of chunk b
    np.testing.assert_allclose(twice[1][:, only_a], good[1][:, only_a], rtol=0, atol=0)
    rows_b = pos >= 32
    assert np.all(twice[1][:, rows_b] > good[1][:, rows_b])
    # a chunk merged with itself: exactly +ln 2 where it is the only contributor
    self2 = lse_merge(o_a, l_a, o_a, l_a)
    fin = np.isfinite(l_a)
    np.testing.assert_allclose(self2[1][fin], l_a[fin] + math.log(2), rtol=1e-14)
    np.testing.assert_allclose(self2[0], o_a, rtol=1e-14, atol=1e-15)
