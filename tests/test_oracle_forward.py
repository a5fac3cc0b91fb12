"""Pins of the forward oracle against closed forms, brute force and invariants.

Each test fixes something the definition of causal softmax attention decides
on its own (no value here comes from the HIP library).
"""

import math

import numpy as np
import pytest

from oracle import attention_forward, visible_pairs, zigzag_perm


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_single_visible_key_returns_v_exactly(rng):
    # one query at position 5, keys at 5, 6, 7: only the first is visible
    q = _rand(rng, 1, 2, 8)
    k = _rand(rng, 3, 2, 8)
    v = _rand(rng, 3, 2, 8)
    o, lse = attention_forward(q, k, v, [5], [5, 6, 7])
    assert np.array_equal(o[0], v[0])
    s = (q[0] * k[0]).sum(-1) / math.sqrt(8)
    np.testing.assert_allclose(lse[:, 0], s, rtol=0, atol=1e-15)


def test_query_at_position_zero_sees_only_the_diagonal(rng):
    n = 40
    q = _rand(rng, n, 3, 16)
    k = _rand(rng, n, 3, 16)
    v = _rand(rng, n, 3, 16)
    o, _ = attention_forward(q, k, v, np.arange(n), np.arange(n))
    assert np.array_equal(o[0], v[0])


def test_identical_keys_give_mean_of_visible_values(rng):
    n, d = 50, 8
    q = _rand(rng, n, 2, d)
    k = np.broadcast_to(_rand(rng, 1, 2, d), (n, 2, d)).copy()
    v = _rand(rng, n, 2, d)
    o, lse = attention_forward(q, k, v, np.arange(n), np.arange(n))
    for i in range(n):
        np.testing.assert_allclose(o[i], v[: i + 1].mean(axis=0), rtol=1e-12, atol=1e-13)
        s = (q[i] * k[0]).sum(-1) / math.sqrt(d)
        np.testing.assert_allclose(lse[:, i], s + math.log(i + 1), rtol=1e-12, atol=1e-12)


def test_zero_query_gives_uniform_weights(rng):
    n = 33
    q = np.zeros((n, 1, 4))
    k = _rand(rng, n, 1, 4)
    v = _rand(rng, n, 1, 4)
    qp = np.arange(n) * 3
    kp = np.arange(n) * 3 + 1  # query i sees keys j < i
    o, lse = attention_forward(q, k, v, qp, kp)
    assert np.isneginf(lse[0, 0]) and np.all(o[0] == 0)
    for i in range(1, n):
        np.testing.assert_allclose(lse[0, i], math.log(i), rtol=1e-13)
        np.testing.assert_allclose(o[i, 0], v[:i, 0].mean(axis=0), rtol=1e-12, atol=1e-13)


def test_fully_masked_rows_are_zero_with_minus_inf_lse(rng):
    q = _rand(rng, 4, 2, 8)
    k = _rand(rng, 6, 2, 8)
    v = _rand(rng, 6, 2, 8)
    o, lse = attention_forward(q, k, v, [0, 1, 2, 3], [10, 11, 12, 13, 14, 15])
    assert np.all(o == 0)
    assert np.all(np.isneginf(lse))


def _brute(q, k, v, qp, kp, scale):
    """Pure-Python loops, direct exp of the raw scores (no max subtraction)."""
    sq, hq, d = len(q), len(q[0]), len(q[0][0])
    sk, hkv = len(k), len(k[0])
    g = hq // hkv
    o = [[[0.0] * d for _ in range(hq)] for _ in range(sq)]
    lse = [[-math.inf] * sq for _ in range(hq)]
    for h in range(hq):
        kv = h // g
        for i in range(sq):
            ws = []
            for j in range(sk):
                if kp[j] <= qp[i]:
                    dot = 0.0
                    for c in range(d):
                        dot += q[i][h][c] * k[j][kv][c]
                    ws.append((j, math.exp(dot * scale)))
            z = sum(w for _, w in ws)
            if z > 0:
                lse[h][i] = math.log(z)
                for c in range(d):
                    o[i][h][c] = sum(w * v[j][kv][c] for j, w in ws) / z
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("sq,sk,hq,hkv,d", [(17, 23, 2, 2, 5), (64, 64, 4, 2, 8), (31, 9, 3, 1, 4)])
def test_brute_force_small(rng, sq, sk, hq, hkv, d):
    q = _rand(rng, sq, hq, d)
    k = _rand(rng, sk, hkv, d)
    v = _rand(rng, sk, hkv, d)
    # interleaved, strictly increasing positions with gaps on both sides
    allpos = np.sort(rng.choice(4 * (sq + sk), size=sq + sk, replace=False))
    sel = np.zeros(sq + sk, bool)
    sel[rng.choice(sq + sk, size=sq, replace=False)] = True
    qp, kp = allpos[sel], allpos[~sel]
    scale = 0.37
    o, lse = attention_forward(q, k, v, qp, kp, scale=scale)
    ob, lb = _brute(q.tolist(), k.tolist(), v.tolist(), qp.tolist(), kp.tolist(), scale)
    np.testing.assert_allclose(o, ob, rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=1e-12, atol=1e-12)


def test_default_scale_is_inverse_sqrt_head_dim(rng):
    q = _rand(rng, 5, 1, 9)
    k = _rand(rng, 5, 1, 9)
    v = _rand(rng, 5, 1, 9)
    a = attention_forward(q, k, v, np.arange(5), np.arange(5))
    b = attention_forward(q, k, v, np.arange(5), np.arange(5), scale=1 / 3.0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_gqa_equals_mha_with_repeated_kv_heads(rng):
    sq, hq, hkv, d = 40, 6, 2, 8
    q = _rand(rng, sq, hq, d)
    k = _rand(rng, sq, hkv, d)
    v = _rand(rng, sq, hkv, d)
    pos = np.arange(sq)
    o, lse = attention_forward(q, k, v, pos, pos)
    # heads 0,1,2 -> kv 0; heads 3,4,5 -> kv 1
    k_rep = np.repeat(k, hq // hkv, axis=1)
    v_rep = np.repeat(v, hq // hkv, axis=1)
    o2, lse2 = attention_forward(q, k_rep, v_rep, pos, pos)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    # and the mapping is contiguous: head 2 uses kv head 0, not kv head 1
    o_h2, _ = attention_forward(q[:, 2:3], k[:, 0:1], v[:, 0:1], pos, pos)
    np.testing.assert_array_equal(o[:, 2:3], o_h2)


def test_shard_rows_equal_unsharded_rows(rng):
    n, p, h, d = 96, 3, 2, 8
    x_q = _rand(rng, n, h, d)
    x_k = _rand(rng, n, h, d)
    x_v = _rand(rng, n, h, d)
    pos = np.arange(n)
    o_full, l_full = attention_forward(x_q, x_k, x_v, pos, pos)
    perm = zigzag_perm(n, p)
    shard = n // p
    for r in range(p):
        rows = perm[r * shard:(r + 1) * shard]
        o_r, l_r = attention_forward(x_q[rows], x_k, x_v, rows, pos)
        np.testing.assert_allclose(o_r, o_full[rows], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(l_r, l_full[:, rows], rtol=1e-13, atol=1e-14)


def test_row_subset_matches_full(rng):
    q = _rand(rng, 300, 2, 8)
    k = _rand(rng, 300, 2, 8)
    v = _rand(rng, 300, 2, 8)
    pos = np.arange(300)
    o, lse = attention_forward(q, k, v, pos, pos)
    rows = np.array([299, 0, 257, 256, 5])
    o2, l2 = attention_forward(q, k, v, pos, pos, rows=rows)
    np.testing.assert_allclose(o2, o[rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l2, lse[:, rows], rtol=1e-13, atol=1e-14)


def test_visible_pairs_brute_force(rng):
    qp = np.sort(rng.choice(500, 60, replace=False))
    kp = np.sort(rng.choice(500, 70, replace=False))
    brute = sum(1 for a in qp for b in kp if b <= a)
    assert visible_pairs(qp, kp) == brute


def test_visible_pairs_zigzag_rank0_closed_form():
    # rank 0 of zigzag P=8 over N=65536: own chunk = two triangles + one full
    # block of the half length L; every other chunk is the second Q half
    # against the whole chunk.
    n, p = 65536, 8
    L = n // (2 * p)
    perm = zigzag_perm(n, p)
    qp = perm[:2 * L]
    own = visible_pairs(qp, qp)
    assert own == 2 * (L * (L + 1) // 2) + L * L
    for s in range(1, p):
        kp = perm[s * 2 * L:(s + 1) * 2 * L]
        assert visible_pairs(qp, kp) == L * 2 * L
