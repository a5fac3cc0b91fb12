"""Pins of the backward oracle: central finite differences and softmax invariants."""

import numpy as np
import pytest

from oracle import (attention_backward, attention_backward_magnitudes, attention_forward,
                    bwd_delta, ring_forward)


def _loss(q, ks, vs, qp, kps, do):
    o, _ = ring_forward(q, ks, vs, qp, kps)
    return float((o * do).sum())


def _chunked_grads(q, ks, vs, qp, kps, do):
    o, lse = ring_forward(q, ks, vs, qp, kps)
    delta = bwd_delta(o, do)
    dq = np.zeros_like(q)
    dks, dvs = [], []
    for k, v, kp in zip(ks, vs, kps):
        a, b, c = attention_backward(q, k, v, do, lse, delta, qp, kp)
        dq += a
        dks.append(b)
        dvs.append(c)
    return dq, dks, dvs


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2)])
def test_central_finite_differences(rng, hq, hkv):
    sq, d, h = 12, 6, 1e-6
    # two chunks with interleaved positions; one query sees nothing in chunk 1
    qp = np.array([0, 2, 3, 5, 8, 9, 11, 14, 15, 17, 20, 23])
    kps = [np.array([0, 1, 4, 6, 9, 10, 13]), np.array([15, 16, 18, 21, 22])]
    q = rng.standard_normal((sq, hq, d))
    ks = [rng.standard_normal((len(kp), hkv, d)) for kp in kps]
    vs = [rng.standard_normal((len(kp), hkv, d)) for kp in kps]
    do = rng.standard_normal((sq, hq, d))
    dq, dks, dvs = _chunked_grads(q, ks, vs, qp, kps, do)

    def fd(arr, idx):
        old = arr[idx]
        arr[idx] = old + h
        lp = _loss(q, ks, vs, qp, kps, do)
        arr[idx] = old - h
        lm = _loss(q, ks, vs, qp, kps, do)
        arr[idx] = old
        return (lp - lm) / (2 * h)

    checks = []
    for idx in [(0, 0, 0), (3, hq - 1, 2), (11, 1, 5), (7, 0, 3)]:
        checks.append((fd(q, idx), dq[idx]))
    for c in range(2):
        for idx in [(0, 0, 0), (len(kps[c]) - 1, hkv - 1, 4), (2, hkv - 1, 1)]:
            checks.append((fd(ks[c], idx), dks[c][idx]))
            checks.append((fd(vs[c], idx), dvs[c][idx]))
    for num, ana in checks:
        assert abs(num - ana) <= 1e-6 * max(1.0, abs(ana)), (num, ana)


def test_gradient_invariants(rng):
    n, hq, hkv, d = 80, 4, 2, 8
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((n, hkv, d))
    v = rng.standard_normal((n, hkv, d))
    do = rng.standard_normal((n, hq, d))
    qp = np.arange(n) + 5  # every query sees at least six keys
    kp = np.arange(n)
    o, lse = attention_forward(q, k, v, qp, kp)
    delta = bwd_delta(o, do)
    dq, dk, dv = attention_backward(q, k, v, do, lse, delta, qp, kp)
    # softmax is invariant to a common shift of all keys -> sum_j dK_j = 0
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-11)
    # rows sum to one -> sum_j dV_j = sum over the KV head's query heads of dO
    g = hq // hkv
    for kv in range(hkv):
        want = do[:, kv * g:(kv + 1) * g, :].sum(axis=(0, 1))
        np.testing.assert_allclose(dv[:, kv, :].sum(axis=0), want, rtol=1e-11, atol=1e-11)


def test_identical_keys_give_zero_dq(rng):
    # sum_j dS_ij = 0 for every row; with all keys equal dQ_i = scale*k*sum_j dS_ij
    n, d = 30, 8
    q = rng.standard_normal((n, 2, d))
    k = np.broadcast_to(rng.standard_normal((1, 2, d)), (n, 2, d)).copy()
    v = rng.standard_normal((n, 2, d))
    do = rng.standard_normal((n, 2, d))
    pos = np.arange(n)
    o, lse = attention_forward(q, k, v, pos, pos)
    dq, _, _ = attention_backward(q, k, v, do, lse, bwd_delta(o, do), pos, pos)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)


def test_empty_rows_have_zero_gradient(rng):
    q = rng.standard_normal((4, 1, 4))
    k = rng.standard_normal((3, 1, 4))
    v = rng.standard_normal((3, 1, 4))
    do = rng.standard_normal((4, 1, 4))
    qp = np.array([0, 1, 2, 9])
    kp = np.array([5, 6, 7])
    o, lse = attention_forward(q, k, v, qp, kp)
    dq, dk, dv = attention_backward(q, k, v, do, lse, bwd_delta(o, do), qp, kp)
    assert np.all(dq[:3] == 0)
    np.testing.assert_allclose(dv.sum(axis=0), do[3], rtol=1e-12)


def test_magnitudes_bound_the_gradients(rng):
    # triangle inequality: every gradient element is at most its sum of |terms|;
    # with all-positive inputs and dO chosen so dS >= 0 the bound is tight for dV
    n, hq, hkv, d = 40, 4, 2, 8
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((n, hkv, d))
    v = rng.standard_normal((n, hkv, d))
    do = rng.standard_normal((n, hq, d))
    pos = np.arange(n)
    o, lse = attention_forward(q, k, v, pos, pos)
    dq, dk, dv = attention_backward(q, k, v, do, lse, bwd_delta(o, do), pos, pos)
    mq, mk, mv = attention_backward_magnitudes(q, k, v, do, o, lse, pos, pos)
    assert np.all(np.abs(dq) <= mq + 1e-12)
    assert np.all(np.abs(dk) <= mk + 1e-12)
    assert np.all(np.abs(dv) <= mv + 1e-12)
    do_pos = np.abs(do)
    _, _, dv2 = attention_backward(q, k, v, do_pos, lse, bwd_delta(o, do_pos), pos, pos)
    _, _, mv2 = attention_backward_magnitudes(q, k, v, do_pos, o, lse, pos, pos)
    np.testing.assert_allclose(dv2, mv2, rtol=1e-12, atol=1e-12)
