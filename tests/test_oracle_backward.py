"""Pins of the backward oracle: central finite differences and softmax invariants."""

import numpy as np
import pytest

import math

from oracle import (attention_abs_dp, attention_backward, attention_backward_magnitudes,
                    attention_forward, bwd_delta, ring_forward)
from long_context_multimodal_amd.workloads import bf16_round


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


def _hand_case():
    """Two queries, two keys, d = 4 (default scale 1/2), worked by hand.

    Query 0 (position 0) sees key 0 only; query 1 (position 5) sees both keys.
    Scores: s_00 = 1; s_10 = 0, s_11 = ln 3, so query 1's weights are
    (1/4, 3/4) with LSE = ln 4, and query 0's weight is 1 with LSE = 1.
    """
    ln3 = math.log(3.0)
    q = np.array([[0, 2, 0, 0], [-1, 0, 0, 0]], float)[:, None, :]
    k = np.array([[0, 1, 0, 0], [-2 * ln3, 0, 0, 0]], float)[:, None, :]
    v = np.array([[1, 2, 0, 0], [-1, 2, 4, 0]], float)[:, None, :]
    do = np.array([[2, 1, 0, 3], [1, 1, -1, 2]], float)[:, None, :]
    qp, kp = np.array([0, 5]), np.array([0, 1])
    return q, k, v, do, qp, kp


def test_backward_and_magnitudes_hand_worked():
    # O_0 = v_0 = (1, 2, 0, 0); O_1 = v_0/4 + 3 v_1/4 = (-1/2, 2, 3, 0)
    # D_0 = dO_0.O_0 = 4; D_1 = dO_1.O_1 = -3/2
    # dP_00 = 4; dP_10 = 3, dP_11 = -3
    # dS_00 = 1 (4 - 4) = 0; dS_10 = (3 + 3/2)/4 = 9/8; dS_11 = 3 (-3 + 3/2)/4 = -9/8
    # sum|dO O|: row 0: 2 + 2 = 4; row 1: 1/2 + 2 + 3 = 11/2
    # C (sum_j P |dP|): row 0: 4; row 1: 3/4 + 9/4 = 3;  A = (8, 17/2)
    # W = |dS| + P A: W_00 = 8; W_10 = 9/8 + 17/8 = 13/4; W_11 = 9/8 + 51/8 = 15/2
    ln3 = math.log(3.0)
    q, k, v, do, qp, kp = _hand_case()
    o, lse = attention_forward(q, k, v, qp, kp)
    np.testing.assert_allclose(lse, [[1.0, math.log(4.0)]], rtol=1e-15)
    np.testing.assert_allclose(o[:, 0], [[1, 2, 0, 0], [-0.5, 2, 3, 0]], atol=1e-15)
    delta = bwd_delta(o, do)
    np.testing.assert_allclose(delta, [[4.0, -1.5]], atol=1e-15)
    dq, dk, dv = attention_backward(q, k, v, do, lse, delta, qp, kp)
    # dQ_i = (1/2) sum_j dS_ij k_j; dK_j = (1/2) sum_i dS_ij q_i; dV_j = sum_i P_ij dO_i
    np.testing.assert_allclose(dq[:, 0], [[0, 0, 0, 0], [9 * ln3 / 8, 9 / 16, 0, 0]], atol=1e-15)
    np.testing.assert_allclose(dk[:, 0], [[-9 / 16, 0, 0, 0], [9 / 16, 0, 0, 0]], atol=1e-15)
    np.testing.assert_allclose(dv[:, 0], [[9 / 4, 5 / 4, -1 / 4, 7 / 2], [3 / 4, 3 / 4, -3 / 4, 3 / 2]],
                               atol=1e-15)
    np.testing.assert_allclose(attention_abs_dp(q, k, v, do, lse, qp, kp), [[4.0, 3.0]],
                               atol=1e-15)
    mq, mk, mv = attention_backward_magnitudes(q, k, v, do, o, lse, qp, kp)
    # Mq_i = (1/2) sum_j W_ij |k_j|; Mk_j = (1/2) sum_i W_ij |q_i|; Mv_j = sum_i P_ij |dO_i|
    np.testing.assert_allclose(mq[:, 0], [[0, 4, 0, 0], [15 * ln3 / 2, 13 / 8, 0, 0]], atol=1e-14)
    np.testing.assert_allclose(mk[:, 0], [[13 / 8, 8, 0, 0], [15 / 4, 0, 0, 0]], atol=1e-14)
    np.testing.assert_allclose(mv[:, 0], [[9 / 4, 5 / 4, 1 / 4, 7 / 2], [3 / 4, 3 / 4, 3 / 4, 3 / 2]],
                               atol=1e-15)
    # an explicit all-chunk C equal to this chunk's changes nothing
    m2 = attention_backward_magnitudes(q, k, v, do, o, lse, qp, kp, dp_abs=[[4.0, 3.0]])
    for a, b in zip((mq, mk, mv), m2):
        np.testing.assert_allclose(a, b, rtol=1e-15)


def test_magnitudes_single_visible_key_closed_form(rng):
    # one visible key per query: P = 1, O = v, dS = dP - D = 0, so
    # Mq_i = scale (sum_c |dO_ic v_c| + |dO_i . v|) |k|, Mv = |dO|
    n, d = 6, 8
    q = rng.standard_normal((n, 1, d))
    k = rng.standard_normal((n, 1, d))
    v = rng.standard_normal((n, 1, d))
    do = rng.standard_normal((n, 1, d))
    qp = kp = np.arange(n) * 10
    qs = qp.copy()  # packed: each query's sample starts at its own position
    o, lse = attention_forward(q, k, v, qp, kp, q_start=qs)
    mq, mk, mv = attention_backward_magnitudes(q, k, v, do, o, lse, qp, kp, q_start=qs)
    a = np.abs(do[:, 0] * v[:, 0]).sum(axis=1) + np.abs((do[:, 0] * v[:, 0]).sum(axis=1))
    sc = 1 / np.sqrt(d)
    np.testing.assert_allclose(mq[:, 0], sc * a[:, None] * np.abs(k[:, 0]), rtol=1e-13)
    np.testing.assert_allclose(mk[:, 0], sc * a[:, None] * np.abs(q[:, 0]), rtol=1e-13)
    np.testing.assert_allclose(mv, np.abs(do), rtol=1e-15)


def _loop_magnitudes(q, ks, vs, do, qp, kps, chunk, scale, qs=None):
    """Pure-Python restatement, one scalar at a time: forward over all chunks
    (no max subtraction), then the sums of absolute terms for one chunk."""
    sq, hq, d = q.shape
    hkv = ks[0].shape[1]
    g = hq // hkv
    lo = [-(10 ** 18)] * sq if qs is None else [int(x) for x in qs]

    def visible(i, kpos):
        return lo[i] <= kpos <= qp[i]

    def dot(a, b):
        return sum(float(x) * float(y) for x, y in zip(a, b))

    mq = np.zeros(q.shape)
    mk = np.zeros(ks[chunk].shape)
    mv = np.zeros(ks[chunk].shape)
    for h in range(hq):
        kv = h // g
        for i in range(sq):
            terms = []  # (chunk, key, weight before normalisation)
            for c, (kc, kpc) in enumerate(zip(ks, kps)):
                for j in range(len(kpc)):
                    if visible(i, int(kpc[j])):
                        terms.append((c, j, math.exp(scale * dot(q[i, h], kc[j, kv]))))
            if not terms:
                continue
            z = sum(t[2] for t in terms)
            o = [sum(w / z * float(vs[c][j, kv, e]) for c, j, w in terms) for e in range(d)]
            delta = dot(do[i, h], o)
            a = sum(abs(float(do[i, h, e]) * o[e]) for e in range(d))
            a += sum(w / z * abs(dot(do[i, h], vs[c][j, kv])) for c, j, w in terms)
            for c, j, w in terms:
                if c != chunk:
                    continue
                p = w / z
                ds = p * (dot(do[i, h], vs[c][j, kv]) - delta)
                wt = abs(ds) + p * a
                for e in range(d):
                    mq[i, h, e] += scale * wt * abs(float(ks[c][j, kv, e]))
                    mk[j, kv, e] += scale * wt * abs(float(q[i, h, e]))
                    mv[j, kv, e] += p * abs(float(do[i, h, e]))
    return mq, mk, mv


@pytest.mark.parametrize("packed", [False, True])
def test_magnitudes_match_scalar_loops(rng, packed):
    # two chunks of interleaved positions, GQA 4/2, a query that sees nothing
    # in chunk 1 and one that sees nothing at all
    sq, hq, hkv, d = 10, 4, 2, 3
    qp = np.array([-3, 0, 2, 3, 5, 8, 11, 14, 17, 23])
    kps = [np.array([0, 1, 4, 6, 9, 13]), np.array([15, 16, 18, 22])]
    qs = np.array([-3, 0, 0, 0, 4, 4, 4, 12, 12, 12]) if packed else None
    q = rng.standard_normal((sq, hq, d))
    ks = [rng.standard_normal((len(kp), hkv, d)) for kp in kps]
    vs = [rng.standard_normal((len(kp), hkv, d)) for kp in kps]
    do = rng.standard_normal((sq, hq, d))
    scale = 0.7
    o, lse = ring_forward(q, ks, vs, qp, kps, scale=scale, q_start=qs)
    c_all = sum(attention_abs_dp(q, k, v, do, lse, qp, kp, scale=scale, q_start=qs)
                for k, v, kp in zip(ks, vs, kps))
    for c in range(2):
        want = _loop_magnitudes(q, ks, vs, do, qp, kps, c, scale, qs)
        got = attention_backward_magnitudes(q, ks[c], vs[c], do, o, lse, qp, kps[c], scale=scale,
                                            q_start=qs, dp_abs=c_all)
        for name, a, b in zip(("Mq", "Mk", "Mv"), got, want):
            np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14, err_msg=name)


def _bf16(x):
    return bf16_round(np.asarray(x, dtype=np.float32))[1].astype(np.float64)


def test_magnitudes_bound_a_rounded_backward(rng):
    """The purpose of the sums: a backward that rounds its weights, its dS and
    its output to bf16 (8 significant bits: unit roundoff u = 2^-8) -- the forward's weights
    before P V, O itself before D = dO . O, and P and dS before the gradient
    contractions -- stays within u times them, element by element, up to
    second-order terms.  Two chunks, GQA, exponents spread by scale 0.9."""
    u = 2.0 ** -8
    sq, hq, hkv, d = 24, 4, 2, 16
    qp = np.arange(sq) * 3 + 2
    kps = [np.arange(0, 36), np.arange(36, 72)]
    q = rng.standard_normal((sq, hq, d))
    ks = [rng.standard_normal((len(kp), hkv, d)) for kp in kps]
    vs = [rng.standard_normal((len(kp), hkv, d)) for kp in kps]
    do = rng.standard_normal((sq, hq, d))
    scale = 0.9
    o, lse = ring_forward(q, ks, vs, qp, kps, scale=scale)
    c_all = sum(attention_abs_dp(q, k, v, do, lse, qp, kp, scale=scale)
                for k, v, kp in zip(ks, vs, kps))
    g = hq // hkv

    def probs(k, kp, h):
        s = (q[:, h] @ k[:, h // g].T) * scale
        vis = kp[None, :] <= qp[:, None]
        return np.where(vis, np.exp(s - lse[h][:, None]), 0.0)

    # forward with rounded weights, then O rounded, then D from it
    o_r = np.zeros_like(o)
    for k, v, kp in zip(ks, vs, kps):
        for h in range(hq):
            o_r[:, h] += _bf16(probs(k, kp, h)) @ v[:, h // g]
    delta_r = bwd_delta(_bf16(o_r), do)
    delta = bwd_delta(o, do)
    worst = 0.0
    dq_r, dq, mq_tot = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    for k, v, kp in zip(ks, vs, kps):
        dk_r, dv_r = np.zeros_like(k), np.zeros_like(v)
        for h in range(hq):
            p = probs(k, kp, h)
            dp = do[:, h] @ v[:, h // g].T
            ds_r = _bf16(p * (dp - delta_r[h][:, None]))
            dq_r[:, h] += scale * ds_r @ k[:, h // g]
            dk_r[:, h // g] += scale * ds_r.T @ q[:, h]
            dv_r[:, h // g] += _bf16(p).T @ do[:, h]
        dq_c, dk, dv = attention_backward(q, k, v, do, lse, delta, qp, kp, scale=scale)
        mq, mk, mv = attention_backward_magnitudes(q, k, v, do, o, lse, qp, kp, scale=scale,
                                                   dp_abs=c_all)
        dq += dq_c
        mq_tot += mq
        for got, want, m in ((dk_r, dk, mk), (dv_r, dv, mv)):
            assert np.all(np.abs(got - want) <= u * m * (1 + 4 * u) + 1e-14)
            worst = max(worst, float((np.abs(got - want) / (u * m + 1e-300)).max()))
    assert np.all(np.abs(dq_r - dq) <= u * mq_tot * (1 + 4 * u) + 1e-14)
    # the sums are not vacuous either: the rounded backward uses a good part of them
    assert worst > 0.05


def test_magnitudes_bound_the_gradients(rng):
    # triangle inequality: every gradient element is at most its sum of |terms|;
    # with dO >= 0 the bound is attained for dV
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
