"""GPU parity of the backward preprocess and the backward chunk kernels against
the float64 oracle: absolute bounds, RMS-relative mean error, and the
elementwise bf16 rounding bound (the bf16 unit roundoff u = 2^-8 times each
element's sum of absolute terms, from the oracle, plus 1/8 for second-order
and fp32 terms)."""

import numpy as np
import pytest

import oracle
from long_context_multimodal_amd.workloads import TINY, normal_bf16
from tests.helpers import (assert_close_abs, assert_close_rms, oracle_ring_grads, to_dev_bf16,
                           to_dev_i32, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mm():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from long_context_multimodal_amd import mmsp, ring
    mmsp.lib()
    return mmsp, ring


def _dev_f32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


@pytest.mark.parametrize("d", [64, 128])
def test_preprocess_matches_definition(mm, d):
    mmsp, _ = mm
    sq, hq = 333, 5
    ob, ov = normal_bf16(31, (sq, hq, d))
    gb, gv = normal_bf16(32, (sq, hq, d))
    import torch
    dq = torch.full((sq, hq, d), 7.0, dtype=torch.float32, device="cuda")
    delta = mmsp.attn_bwd_preprocess(to_dev_bf16(ob), to_dev_bf16(gb), dq_zero=dq)
    want = oracle.bwd_delta(ov, gv)
    np.testing.assert_allclose(to_np(delta), want, rtol=1e-5, atol=1e-5)
    assert np.all(to_np(dq) == 0)


def _interleaved(rng, sq, sk):
    allpos = np.sort(rng.choice(3 * (sq + sk), size=sq + sk, replace=False))
    sel = np.zeros(sq + sk, bool)
    sel[rng.choice(sq + sk, size=sq, replace=False)] = True
    return allpos[sel].astype(np.int32), allpos[~sel].astype(np.int32)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (7, 1)])
def test_bwd_chunk_kernel_ragged(mm, d, hq, hkv):
    """Kernel alone: LSE and delta come from the oracle (float64 -> fp32)."""
    mmsp, _ = mm
    sq, sk = 300, 333
    rng = np.random.default_rng(40 + d + hq)
    qp, kp = _interleaved(rng, sq, sk)
    qb, qv = normal_bf16(41, (sq, hq, d))
    kb, kv = normal_bf16(42, (sk, hkv, d))
    vb, vv = normal_bf16(43, (sk, hkv, d))
    gb, gv = normal_bf16(44, (sq, hq, d))
    o, lse = oracle.attention_forward(qv, kv, vv, qp, kp)
    delta = oracle.bwd_delta(o, gv)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(qv, kv, vv, gv, lse, delta, qp, kp)
    import torch
    dq = torch.zeros((sq, hq, d), dtype=torch.float32, device="cuda")
    dk, dv = mmsp.attn_bwd_chunk(to_dev_bf16(qb), to_dev_bf16(kb), to_dev_bf16(vb),
                                 to_dev_bf16(gb), _dev_f32(lse), _dev_f32(delta),
                                 to_dev_i32(qp), to_dev_i32(kp), dq)
    mq, mk, mv = oracle.attention_backward_magnitudes(qv, kv, vv, gv, o, lse, qp, kp)
    assert_close_rms(to_np(dq), dq_ref, bound=mq, what="dQ")
    assert_close_rms(to_np(dk), dk_ref, bound=mk, what="dK")
    assert_close_rms(to_np(dv), dv_ref, bound=mv, what="dV")
    # empty query rows get exactly zero gradient
    empty = np.isneginf(lse[0])
    assert np.all(to_np(dq)[empty] == 0)


@pytest.mark.parametrize("packed", [False, True])
def test_bwd_peaked_softmax_from_gpu_forward(mm, packed):
    """Logits about 5.7 times the 1/sqrt(d) scale (scale 0.5 at d = 128), so most
    rows put nearly all their weight on a few keys: the forward's running max is
    raised many times and P spans the full fp32 range in the backward.  The
    GPU forward's LSE and bf16 output feed the GPU backward, as in training;
    the expected values are the oracle's alone."""
    mmsp, _ = mm
    import torch
    sq, sk, hq, hkv, d, scale = 257, 300, 4, 2, 128, 0.5
    rng = np.random.default_rng(61 + packed)
    qp, kp = _interleaved(rng, sq, sk)
    qs = None
    if packed:  # three samples: every query's start is the largest cut at or below it
        cuts = np.array([0, int(qp[sq // 3]), int(qp[2 * sq // 3])])
        qs = cuts[np.searchsorted(cuts, qp, side="right") - 1].astype(np.int32)
    qb, qv = normal_bf16(62, (sq, hq, d))
    kb, kv = normal_bf16(63, (sk, hkv, d))
    vb, vv = normal_bf16(64, (sk, hkv, d))
    gb, gv = normal_bf16(65, (sq, hq, d))
    qd, kd, vd, gd = (to_dev_bf16(x) for x in (qb, kb, vb, gb))
    qs_d = to_dev_i32(qs) if packed else None
    o, lse = mmsp.attn_fwd_chunk(qd, kd, vd, to_dev_i32(qp), to_dev_i32(kp), scale=scale,
                                 q_start=qs_d)
    o_ref, lse_ref = oracle.attention_forward(qv, kv, vv, qp, kp, scale=scale, q_start=qs)
    assert_close_abs(to_np(o), o_ref, what="O")
    finite = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(to_np(lse)), finite)
    assert np.abs(to_np(lse)[finite] - lse_ref[finite]).max() <= 2e-2
    o16 = o.to(torch.bfloat16)
    delta = mmsp.attn_bwd_preprocess(o16, gd)
    dq = torch.zeros((sq, hq, d), dtype=torch.float32, device="cuda")
    dk, dv = mmsp.attn_bwd_chunk(qd, kd, vd, gd, lse, delta, to_dev_i32(qp), to_dev_i32(kp), dq,
                                 scale=scale, q_start=qs_d)
    # delta from the oracle's own O (the sums of absolute terms cover the
    # GPU's delta, taken from its bf16 rounding of its own forward's O)
    delta_ref = oracle.bwd_delta(o_ref, gv)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(qv, kv, vv, gv, lse_ref, delta_ref, qp,
                                                       kp, scale=scale, q_start=qs)
    mq, mk, mv = oracle.attention_backward_magnitudes(qv, kv, vv, gv, o_ref, lse_ref, qp, kp,
                                                      scale=scale, q_start=qs)
    # Gradients reach ~20 at this scale (dQ, dK carry the scale), so the
    # absolute and RMS bounds that suit unit-scale values do not apply; the
    # elementwise bound u * sum|terms| scales with each element's own terms.
    loose = dict(mean_rel=np.inf, max_abs=np.inf, mean_abs=np.inf)
    assert_close_rms(to_np(dq), dq_ref, bound=mq, what="dQ", **loose)
    assert_close_rms(to_np(dk), dk_ref, bound=mk, what="dK", **loose)
    assert_close_rms(to_np(dv), dv_ref, bound=mv, what="dV", **loose)


def test_bwd_chunk_non_causal_and_accumulate(mm):
    mmsp, _ = mm
    import torch
    sq, sk, hq, hkv, d = 150, 97, 4, 2, 128
    qb, qv = normal_bf16(51, (sq, hq, d))
    kb, kv = normal_bf16(52, (sk, hkv, d))
    vb, vv = normal_bf16(53, (sk, hkv, d))
    gb, gv = normal_bf16(54, (sq, hq, d))
    big = np.full(sq, 10 ** 6)
    kp = np.arange(sk)
    o, lse = oracle.attention_forward(qv, kv, vv, big, kp)
    delta = oracle.bwd_delta(o, gv)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(qv, kv, vv, gv, lse, delta, big, kp)
    dq = torch.zeros((sq, hq, d), dtype=torch.float32, device="cuda")
    args = (to_dev_bf16(qb), to_dev_bf16(kb), to_dev_bf16(vb), to_dev_bf16(gb), _dev_f32(lse),
            _dev_f32(delta), None, None, dq)
    dk, dv = mmsp.attn_bwd_chunk(*args, causal=False)
    mq, mk, mv = oracle.attention_backward_magnitudes(qv, kv, vv, gv, o, lse, big, kp)
    assert_close_rms(to_np(dq), dq_ref, bound=mq, what="dQ")
    assert_close_rms(to_np(dk), dk_ref, bound=mk, what="dK")
    assert_close_rms(to_np(dv), dv_ref, bound=mv, what="dV")
    # ACCUMULATE adds into dK/dV; dQ always accumulates
    mmsp.attn_bwd_chunk(*args, dk=dk, dv=dv, causal=False, accumulate=True)
    assert_close_rms(to_np(dk), 2 * dk_ref, bound=2 * mk, what="2 dK")
    assert_close_rms(to_np(dv), 2 * dv_ref, bound=2 * mv, what="2 dV")
    assert_close_rms(to_np(dq), 2 * dq_ref, bound=2 * mq, what="2 dQ")


def test_tiny_training_step_chain(mm):
    """GPU forward -> bf16 O -> preprocess -> backward over 4 chunks vs oracle."""
    mmsp, ring = mm
    w = TINY
    qb, qv = w.q()
    kb, kv = w.k()
    vb, vv = w.v()
    gb, gv = w.do()
    pos = np.arange(w.n_tokens, dtype=np.int32)
    kps = [pos[c * w.chunk:(c + 1) * w.chunk] for c in range(w.n_chunks)]
    q = to_dev_bf16(qb)
    ks = [to_dev_bf16(kb[c]) for c in range(4)]
    vs = [to_dev_bf16(vb[c]) for c in range(4)]
    qp, kpd = to_dev_i32(pos), [to_dev_i32(k) for k in kps]
    o, lse, o16 = ring.ring_forward(q, ks, vs, qp, kpd)
    dq, dks, dvs = ring.ring_backward(q, ks, vs, to_dev_bf16(gb), o16, lse, qp, kpd)

    ref = oracle_ring_grads(qv, list(kv), list(vv), gv, pos, kps)
    for c in range(4):
        assert_close_rms(to_np(dks[c]), ref["dk"][c], bound=ref["mk"][c], what=f"dK chunk {c}")
        assert_close_rms(to_np(dvs[c]), ref["dv"][c], bound=ref["mv"][c], what=f"dV chunk {c}")
    assert_close_rms(to_np(dq), ref["dq"], bound=ref["mq"], what="dQ")
    assert_close_abs(to_np(o), ref["o"], what="O")


@pytest.mark.parametrize("packed", [False, True])
def test_bwd_halves_equal_the_whole(mm, packed):
    """``part="dkdv"`` and ``part="dq"`` enqueue one kernel each; together
    they give bit-for-bit what one call gives, also on two streams."""
    import torch
    mmsp = mm[0] if isinstance(mm, tuple) else mm
    rng = np.random.default_rng(5)
    sq, sk, hq, hkv, d = 300, 260, 4, 2, 128
    qp = np.sort(rng.choice(2000, sq, replace=False)).astype(np.int32)
    kp = np.sort(rng.choice(2000, sk, replace=False)).astype(np.int32)
    qs = np.minimum(qp, (qp // 400) * 400).astype(np.int32) if packed else None
    dev = lambda a: torch.from_numpy(a).cuda()
    bf = lambda *s: torch.from_numpy(rng.standard_normal(s).astype(np.float32)).to(
        torch.bfloat16).cuda()
    q, k, v, do = bf(sq, hq, d), bf(sk, hkv, d), bf(sk, hkv, d), bf(sq, hq, d)
    # device tensors kept alive for the whole test: the side stream reads them
    q_start = dev(qs) if packed else None
    qp_d, kp_d = dev(qp), dev(kp)
    o, lse = mmsp.attn_fwd_chunk(q, k, v, qp_d, kp_d, q_start=q_start)
    delta = mmsp.attn_bwd_preprocess(o.to(torch.bfloat16), do)
    dq_a = torch.zeros(sq, hq, d, device="cuda")
    dk_a, dv_a = mmsp.attn_bwd_chunk(q, k, v, do, lse, delta, qp_d, kp_d, dq_a,
                                     q_start=q_start)
    dq_b = torch.zeros(sq, hq, d, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    dk_b, dv_b = mmsp.attn_bwd_chunk(q, k, v, do, lse, delta, qp_d, kp_d, None,
                                     q_start=q_start, part="dkdv")
    with torch.cuda.stream(side):
        mmsp.attn_bwd_chunk(q, k, v, do, lse, delta, qp_d, kp_d, dq_b, q_start=q_start,
                            part="dq")
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(dq_a, dq_b) and torch.equal(dk_a, dk_b) and torch.equal(dv_a, dv_b)


@pytest.mark.parametrize("packed", [False, True])
def test_backward_is_deterministic(mm, packed):
    """No atomics: every dQ, dK and dV element is summed by one thread in a
    fixed order, so two runs on the same inputs agree bit for bit."""
    import torch
    mmsp, ring = mm
    n, p, rank, hq, hkv, d = 4096, 4, 2, 8, 2, 128
    shard = n // p
    if packed:
        starts = torch.tensor([0, 1024, 1536, n], dtype=torch.int32, device="cuda")
        perm, _, first = mmsp.shard_balance_packed(starts, n, p)
        qs = first[rank * shard:(rank + 1) * shard]
    else:
        perm, _ = mmsp.shard_balance(n, p, with_inverse=False)
        qs = None
    qp = perm[rank * shard:(rank + 1) * shard]
    kps = [perm[c * shard:(c + 1) * shard] for c in range(p)]
    qb, _ = normal_bf16(81, (shard, hq, d))
    kb, _ = normal_bf16(82, (p, shard, hkv, d))
    vb, _ = normal_bf16(83, (p, shard, hkv, d))
    gb, _ = normal_bf16(84, (shard, hq, d))
    q, do = to_dev_bf16(qb), to_dev_bf16(gb)
    ks = [to_dev_bf16(kb[c]) for c in range(p)]
    vs = [to_dev_bf16(vb[c]) for c in range(p)]
    _, lse, o16 = ring.ring_forward(q, ks, vs, qp, kps, rank=rank, q_start=qs)
    runs = []
    for _ in range(2):
        dq, dks, dvs = ring.ring_backward(q, ks, vs, do, o16, lse, qp, kps, rank=rank,
                                          q_start=qs)
        torch.cuda.synchronize()
        runs.append([dq.clone()] + [t.clone() for t in dks] + [t.clone() for t in dvs])
    for a, b in zip(*runs):
        assert torch.equal(a, b)
