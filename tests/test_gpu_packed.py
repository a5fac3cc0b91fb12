"""GPU parity of the packed-sample path (reset attention masks between
samples packed into one buffer) against the float64 oracle: the per-sample
zigzag permutation bit-exactly, and the forward ring and backward kernels with
per-query sample starts within the same bounds as the plain causal path."""

import numpy as np
import pytest

import oracle
from long_context_multimodal_amd.workloads import normal_bf16
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


def _lens(rng, n_samples, p, lo, hi):
    return (rng.integers(lo, hi + 1, size=n_samples) * 2 * p).tolist()


@pytest.mark.parametrize("lens,p", [([16], 2), ([8, 24, 40], 4), ([6, 6, 12, 30], 3),
                                    ("random", 8), ("big", 32)])
def test_shard_balance_packed_bit_exact(mm, lens, p):
    mmsp, _ = mm
    rng = np.random.default_rng(7)
    if lens == "random":
        lens = _lens(rng, 57, p, 1, 40)
    elif lens == "big":  # about 1.5M tokens of video-length samples
        lens = _lens(rng, 30, p, 300, 1300)
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = int(starts[-1])
    perm, inv, first = mmsp.shard_balance_packed(to_dev_i32(starts), n, p, with_inverse=True)
    want_perm, want_first = oracle.zigzag_packed_perm(starts, p)
    assert np.array_equal(to_np(perm), want_perm)
    assert np.array_equal(to_np(first), want_first)
    assert np.array_equal(to_np(inv), oracle.inverse_perm(want_perm))


def test_shard_balance_packed_leaves_bad_samples_unplaced(mm):
    mmsp, _ = mm
    # P = 2: boundaries must be multiples of 4; 6 is not, so both samples
    # touching it are left out and their slots keep -1
    starts = np.array([0, 6, 16, 24], dtype=np.int32)
    perm, inv, first = mmsp.shard_balance_packed(to_dev_i32(starts), 24, 2, with_inverse=True)
    perm, first = to_np(perm), to_np(first)
    placed = perm[perm >= 0]
    assert sorted(placed.tolist()) == list(range(16, 24))
    assert np.all(first[perm < 0] == -1) and np.all(first[perm >= 0] == 16)
    assert np.all(to_np(inv)[:16] == -1)
    # the valid last sample sits where the per-sample zigzag puts it
    want, _ = oracle.zigzag_packed_perm([0, 8], 2)
    for r in range(2):
        mine = perm[r * 12:(r + 1) * 12]
        assert mine[mine >= 0].tolist() == (want[r * 4:(r + 1) * 4] + 16).tolist()


def _packed_ring_inputs(lens, p, rank, hq, hkv, d, seed):
    starts = np.concatenate([[0], np.cumsum(lens)])
    perm, first = oracle.zigzag_packed_perm(starts, p)
    shard = perm.size // p
    qp = perm[rank * shard:(rank + 1) * shard].astype(np.int32)
    qs = first[rank * shard:(rank + 1) * shard].astype(np.int32)
    kps = [perm[c * shard:(c + 1) * shard].astype(np.int32) for c in range(p)]
    qb, qv = normal_bf16(seed, (shard, hq, d))
    kb, kv = normal_bf16(seed + 1, (p, shard, hkv, d))
    vb, vv = normal_bf16(seed + 2, (p, shard, hkv, d))
    gb, gv = normal_bf16(seed + 3, (shard, hq, d))
    return qp, qs, kps, (qb, qv), (kb, kv), (vb, vv), (gb, gv)


@pytest.mark.parametrize("lens,p,rank,hq,hkv,d", [
    ([1024, 512, 2048, 512], 2, 0, 8, 2, 128),   # several tiles per sample
    ([1024, 512, 2048, 512], 2, 1, 4, 4, 64),
    ([100, 60, 200, 44], 2, 1, 7, 1, 128),         # ragged shard (202 rows), GQA 7
    ([32] * 20 + [640], 4, 3, 4, 2, 128),          # many short samples + one long
])
def test_packed_ring_forward_backward(mm, lens, p, rank, hq, hkv, d):
    mmsp, ring = mm
    import torch
    qp, qs, kps, (qb, qv), (kb, kv), (vb, vv), (gb, gv) = _packed_ring_inputs(
        lens, p, rank, hq, hkv, d, seed=60 + rank + d)
    order = ring.ring_order(rank, p)
    q = to_dev_bf16(qb)
    ks = [to_dev_bf16(kb[c]) for c in range(p)]
    vs = [to_dev_bf16(vb[c]) for c in range(p)]
    qp_d, qs_d = to_dev_i32(qp), to_dev_i32(qs)
    kps_d = [to_dev_i32(x) for x in kps]
    o, lse, o16 = ring.ring_forward(q, ks, vs, qp_d, kps_d, rank=rank, q_start=qs_d)
    o_ref, l_ref = oracle.ring_forward(qv, list(kv), list(vv), qp, kps, order=order, q_start=qs)
    assert_close_abs(to_np(o), o_ref, what="packed O")
    assert_close_abs(to_np(lse), l_ref, what="packed LSE")
    # every query sees at least its own (diagonal) key
    assert np.isfinite(to_np(lse)).all()
    dq, dks, dvs = ring.ring_backward(q, ks, vs, to_dev_bf16(gb), o16, lse, qp_d, kps_d,
                                      rank=rank, q_start=qs_d)
    torch.cuda.synchronize()
    ref = oracle_ring_grads(qv, list(kv), list(vv), gv, qp, kps, order=order, q_start=qs)
    for c in range(p):
        assert_close_rms(to_np(dks[c]), ref["dk"][c], bound=ref["mk"][c],
                         what=f"packed dK chunk {c}")
        assert_close_rms(to_np(dvs[c]), ref["dv"][c], bound=ref["mv"][c],
                         what=f"packed dV chunk {c}")
    assert_close_rms(to_np(dq), ref["dq"], bound=ref["mq"], what="packed dQ")


def test_packed_single_sample_equals_plain_causal(mm):
    """One sample spanning the buffer: q_start = 0 everywhere must give exactly
    the plain causal kernels' results (same tiles, same arithmetic)."""
    mmsp, ring = mm
    import torch
    qp, qs, kps, (qb, _), (kb, _), (vb, _), (gb, _) = _packed_ring_inputs(
        [4096], 2, 0, 4, 2, 128, seed=80)
    q = to_dev_bf16(qb)
    ks = [to_dev_bf16(kb[c]) for c in range(2)]
    vs = [to_dev_bf16(vb[c]) for c in range(2)]
    qp_d, qs_d = to_dev_i32(qp), to_dev_i32(qs)
    kps_d = [to_dev_i32(x) for x in kps]
    a = ring.ring_forward(q, ks, vs, qp_d, kps_d, rank=0)
    b = ring.ring_forward(q, ks, vs, qp_d, kps_d, rank=0, q_start=qs_d)
    ga = ring.ring_backward(q, ks, vs, to_dev_bf16(gb), a[2], a[1], qp_d, kps_d, rank=0)
    gb_ = ring.ring_backward(q, ks, vs, to_dev_bf16(gb), b[2], b[1], qp_d, kps_d, rank=0,
                             q_start=qs_d)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert torch.equal(ga[0], gb_[0])
    for c in range(2):
        assert torch.equal(ga[1][c], gb_[1][c]) and torch.equal(ga[2][c], gb_[2][c])
