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


# Tile shapes of the kernels the plan orders (scheduling, not the method):
# forward workgroups of 256 query rows over 64-key tiles, dQ workgroups of 128
# rows over 64-key tiles, dK/dV workgroups of 128 keys over 32-row tiles.
_FWD_BM, _FWD_BN, _DQ_BM, _DQ_BN, _KV_BK, _KV_BQ = 256, 64, 128, 64, 128, 32


def _expected_plan(qp, qs, kp):
    """Header, heaviest-first tile lists and work counts of a tile plan,
    counted directly from the positions (ties in ascending tile order)."""
    sq, sk = qp.size, kp.size

    def qtiles(bm, bn):
        w = []
        for q0 in range(0, sq, bm):
            qmax = qp[min(q0 + bm, sq) - 1]
            nk = np.searchsorted(kp, qmax, side="right")
            kbeg = np.searchsorted(kp, qs[q0], side="left")
            w.append(max(0, -(-nk // bn) - kbeg // bn))
        return np.array(w, dtype=np.int64)

    def ktiles():
        w = []
        for j0 in range(0, sk, _KV_BK):
            kk = kp[j0:j0 + _KV_BK]
            qbeg = np.searchsorted(qp, kk[0], side="left")
            qend = np.searchsorted(qs, kk[-1], side="right")
            w.append(max(0, -(-qend // _KV_BQ) - qbeg // _KV_BQ))
        return np.array(w, dtype=np.int64)

    works = [qtiles(_FWD_BM, _FWD_BN), qtiles(_DQ_BM, _DQ_BN), ktiles()]
    lists = [np.lexsort((np.arange(w.size), -w)) for w in works]
    header = [0x4E414C50, sq, sk] + [w.size for w in works] + [0, 0]
    return np.concatenate([header] + lists + works).astype(np.int32)


def _plan_cases():
    cases = []
    # shards up to 8192 positions take the one-workgroup plan; the last case
    # (16384-row shard) the two-kernel plan for larger shards
    for lens, p, rank in (([2], 1, 0), ([4, 8], 2, 1), ([1024, 512, 2048, 512], 2, 0),
                          ([100, 60, 200, 44], 2, 1), ([32] * 20 + [640], 4, 3),
                          ([8192, 4100, 12284, 8192], 2, 1)):
        starts = np.concatenate([[0], np.cumsum(lens)])
        perm, first = oracle.zigzag_packed_perm(starts, p)
        shard = perm.size // p
        qp, qs = perm[rank * shard:(rank + 1) * shard], first[rank * shard:(rank + 1) * shard]
        for c in range(p):
            cases.append((qp, qs, perm[c * shard:(c + 1) * shard]))
    return cases


def test_packed_plan_lists_tiles_heaviest_first(mm):
    """Bit-exact plan on small shards and on every chunk of the 65,536-token
    packed workload's rank 0 (5 clips, per-sample zigzag over 8 ranks)."""
    mmsp, ring = mm
    from long_context_multimodal_amd import workloads as W
    cases = _plan_cases()
    w = W.PACKED_TRAIN
    perm, first = oracle.zigzag_packed_perm(w.sample_starts(), w.n_ranks)
    for c in range(w.n_chunks):
        cases.append((perm[:w.shard], first[:w.shard], perm[c * w.chunk:(c + 1) * w.chunk]))
    for i, (qp, qs, kp) in enumerate(cases):
        want = _expected_plan(qp, qs, kp)
        got = to_np(mmsp.packed_plan(to_dev_i32(qp), to_dev_i32(qs), to_dev_i32(kp)))
        assert got.size == want.size, i
        assert np.array_equal(got, want), f"case {i}"
        n = want[3:6]
        lists = np.split(want[8:8 + n.sum()], np.cumsum(n)[:2])
        for lst, m in zip(lists, n):  # every tile exactly once
            assert sorted(lst.tolist()) == list(range(m))


@pytest.mark.parametrize("lens,p,rank,hq,hkv,d", [
    ([4, 8], 2, 1, 2, 1, 64),                   # 6-row shard: one tile in every list
    ([1024, 512, 2048, 512], 2, 0, 8, 8, 128),  # 8 heads: each XCD keeps its own head
    ([1024, 512, 2048, 512], 2, 1, 4, 2, 64),   # heads simply take turns
    ([100, 60, 200, 44], 2, 1, 7, 1, 128),      # ragged shard, GQA 7
])
def test_packed_plan_leaves_results_unchanged(mm, lens, p, rank, hq, hkv, d):
    """A plan only reorders workgroups: forward and backward give the same
    bits with the plan, without it, with a plan of other positions of the same
    sizes, and with a plan of other sizes (which the kernels ignore)."""
    mmsp, ring = mm
    import torch
    qp, qs, kps, (qb, _), (kb, _), (vb, _), (gb, _) = _packed_ring_inputs(
        lens, p, rank, hq, hkv, d, seed=90 + d)
    q, do = to_dev_bf16(qb), to_dev_bf16(gb)
    qp_d, qs_d = to_dev_i32(qp), to_dev_i32(qs)
    c = (rank + 1) % p  # a chunk of another rank
    k, v, kp_d = to_dev_bf16(kb[c]), to_dev_bf16(vb[c]), to_dev_i32(kps[c])
    sq, sk = qp.size, kps[c].size
    plans = {
        "none": None,
        "own": mmsp.packed_plan(qp_d, qs_d, kp_d),
        # the rank's own chunk: same sizes, other positions
        "other positions": mmsp.packed_plan(qp_d, qs_d, to_dev_i32(kps[rank])),
    }
    # a plan made for fewer queries, in a buffer large enough for these sizes
    small = mmsp.packed_plan(qp_d[:sq // 2].contiguous(), qs_d[:sq // 2].contiguous(), kp_d)
    buf = torch.zeros(mmsp.lib().mmsp_attn_packed_plan_bytes(sq, sk) // 4, dtype=torch.int32,
                      device=q.device)
    buf[:small.numel()] = small
    plans["other sizes"] = buf
    outs = {}
    for name, plan in plans.items():
        o, lse = mmsp.attn_fwd_chunk(q, k, v, qp_d, kp_d, q_start=qs_d, plan=plan)
        o16 = torch.empty(o.shape, dtype=torch.bfloat16, device=o.device)
        mmsp.lse_merge(o, lse, None, None, o_final=o16)
        delta = mmsp.attn_bwd_preprocess(o16, do)
        dq = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
        dk, dv = mmsp.attn_bwd_chunk(q, k, v, do, lse, delta, qp_d, kp_d, dq, q_start=qs_d,
                                     plan=plan)
        outs[name] = (o, lse, dq, dk, dv)
    torch.cuda.synchronize()
    for name, got in outs.items():
        for x, y, what in zip(outs["none"], got, ("O", "LSE", "dQ", "dK", "dV")):
            assert torch.equal(x, y), f"{what} with plan '{name}'"


@pytest.mark.parametrize("lens,p", [([1024, 512, 2048, 512], 2), ([32] * 20 + [640], 4),
                                    ([8192, 4100, 12284, 8192], 2)])
def test_batched_plans_equal_single_plans(mm, lens, p):
    """The plans of all chunks in one launch (positions back to back) equal the
    per-chunk plans bit for bit, also for shards above 8192 positions (the
    two-kernel path); the ring helper takes the batched path for slices of one
    permutation."""
    mmsp, ring = mm
    import torch
    starts = np.concatenate([[0], np.cumsum(lens)])
    perm, first = oracle.zigzag_packed_perm(starts, p)
    shard = perm.size // p
    for rank in range(p):
        qp = to_dev_i32(perm[rank * shard:(rank + 1) * shard])
        qs = to_dev_i32(first[rank * shard:(rank + 1) * shard])
        perm_d = to_dev_i32(perm)
        kps = [perm_d[c * shard:(c + 1) * shard] for c in range(p)]
        block = ring.packed_plans(qp, qs, kps)
        assert isinstance(block, torch.Tensor) and block.shape[0] == p
        for c in range(p):
            single = mmsp.packed_plan(qp, qs, kps[c].contiguous().clone())
            assert torch.equal(block[c], single), f"rank {rank} chunk {c}"
        # reusing the buffers gives the same plans
        again = ring.packed_plans(qp, qs, kps, plans=block.clone())
        assert torch.equal(again, block)
        # separate arrays take the per-chunk path
        lst = ring.packed_plans(qp, qs, [k.clone() for k in kps])
        assert isinstance(lst, list) and all(torch.equal(a, b) for a, b in zip(lst, block))
