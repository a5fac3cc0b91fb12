"""GPU parity at the full per-rank workload sizes, in the launch configuration
bench.py times (GPU shard balance -> fused ring forward -> backward).

The oracle cannot redo whole 8K x 64K backward passes in seconds, so:

* the bench's training step: O and LSE on every element; dQ on sampled rows
  (all heads; rows at tile, half and block boundaries plus seeded random
  rows); dK and dV of every head at sampled keys of every chunk (a key's
  gradient needs the final statistics of every row, which the all-row oracle
  forward provides); two whole heads of dK/dV;
* the 2M-token per-GPU share (65,536 rows x 32 chunks): O and dQ on sampled
  rows, and dK/dV of every head at the keys that only a few rows see (the
  end of the stream);
* packed clips: O and LSE on every element, dQ on sampled rows, dK/dV of
  every head at sampled keys including clip edges;
* and two identities that hold at any size (sums of dV and of dK over every
  key of every chunk) within derived worst-case bounds.

Gradient references take delta from the oracle's own O; the elementwise
bounds (oracle.attention_backward_magnitudes) cover the GPU's delta from its
bf16 output.
"""

import numpy as np
import pytest

import oracle
from long_context_multimodal_amd.workloads import (GQA, MODALITY, PACKED, PACKED_TRAIN, RANK_FWD,
                                                   TRAIN, ULYSSES, ULYSSES_TRAIN)
from tests.helpers import (BF16_U, ROUNDING_SLACK, assert_close_abs, assert_close_rms,
                           to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mm():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from long_context_multimodal_amd import mmsp, ring
    mmsp.lib()
    return mmsp, ring


def _dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _sample_rows(n, extra_edges=(), seed=0, n_random=16):
    rows = {0, 1, 31, 32, 63, 64, 127, 128, 255, 256, n // 2 - 1, n // 2, n // 2 + 1, n - 1}
    rows |= {e for e in extra_edges if 0 <= e < n}
    rng = np.random.default_rng(seed)
    rows |= set(rng.choice(n, n_random, replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def _run(mm, w, backward=False, rank=0, kv_grads="full", tail_keys=0):
    """Run the hot path on the GPU; return host copies and the oracle inputs.

    ``kv_grads``: ``"full"`` copies every dK/dV chunk to the host; ``"sums"``
    only the float64 sums of dK and dV over all keys of all chunks
    (``[Hkv, d]`` each) and the last ``tail_keys`` keys of chunk 0.
    """
    mmsp, ring = mm
    import torch
    qb, qv = w.q()
    kb, kv = w.k()
    vb, vv = w.v()
    qs = qs_np = None
    if w.layout == "packed":
        starts = w.sample_starts()
        perm, _, first = mmsp.shard_balance_packed(torch.from_numpy(starts).cuda(), w.n_tokens,
                                                   w.n_ranks)
        perm_np = to_np(perm).astype(np.int64)
        want_perm, want_first = oracle.zigzag_packed_perm(starts, w.n_ranks)
        assert np.array_equal(to_np(first), want_first)  # bit-exact sample starts
        qs = first[rank * w.shard:(rank + 1) * w.shard]
        qs_np = want_first[rank * w.shard:(rank + 1) * w.shard]
    else:
        labels = w.labels()
        mode = mmsp.BALANCE_MODALITY if w.layout == "modality" else mmsp.BALANCE_ZIGZAG
        perm, _ = mmsp.shard_balance(w.n_tokens, w.n_ranks, mode, w.granularity,
                                     labels=torch.from_numpy(labels).cuda()
                                     if mode == mmsp.BALANCE_MODALITY else None,
                                     with_inverse=False)
        perm_np = to_np(perm).astype(np.int64)
        want_perm = (oracle.modality_perm(labels, w.n_ranks, w.granularity)
                     if mode == mmsp.BALANCE_MODALITY
                     else oracle.zigzag_perm(w.n_tokens, w.n_ranks))
    assert np.array_equal(perm_np, want_perm)  # bit-exact shard permutation
    qp = perm[rank * w.shard:(rank + 1) * w.shard]
    kps = [perm[c * w.chunk:(c + 1) * w.chunk] for c in range(w.n_chunks)]
    q = _dev_bf16(qb)
    ks = [_dev_bf16(kb[c]) for c in range(w.n_chunks)]
    vs = [_dev_bf16(vb[c]) for c in range(w.n_chunks)]
    o, lse, o16 = ring.ring_forward(q, ks, vs, qp, kps, rank=rank, q_start=qs)
    out = {"o": to_np(o), "lse": to_np(lse)}
    gv = None
    if backward:
        gb, gv = w.do()
        dq, dks, dvs = ring.ring_backward(q, ks, vs, _dev_bf16(gb), o16, lse, qp, kps, rank=rank,
                                          q_start=qs)
        out["dq"] = to_np(dq)
        if kv_grads == "full":
            out["dk"] = [to_np(t) for t in dks]
            out["dv"] = [to_np(t) for t in dvs]
        else:
            out["dk_sum"] = to_np(sum(t.double().sum(dim=0) for t in dks))
            out["dv_sum"] = to_np(sum(t.double().sum(dim=0) for t in dvs))
            if tail_keys:
                out["dk_tail"] = to_np(dks[0][-tail_keys:])
                out["dv_tail"] = to_np(dvs[0][-tail_keys:])
        del dks, dvs
    torch.cuda.synchronize()
    host = {"q": qv, "k": kv, "v": vv, "do": gv, "qs": qs_np,
            "qp": perm_np[rank * w.shard:(rank + 1) * w.shard],
            "kps": [perm_np[c * w.chunk:(c + 1) * w.chunk] for c in range(w.n_chunks)],
            "order": [(rank - t) % w.n_chunks for t in range(w.n_chunks)]}
    return out, host


# ---- derived bounds of two identities that hold at any size ----------------
#
# Every row of these shards sees at least its own diagonal key, and its
# weights over all keys of all chunks sum to one.
#  * dV:  sum_j dV_j = sum_i (sum_j P_ij) dO_i = sum_i dO_i.  The backward
#    uses bf16(P_ij) = P_ij (1 + r_ij), |r_ij| <= u, so each row's weights sum
#    to one within u and the two sides differ by at most u sum_i |dO_i|.
#  * dK:  sum_j dK_j = scale sum_i q_i (sum_j dS_ij) = 0, because
#    sum_j P_ij dP_ij = dO_i . O_i = D_i and sum_j P_ij = 1.  With dS rounded
#    to bf16 and D taken from the bf16 rounding of a forward whose weights were
#    rounded, |sum_j dS_ij| <= u (sum_j |dS_ij| + sum_c |dO_ic O_ic|
#    + sum_j P_ij |dP_ij|) to first order, and each of the three sums is at
#    most ||dO_i|| V (|dP_ij| <= ||dO_i|| ||v_j||, ||O_i|| <= max ||v_j||,
#    sum_j P_ij = 1), twice for the first, where V = max_j ||v_j||.  So
#    |sum_j dK_jc| <= scale sum_i |q_ic| 4 u ||dO_i|| V, summed over the
#    query heads of the KV head.
# Both are worst-case sums of rounding errors over every row, so they are far
# above what the kernels produce (printed); they catch gross errors only --
# the elementwise comparisons at sampled keys and rows do the real checking.


def _check_sum_identities(out, host, w):
    u, slack = BF16_U, ROUNDING_SLACK
    do = host["do"].astype(np.float64)
    q = host["q"].astype(np.float64)
    g = w.hq // w.hkv
    dv_sum = out["dv_sum"] if "dv_sum" in out else sum(
        x.astype(np.float64).sum(axis=0) for x in out["dv"])
    dk_sum = out["dk_sum"] if "dk_sum" in out else sum(
        x.astype(np.float64).sum(axis=0) for x in out["dk"])
    want_dv = do.reshape(w.shard, w.hkv, g, w.d).sum(axis=(0, 2))
    bound_dv = slack * u * np.abs(do).reshape(w.shard, w.hkv, g, w.d).sum(axis=(0, 2))
    err_dv = np.abs(dv_sum - want_dv)
    assert np.all(err_dv <= bound_dv), "sum of dV over keys"
    vmax = np.zeros(w.hkv)
    for c in range(w.n_chunks):
        vmax = np.maximum(vmax, np.sqrt((host["v"][c].astype(np.float64) ** 2).sum(axis=2)).max(0))
    dnorm = np.sqrt((do ** 2).sum(axis=2))                      # [Sq, Hq]
    kvh = np.arange(w.hq) // g
    per_row = 4 * u * dnorm * vmax[kvh][None, :]                  # [Sq, Hq]
    terms = np.abs(q) * per_row[:, :, None]                       # [Sq, Hq, d]
    bound_dk = slack * (1.0 / np.sqrt(w.d)) * terms.reshape(w.shard, w.hkv, g, w.d).sum(axis=(0, 2))
    assert np.all(np.abs(dk_sum) <= bound_dk), "sum of dK over keys"
    print(f"[identities] {w.name}: |sum dV - sum dO| max {err_dv.max():.2e} (bound min "
          f"{bound_dv.min():.2e}); |sum dK| max {np.abs(dk_sum).max():.2e} (bound min "
          f"{bound_dk.min():.2e})", flush=True)


def _dq_rows_check(out, host, w, rows, o_rows=None, l_rows=None):
    """dQ (all heads) on sampled rows against the exact per-row oracle."""
    q, k, v, do = host["q"], host["k"], host["v"], host["do"]
    qp, kps, order = host["qp"], host["kps"], host["order"]
    qs = host["qs"]
    qsr = None if qs is None else qs[rows]
    if o_rows is None:
        o_rows, l_rows = oracle.ring_forward(q, list(k), list(v), qp, kps, order=order,
                                             rows=rows, q_start=qs)
    assert_close_abs(out["o"][rows], o_rows, what="O rows")
    delta_rows = oracle.bwd_delta(o_rows, do[rows])
    c_rows = sum(oracle.attention_abs_dp(q[rows], k[c], v[c], do[rows], l_rows, qp[rows], kps[c],
                                         q_start=qsr) for c in order)
    dq_ref = np.zeros((len(rows), w.hq, w.d))
    mq_ref = np.zeros((len(rows), w.hq, w.d))
    for c in order:
        dq_c, _, _ = oracle.attention_backward(q[rows], k[c], v[c], do[rows], l_rows, delta_rows,
                                               qp[rows], kps[c], q_start=qsr)
        mq_c, _, _ = oracle.attention_backward_magnitudes(q[rows], k[c], v[c], do[rows], o_rows,
                                                          l_rows, qp[rows], kps[c], q_start=qsr,
                                                          dp_abs=c_rows)
        dq_ref += dq_c
        mq_ref += mq_c
    assert_close_rms(out["dq"][rows], dq_ref, bound=mq_ref, what="dQ rows")


def _dkdv_keys_check(out, host, w, o_ref, l_ref, keys_per_chunk):
    """dK and dV of every head at sampled keys of every chunk, against the
    oracle given the final O and LSE of every row (a key's gradient sums over
    every row that sees it)."""
    q, k, v, do = host["q"], host["k"], host["v"], host["do"]
    qp, kps, qs = host["qp"], host["kps"], host["qs"]
    print(f"[keys] {w.name}: oracle sum of P|dP| on every row", flush=True)
    delta = oracle.bwd_delta(o_ref, do)
    c_all = sum(oracle.attention_abs_dp(q, k[c], v[c], do, l_ref, qp, kps[c], q_start=qs)
                for c in range(w.n_chunks))
    got_k, got_v, want_k, want_v, mag_k, mag_v = [], [], [], [], [], []
    for c in range(w.n_chunks):
        keys = keys_per_chunk[c]
        kc, vc, kpc = k[c][keys], v[c][keys], kps[c][keys]
        _, dk_s, dv_s = oracle.attention_backward(q, kc, vc, do, l_ref, delta, qp, kpc,
                                                  q_start=qs)
        _, mk_s, mv_s = oracle.attention_backward_magnitudes(q, kc, vc, do, o_ref, l_ref, qp, kpc,
                                                             q_start=qs, dp_abs=c_all)
        got_k.append(out["dk"][c][keys])
        got_v.append(out["dv"][c][keys])
        want_k.append(dk_s)
        want_v.append(dv_s)
        mag_k.append(mk_s)
        mag_v.append(mv_s)
    n = sum(len(x) for x in keys_per_chunk)
    print(f"[keys] {w.name}: dK, dV of {n} keys x {w.hkv} KV heads", flush=True)
    assert_close_rms(np.concatenate(got_k), np.concatenate(want_k), bound=np.concatenate(mag_k),
                     what="dK sampled keys, every head")
    assert_close_rms(np.concatenate(got_v), np.concatenate(want_v), bound=np.concatenate(mag_v),
                     what="dV sampled keys, every head")


@pytest.mark.parametrize("w", [RANK_FWD, GQA, MODALITY, ULYSSES, PACKED], ids=lambda w: w.name)
def test_forward_full_size_sampled_rows(mm, w):
    out, host = _run(mm, w)
    edges = [w.granularity * k - 1 for k in range(1, 6)] + [w.granularity * k for k in range(1, 6)]
    rows = _sample_rows(w.shard, extra_edges=edges if w.granularity else ())
    o_ref, l_ref = oracle.ring_forward(host["q"], list(host["k"]), list(host["v"]), host["qp"],
                                       host["kps"], order=host["order"], rows=rows,
                                       q_start=None if host["qs"] is None else host["qs"])
    assert_close_abs(out["o"][rows], o_ref, what=f"{w.name} O")
    assert_close_abs(out["lse"][:, rows], l_ref, what=f"{w.name} LSE")
    # every row of a shard sees at least its own diagonal key
    assert np.isfinite(out["lse"]).all()


@pytest.fixture(scope="module")
def zigzag_step(mm):
    """The bench's training step (rank 0 of zigzag P = 8 over 65,536 tokens,
    8192-row shard, 32 heads, d = 128, 8 chunks, fused merge) on the GPU, and
    the oracle's forward on every row (about a minute on 16 host cores).  Its
    forward is exactly the forward-only configuration of the same shape."""
    out, host = _run(mm, TRAIN, backward=True)
    w = TRAIN
    print(f"[full] {w.name}: oracle forward on all {w.shard} rows x {w.hq} heads", flush=True)
    o_ref, l_ref = oracle.ring_forward(host["q"], list(host["k"]), list(host["v"]), host["qp"],
                                       host["kps"], order=host["order"])
    return out, host, o_ref, l_ref


def test_forward_full_size_every_element(zigzag_step):
    """The bench's forward configuration compared on every element of O and
    LSE, not a sample."""
    out, host, o_ref, l_ref = zigzag_step
    assert_close_abs(out["o"], o_ref, what=f"{RANK_FWD.name} O, every element")
    assert_close_abs(out["lse"], l_ref, what=f"{RANK_FWD.name} LSE, every element")


def test_training_step_full_size(zigzag_step):
    """dQ on sampled rows (all heads); dK and dV of every head at sampled keys
    of every chunk (tile edges, chunk halves, random keys); two whole heads of
    dK/dV (every key of every chunk); the dV- and dK-sum identities."""
    out, host, o_ref, l_ref = zigzag_step
    w = TRAIN
    rows = _sample_rows(w.shard, seed=1)
    _dq_rows_check(out, host, w, rows, o_ref[rows], l_ref[:, rows])
    keys = [_sample_rows(w.chunk, seed=100 + c) for c in range(w.n_chunks)]
    _dkdv_keys_check(out, host, w, o_ref, l_ref, keys)
    q, k, v, do = host["q"], host["k"], host["v"], host["do"]
    qp, kps = host["qp"], host["kps"]
    for h in (0, 31):
        q1, do1 = q[:, h:h + 1], do[:, h:h + 1]
        k1 = [k[c][:, h:h + 1] for c in range(w.n_chunks)]
        v1 = [v[c][:, h:h + 1] for c in range(w.n_chunks)]
        o1, l1 = o_ref[:, h:h + 1], l_ref[h:h + 1]
        d1 = oracle.bwd_delta(o1, do1)
        c1 = sum(oracle.attention_abs_dp(q1, k1[c], v1[c], do1, l1, qp, kps[c])
                 for c in range(w.n_chunks))
        dk_ref, dv_ref, mk_ref, mv_ref = [], [], [], []
        for c in range(w.n_chunks):
            _, dk_c, dv_c = oracle.attention_backward(q1, k1[c], v1[c], do1, l1, d1, qp, kps[c])
            _, mk_c, mv_c = oracle.attention_backward_magnitudes(q1, k1[c], v1[c], do1, o1, l1,
                                                                 qp, kps[c], dp_abs=c1)
            dk_ref.append(dk_c[:, 0])
            dv_ref.append(dv_c[:, 0])
            mk_ref.append(mk_c[:, 0])
            mv_ref.append(mv_c[:, 0])
        assert_close_rms(np.stack([x[:, h] for x in out["dk"]]), np.stack(dk_ref),
                         bound=np.stack(mk_ref), what=f"dK head {h}")
        assert_close_rms(np.stack([x[:, h] for x in out["dv"]]), np.stack(dv_ref),
                         bound=np.stack(mv_ref), what=f"dV head {h}")
    _check_sum_identities(out, host, w)


def test_ulysses_training_step_full_size(mm):
    """The hybrid scheme's per-GPU share (65,536-token rows, 4 heads, 32 ring
    steps over 2,097,152 tokens): O and dQ on sampled rows; dK and dV of every
    head at the last 256 keys of the stream, whose gradients need the final
    statistics of only the 256 rows that can see them; the dV- and dK-sum
    identities over every key of all 32 chunks.  The elementwise dK/dV check
    of every key at this tiling (512 key tiles per head, 4 KV heads) is in
    test_gpu_tile_order.py."""
    w = ULYSSES_TRAIN
    tail = 256
    out, host = _run(mm, w, backward=True, kv_grads="sums", tail_keys=tail)
    rows = _sample_rows(w.shard, seed=2, n_random=8)
    _dq_rows_check(out, host, w, rows)
    q, k, v, do = host["q"], host["k"], host["v"], host["do"]
    qp, kps, order = host["qp"], host["kps"], host["order"]
    kp_tail = kps[0][-tail:]
    sees = np.flatnonzero(qp >= kp_tail.min())
    rows_t = np.arange(w.shard - tail, w.shard)
    assert np.array_equal(sees, rows_t)  # the rows that see the tail keys: the last 256
    print(f"[tail] {w.name}: oracle forward of {tail} rows over all {w.n_chunks} chunks",
          flush=True)
    o_t, l_t = oracle.ring_forward(q[rows_t], list(k), list(v), qp[rows_t], kps, order=order)
    d_t = oracle.bwd_delta(o_t, do[rows_t])
    c_t = sum(oracle.attention_abs_dp(q[rows_t], k[c], v[c], do[rows_t], l_t, qp[rows_t], kps[c])
              for c in order)
    _, dk_ref, dv_ref = oracle.attention_backward(q[rows_t], k[0][-tail:], v[0][-tail:],
                                                  do[rows_t], l_t, d_t, qp[rows_t], kp_tail)
    _, mk, mv = oracle.attention_backward_magnitudes(q[rows_t], k[0][-tail:], v[0][-tail:],
                                                     do[rows_t], o_t, l_t, qp[rows_t], kp_tail,
                                                     dp_abs=c_t)
    assert_close_rms(out["dk_tail"], dk_ref, bound=mk, what="dK, last keys of the stream")
    assert_close_rms(out["dv_tail"], dv_ref, bound=mv, what="dV, last keys of the stream")
    _check_sum_identities(out, host, w)


def test_packed_training_step_full_size(mm):
    """Video clips packed into 65,536 tokens, each zigzagged over 8 ranks (reset
    masks between clips): the oracle forward on every row (each row sees only
    its own clip), O and dQ on sampled rows (including rows next to clip
    boundaries), dK and dV of every head at sampled keys of every chunk
    (including keys next to clip boundaries), and both sum identities."""
    w = PACKED_TRAIN
    out, host = _run(mm, w, backward=True)
    starts = w.sample_starts()
    bnd = np.concatenate([starts[1:-1], starts[1:-1] - 1])
    print(f"[full] {w.name}: oracle forward on all {w.shard} rows x {w.hq} heads", flush=True)
    o_ref, l_ref = oracle.ring_forward(host["q"], list(host["k"]), list(host["v"]), host["qp"],
                                       host["kps"], order=host["order"], q_start=host["qs"])
    assert_close_abs(out["o"], o_ref, what="packed O, every element")
    assert_close_abs(out["lse"], l_ref, what="packed LSE, every element")
    edges = np.flatnonzero(np.isin(host["qp"], bnd))
    rows = np.unique(np.concatenate([_sample_rows(w.shard, seed=3, n_random=8), edges[:16]]))
    _dq_rows_check(out, host, w, rows, o_ref[rows], l_ref[:, rows])
    keys = []
    for c in range(w.n_chunks):
        kedge = np.flatnonzero(np.isin(host["kps"][c], bnd))[:8]
        keys.append(np.unique(np.concatenate([_sample_rows(w.chunk, seed=200 + c, n_random=16),
                                              kedge])))
    _dkdv_keys_check(out, host, w, o_ref, l_ref, keys)
    _check_sum_identities(out, host, w)
