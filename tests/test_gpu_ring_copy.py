"""Ring with double-buffered chunk arrival (a second stream copies the next
KV chunk while the current one is computed; dK/dV are copied out as they are
produced): its outputs against the float64 oracle, and -- since it runs the
same kernels in the same order as the resident ring -- bit-identical to the
resident ring's, on repeated calls too."""

import numpy as np
import pytest

import oracle
from tests.helpers import to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mm():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from long_context_multimodal_amd import mmsp, ring
    mmsp.lib()
    return mmsp, ring


def _inputs(n_tokens, n_ranks, hq, hkv, d, seed):
    import torch
    rng = np.random.default_rng(seed)
    perm = oracle.zigzag_perm(n_tokens, n_ranks)
    shard = n_tokens // n_ranks

    def t(shape):
        return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).cuda().to(
            torch.bfloat16)
    q = t((shard, hq, d))
    ks = [t((shard, hkv, d)) for _ in range(n_ranks)]
    vs = [t((shard, hkv, d)) for _ in range(n_ranks)]
    do = t((shard, hq, d))
    pos = torch.from_numpy(perm.astype(np.int32)).cuda()
    kps = [pos[c * shard:(c + 1) * shard] for c in range(n_ranks)]
    return q, ks, vs, do, kps


@pytest.mark.parametrize("rank", [0, 2])
@pytest.mark.parametrize("fused", [True, False])
def test_received_ring_matches_resident(mm, rank, fused):
    import torch
    mmsp, ring = mm
    q, ks, vs, do, kps = _inputs(4096, 4, 8, 2, 128, seed=11 + rank)
    qp = kps[rank]
    o_a, l_a, o16_a = ring.ring_forward(q, ks, vs, qp, kps, rank=rank, fused=fused)
    dq_a, dk_a, dv_a = ring.ring_backward(q, ks, vs, do, o16_a, l_a, qp, kps, rank=rank)
    rx = ring.ChunkReceiver(ks[0], vs[0])
    dk_sent = [torch.zeros(k.shape, dtype=torch.float32, device=k.device) for k in ks]
    dv_sent = [torch.zeros(k.shape, dtype=torch.float32, device=k.device) for k in ks]
    order = ring.ring_order(rank, len(ks))
    for it in range(2):  # the receiver's buffers and events are reused
        o_b, l_b, o16_b = ring.ring_forward_received(q, ks, vs, qp, kps, rx, rank=rank,
                                                     fused=fused)
        dq_b, dk_b, dv_b = ring.ring_backward_received(q, ks, vs, do, o16_b, l_b, qp, kps, rx,
                                                       rank=rank, dk_sent=dk_sent,
                                                       dv_sent=dv_sent)
        torch.cuda.synchronize()
        # per-chunk equality first, so a mismatch names the chunk (and its
        # receive buffer, step % 2 in ring order) that differs
        same = {f"{name}[chunk {c}, step {order.index(c)}]": torch.equal(a[c], b[c])
                for name, a, b in (("dK", dk_a, dk_b), ("dV", dv_a, dv_b),
                                   ("dK sent", dk_b, dk_sent), ("dV sent", dv_b, dv_sent))
                for c in range(len(ks))}
        same["O"] = torch.equal(o_a, o_b) and torch.equal(o16_a, o16_b)
        same["LSE"] = torch.equal(l_a, l_b)
        same["dQ"] = torch.equal(dq_a, dq_b)
        if not all(same.values()):
            # which side is the odd one: run the resident backward once more
            dq_c, dk_c, dv_c = ring.ring_backward(q, ks, vs, do, o16_a, l_a, qp, kps, rank=rank)
            torch.cuda.synchronize()
            note = {
                "max |dQ a-b|": float((dq_a - dq_b).abs().max()),
                "rerun == resident": torch.equal(dq_c, dq_a) and all(
                    torch.equal(x, y) for x, y in zip(dk_c, dk_a)),
                "rerun == received": torch.equal(dq_c, dq_b) and all(
                    torch.equal(x, y) for x, y in zip(dk_c, dk_b)),
                "max |dK a-b| per chunk": [float((x - y).abs().max()) for x, y in zip(dk_a, dk_b)],
            }
            raise AssertionError(f"pass {it}: differs: "
                                 f"{[k for k, v in same.items() if not v]}; {note}")
    # every chunk but the rank's own arrived through the copy stream, twice per pass
    per_chunk = ks[0].numel() * ks[0].element_size() * 2
    assert rx.bytes_received == 2 * 2 * (len(ks) - 1) * per_chunk
    assert np.isfinite(to_np(l_b)).all()


@pytest.mark.parametrize("fused", [True, False])
def test_received_ring_matches_oracle(mm, fused):
    """The double-buffered ring's own outputs -- O, LSE, dQ, and the dK/dV
    sent back through the copy stream -- against the float64 oracle, every
    element (rank 1 of P = 4, GQA 8/2, d = 128)."""
    import torch
    from long_context_multimodal_amd.workloads import normal_bf16
    from tests.helpers import (assert_close_abs, assert_close_rms, oracle_ring_grads,
                               to_dev_bf16, to_dev_i32)
    mmsp, ring = mm
    n, p, rank, hq, hkv, d = 4096, 4, 1, 8, 2, 128
    shard = n // p
    perm = oracle.zigzag_perm(n, p)
    qp = perm[rank * shard:(rank + 1) * shard]
    kps = [perm[c * shard:(c + 1) * shard] for c in range(p)]
    qb, qv = normal_bf16(121, (shard, hq, d))
    kb, kv = normal_bf16(122, (p, shard, hkv, d))
    vb, vv = normal_bf16(123, (p, shard, hkv, d))
    gb, gv = normal_bf16(124, (shard, hq, d))
    q, do = to_dev_bf16(qb), to_dev_bf16(gb)
    ks = [to_dev_bf16(kb[c]) for c in range(p)]
    vs = [to_dev_bf16(vb[c]) for c in range(p)]
    kps_d = [to_dev_i32(x) for x in kps]
    qp_d = kps_d[rank]
    rx = ring.ChunkReceiver(ks[0], vs[0])
    dk_sent = [torch.zeros(k.shape, dtype=torch.float32, device=k.device) for k in ks]
    dv_sent = [torch.zeros(k.shape, dtype=torch.float32, device=k.device) for k in ks]
    o, lse, o16 = ring.ring_forward_received(q, ks, vs, qp_d, kps_d, rx, rank=rank, fused=fused)
    dq, _, _ = ring.ring_backward_received(q, ks, vs, do, o16, lse, qp_d, kps_d, rx, rank=rank,
                                           dk_sent=dk_sent, dv_sent=dv_sent)
    torch.cuda.synchronize()
    ref = oracle_ring_grads(qv, list(kv), list(vv), gv, qp, kps, order=ring.ring_order(rank, p))
    assert_close_abs(to_np(o), ref["o"], what="O")
    assert_close_abs(to_np(lse), ref["lse"], what="LSE")
    assert_close_rms(to_np(dq), ref["dq"], bound=ref["mq"], what="dQ")
    for c in range(p):
        assert_close_rms(to_np(dk_sent[c]), ref["dk"][c], bound=ref["mk"][c],
                         what=f"dK sent, chunk {c}")
        assert_close_rms(to_np(dv_sent[c]), ref["dv"][c], bound=ref["mv"][c],
                         what=f"dV sent, chunk {c}")
