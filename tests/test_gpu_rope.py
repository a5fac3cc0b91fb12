"""GPU parity of the rotary-embedding kernel (theta 1e7, global positions up to
2M) against the float64 oracle, and of a training step on rotated queries and
keys with the gradients rotated back."""

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


@pytest.mark.parametrize("s,h,d", [(777, 5, 64), (777, 5, 128), (1001, 32, 128), (333, 1, 128),
                                   (129, 4, 64), (1, 3, 128)])
def test_rope_bf16_bit_exact(mm, s, h, d):
    """Ragged token counts and head counts from 1 to 32 (the number of tokens a
    block takes depends on the head count)."""
    mmsp, _ = mm
    rng = np.random.default_rng(d + s)
    pos = np.sort(rng.choice(2097152, s, replace=False)).astype(np.int32)
    xb, xv = normal_bf16(90 + d + h, (s, h, d))
    x = to_dev_bf16(xb)
    y = mmsp.rope(x, to_dev_i32(pos))
    want_bits, _ = oracle.rope_bf16(xv, pos, 1e7)
    # bit-exact: a flip would need a result within ~1e-10 (the angle's
    # last-bit sensitivity, see the fp32 test) of a bf16 rounding boundary
    assert np.array_equal(to_np(y), want_bits)
    # in place gives the same bits
    mmsp.rope(x, to_dev_i32(pos), out=x)
    assert np.array_equal(to_np(x), want_bits)


@pytest.mark.parametrize("s,h,d", [(500, 3, 128), (257, 32, 64)])
def test_rope_fp32_inverse_within_one_ulp(mm, s, h, d):
    mmsp, _ = mm
    import torch
    rng = np.random.default_rng(3)
    pos = np.sort(rng.choice(2097152, s, replace=False)).astype(np.int32)
    x = rng.standard_normal((s, h, d)).astype(np.float32)
    y = to_np(mmsp.rope(torch.from_numpy(x).cuda(), to_dev_i32(pos), inverse=True))
    want = oracle.rope(x, pos, 1e7, inverse=True).astype(np.float32)
    # rounded once from fp64: within one float32 ulp, plus the fp64 error of
    # the angle and of x1*cos - x2*sin.  The angle pos * theta^(-2i/d) carries
    # the last-bit difference of two correctly rounded pow() (GPU library vs
    # numpy) times pos (up to 2^21), i.e. up to ~1e-10 rad; that only shows
    # where the two terms nearly cancel and the result is far below 1.
    ulp = np.spacing(np.abs(want))
    ang = oracle.rope_angles(pos, d, 1e7)[:, None, :]
    pair = (np.abs(x[..., :d // 2]) + np.abs(x[..., d // 2:])) * (1.0 + ang)
    fp64_err = 8 * 2.0 ** -53 * np.concatenate([pair, pair], axis=-1)
    assert np.all(np.abs(y.astype(np.float64) - want) <= ulp + fp64_err)
    back = to_np(mmsp.rope(torch.from_numpy(y).cuda(), to_dev_i32(pos)))
    np.testing.assert_allclose(back, x, rtol=0, atol=2e-6)


def _pair_sum(m):
    d = m.shape[-1]
    t = m[..., : d // 2] + m[..., d // 2:]
    return np.concatenate([t, t], axis=-1)


def test_training_step_on_rotated_queries_and_keys(mm):
    """Rotate Q and every K chunk at their global positions (zigzag P=4 over
    4096 tokens, positions shifted deep into a 2M context), run the ring
    forward and backward, rotate dQ and dK back; compare with the oracle's
    rotate -> attention -> gradients -> inverse rotation."""
    mmsp, ring = mm
    import torch
    n, p, rank, hq, hkv, d = 4096, 4, 1, 8, 2, 128
    offset = 2097152 - n  # the last 4096 positions of a 2M context
    perm = oracle.zigzag_perm(n, p) + offset
    shard = n // p
    qp = perm[rank * shard:(rank + 1) * shard].astype(np.int32)
    kps = [perm[c * shard:(c + 1) * shard].astype(np.int32) for c in range(p)]
    qb, qv = normal_bf16(101, (shard, hq, d))
    kb, kv = normal_bf16(102, (p, shard, hkv, d))
    vb, vv = normal_bf16(103, (p, shard, hkv, d))
    gb, gv = normal_bf16(104, (shard, hq, d))
    qp_d = to_dev_i32(qp)
    kps_d = [to_dev_i32(x) for x in kps]
    q_rot = mmsp.rope(to_dev_bf16(qb), qp_d)
    k_rot = [mmsp.rope(to_dev_bf16(kb[c]), kps_d[c]) for c in range(p)]
    vs = [to_dev_bf16(vb[c]) for c in range(p)]
    o, lse, o16 = ring.ring_forward(q_rot, k_rot, vs, qp_d, kps_d, rank=rank)
    dq_r, dks_r, dvs = ring.ring_backward(q_rot, k_rot, vs, to_dev_bf16(gb), o16, lse, qp_d,
                                          kps_d, rank=rank)
    dq = mmsp.rope(dq_r, qp_d, inverse=True)
    dks = [mmsp.rope(dks_r[c], kps_d[c], inverse=True) for c in range(p)]
    torch.cuda.synchronize()
    # oracle: the same bf16 rotations, then attention in float64
    _, qrv = oracle.rope_bf16(qv, qp, 1e7)
    krv = [oracle.rope_bf16(kv[c], kps[c], 1e7)[1] for c in range(p)]
    assert np.array_equal(to_np(q_rot), oracle.rope_bf16(qv, qp, 1e7)[0])
    order = ring.ring_order(rank, p)
    ref = oracle_ring_grads(qrv, krv, list(vv), gv, qp, kps, order=order)
    assert_close_abs(to_np(o), ref["o"], what="O")
    assert_close_abs(to_np(lse), ref["lse"], what="LSE")
    for c in range(p):
        dk_ref = oracle.rope(ref["dk"][c], kps[c], 1e7, inverse=True)
        assert_close_rms(to_np(dks[c]), dk_ref, bound=_pair_sum(ref["mk"][c]),
                         what=f"dK chunk {c}")
        assert_close_rms(to_np(dvs[c]), ref["dv"][c], bound=ref["mv"][c], what=f"dV chunk {c}")
    dq_ref, mq_ref = ref["dq"], ref["mq"]
    assert_close_rms(to_np(dq), oracle.rope(dq_ref, qp, 1e7, inverse=True),
                     bound=_pair_sum(mq_ref), what="dQ")


@pytest.mark.parametrize("wname", ["zigzag_p8_shard8192_h32_d128_fwd_bwd",
                                   "ulysses_p32_shard65536_h4_d128_fwd_bwd"])
def test_rope_full_size(mm, wname):
    """The rotations a training step makes, at full size and in the launch
    shape the step uses: the bf16 query shard at the rank's global positions
    (up to 2^21 - 1 for the 2M-token shape) bit-exactly, and the fp32 inverse
    of a gradient-sized tensor within one ulp plus the angle's fp64 error."""
    mmsp, _ = mm
    import torch
    from long_context_multimodal_amd.workloads import WORKLOADS
    w = WORKLOADS[wname]
    pos = oracle.zigzag_perm(w.n_tokens, w.n_ranks)[:w.shard].astype(np.int32)
    qb, qv = w.q()
    pos_d = to_dev_i32(pos)
    y = mmsp.rope(to_dev_bf16(qb), pos_d)
    assert np.array_equal(to_np(y), oracle.rope_bf16(qv, pos, 1e7)[0])
    del y
    # an fp32 tensor of the same shape, rotated back in place
    g = np.random.default_rng(5).standard_normal(qv.shape).astype(np.float32)
    gd = torch.from_numpy(g).cuda()
    mmsp.rope(gd, pos_d, inverse=True, out=gd)
    got = to_np(gd).astype(np.float64)
    want = oracle.rope(g, pos, 1e7, inverse=True).astype(np.float32).astype(np.float64)
    d = w.d
    ang = oracle.rope_angles(pos, d, 1e7)[:, None, :]
    pair = (np.abs(g[..., :d // 2]) + np.abs(g[..., d // 2:])) * (1.0 + ang)
    bound = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64) + \
        8 * 2.0 ** -53 * np.concatenate([pair, pair], axis=-1)
    assert np.all(np.abs(got - want) <= bound)
