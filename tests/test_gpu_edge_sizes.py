"""Forward and backward at the edges of the tiling against the float64
oracle: one query row or one key, sizes below one MFMA block, exactly whole
tiles, chunks whose keys all precede or all follow the queries, and packed
samples of one token -- with the same bounds as the other parity tests."""

import numpy as np
import pytest

import oracle
from long_context_multimodal_amd.workloads import normal_bf16
from tests.helpers import (BF16_U, ROUNDING_SLACK, assert_close_abs, assert_close_rms,
                           to_dev_bf16, to_dev_i32, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mmsp():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from long_context_multimodal_amd import mmsp as m
    m.lib()
    return m


def _positions(layout, sq, sk, rng):
    if layout == "interleaved":
        allp = np.sort(rng.choice(4 * (sq + sk), sq + sk, replace=False))
        pick = rng.permutation(sq + sk)
        return np.sort(allp[pick[:sq]]), np.sort(allp[pick[sq:]])
    if layout == "keys_before":   # every key visible to every query
        return np.arange(sk, sk + sq), np.arange(sk)
    if layout == "keys_after":    # nothing visible: O = 0, LSE = -inf, zero gradients
        return np.arange(sq), np.arange(sq, sq + sk)
    raise ValueError(layout)


CASES = [  # (sq, sk, hq, hkv, d, layout)
    (1, 1, 1, 1, 64, "keys_before"),
    (1, 300, 2, 1, 128, "keys_before"),
    (300, 1, 2, 2, 64, "interleaved"),
    (5, 3, 4, 2, 128, "interleaved"),
    (31, 33, 4, 4, 64, "interleaved"),
    (256, 256, 2, 1, 128, "interleaved"),   # whole tiles, no tail
    (128, 64, 3, 3, 128, "keys_after"),
    (65, 200, 8, 2, 64, "keys_before"),
    # 2, 3 and 7 key tiles at d = 128: the forward's tile loop is unrolled
    # four stages deep, and these leave it after its second and third stage
    (96, 128, 2, 2, 128, "interleaved"),
    (200, 190, 3, 1, 128, "keys_before"),
    (300, 448, 4, 2, 128, "keys_before"),
]


@pytest.mark.parametrize("sq,sk,hq,hkv,d,layout", CASES)
def test_edge_sizes_forward_and_backward(mmsp, sq, sk, hq, hkv, d, layout):
    import torch
    rng = np.random.default_rng(sq * 1000 + sk)
    qp, kp = (np.asarray(a, dtype=np.int32) for a in _positions(layout, sq, sk, rng))
    seed = sq + sk + hq + d
    qb, qv = normal_bf16(seed, (sq, hq, d))
    kb, kv = normal_bf16(seed + 1, (sk, hkv, d))
    vb, vv = normal_bf16(seed + 2, (sk, hkv, d))
    gb, gv = normal_bf16(seed + 3, (sq, hq, d))
    q, k, v, do = to_dev_bf16(qb), to_dev_bf16(kb), to_dev_bf16(vb), to_dev_bf16(gb)
    qp_d, kp_d = to_dev_i32(qp), to_dev_i32(kp)
    o, lse = mmsp.attn_fwd_chunk(q, k, v, qp_d, kp_d)
    o_ref, l_ref = oracle.attention_forward(qv, kv, vv, qp, kp)
    assert_close_abs(to_np(o), o_ref, what="O")
    l_got = to_np(lse)
    assert np.array_equal(np.isneginf(l_got), np.isneginf(l_ref)), "empty rows differ"
    fin = np.isfinite(l_ref)
    if fin.any():
        assert_close_abs(l_got[fin], l_ref[fin], what="LSE")
    o16 = o.to(torch.bfloat16)
    delta = mmsp.attn_bwd_preprocess(o16, do)
    dq = torch.zeros(sq, hq, d, device="cuda")
    dk, dv = mmsp.attn_bwd_chunk(q, k, v, do, lse, delta, qp_d, kp_d, dq)
    torch.cuda.synchronize()
    delta_ref = oracle.bwd_delta(o_ref, gv)
    g = oracle.attention_backward(qv, kv, vv, gv, l_ref, delta_ref, qp, kp)
    m = oracle.attention_backward_magnitudes(qv, kv, vv, gv, o_ref, l_ref, qp, kp)
    for got, want, mag, name in zip((dq, dk, dv), g, m, ("dQ", "dK", "dV")):
        got = to_np(got)
        if not np.any(mag):  # nothing visible: exactly zero
            assert not np.any(got), f"{name} should be zero"
        elif not np.any(want):
            # the exact gradient cancels (one visible key: dS = P (dP - delta) = 0);
            # what is left is rounding, within the elementwise bound
            assert np.all(np.abs(got) <= ROUNDING_SLACK * BF16_U * mag + 1e-12), \
                f"{name} beyond rounding"
        else:
            assert_close_rms(got, want, bound=mag, what=name)


def test_packed_single_token_samples(mmsp):
    """Samples of 2P tokens with P = 1 hold one token per zigzag block: every
    query sees itself and at most one other key."""
    import torch
    lens = [2] * 40 + [64]
    starts = np.concatenate([[0], np.cumsum(lens)])
    perm, first = oracle.zigzag_packed_perm(starts, 1)
    n = perm.size
    qp = perm.astype(np.int32)
    qs = first.astype(np.int32)
    qb, qv = normal_bf16(7, (n, 4, 64))
    kb, kv = normal_bf16(8, (n, 2, 64))
    vb, vv = normal_bf16(9, (n, 2, 64))
    o, lse = mmsp.attn_fwd_chunk(to_dev_bf16(qb), to_dev_bf16(kb), to_dev_bf16(vb),
                                 to_dev_i32(qp), to_dev_i32(qp), q_start=to_dev_i32(qs))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_forward(qv, kv, vv, qp, qp, q_start=qs)
    assert_close_abs(to_np(o), o_ref, what="O")
    assert_close_abs(to_np(lse), l_ref, what="LSE")
