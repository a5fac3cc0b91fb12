"""Pins of the rotary-embedding oracle: a hand-worked example, position 0 is
the identity, pair norms are kept, scores depend only on relative positions,
the inverse undoes the rotation, and a scalar restatement with math.cos/sin."""

import json
import math
import os

import numpy as np

from oracle import rope, rope_angles, rope_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rope_theta1e7_example.json")


def test_hand_worked_example():
    g = json.load(open(GOLDEN))
    y = rope(np.array(g["x"]).reshape(1, 1, 4), np.array([g["pos"]]), g["theta"])
    np.testing.assert_allclose(y.ravel(), g["y"], rtol=0, atol=1e-14)


def test_position_zero_is_identity_and_norms_are_kept(rng):
    x = rng.standard_normal((5, 3, 128))
    pos = np.array([0, 1, 1000, 65535, 2097151])
    y = rope(x, pos, 1e7)
    np.testing.assert_array_equal(y[0], x[0])
    pair = lambda t: t[..., :64] ** 2 + t[..., 64:] ** 2
    np.testing.assert_allclose(pair(y), pair(x), rtol=1e-12, atol=1e-12)


def test_scores_depend_only_on_relative_position(rng):
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    for m, n, t in [(7, 3, 100), (2000000, 1999000, -1999000), (5, 50, 12345)]:
        a = float((rope(q, np.array([m]), 1e7) * rope(k, np.array([n]), 1e7)).sum())
        b = float((rope(q, np.array([m + t]), 1e7) * rope(k, np.array([n + t]), 1e7)).sum())
        assert abs(a - b) <= 1e-9 * max(1.0, abs(a))


def test_inverse_undoes_rotation(rng):
    x = rng.standard_normal((4, 2, 64))
    pos = np.array([3, 17, 400000, 2097000])
    np.testing.assert_allclose(rope(rope(x, pos, 1e7), pos, 1e7, inverse=True), x, atol=1e-12)


def test_scalar_restatement(rng):
    d, theta = 8, 1e7
    x = rng.standard_normal((3, 1, d))
    pos = [0, 9, 123456]
    y = rope(x, np.array(pos), theta)
    for s, p in enumerate(pos):
        for i in range(d // 2):
            a = p * theta ** (-2.0 * i / d)
            assert abs(y[s, 0, i] - (x[s, 0, i] * math.cos(a) - x[s, 0, i + d // 2] * math.sin(a))) < 1e-12
            assert abs(y[s, 0, i + d // 2]
                       - (x[s, 0, i + d // 2] * math.cos(a) + x[s, 0, i] * math.sin(a))) < 1e-12
    assert rope_angles(np.array([2]), 4, 100.0).tolist() == [[2.0, 0.2]]


def test_bf16_rounding_goes_through_float32(rng):
    x = rng.standard_normal((16, 2, 64))
    pos = np.arange(16) * 99991
    bits, vals = rope_bf16(x, pos, 1e7)
    y32 = rope(x, pos, 1e7).astype(np.float32)
    # every result is the bf16 nearest to the float32 rotation (ties to even)
    up = (vals.view(np.uint32) + np.uint32(0x10000)).view(np.float32)
    dn = (vals.view(np.uint32) - np.uint32(0x10000)).view(np.float32)
    err = np.abs(vals.astype(np.float64) - y32)
    assert np.all(err <= np.abs(up.astype(np.float64) - y32))
    assert np.all(err <= np.abs(dn.astype(np.float64) - y32))
    assert bits.dtype == np.uint16
