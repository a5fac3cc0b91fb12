"""Pins of the oracle's row gather and scatter into shard order: a hand-worked
example, the zigzag closed form, and gather followed by scatter restoring the
stream."""

import numpy as np

from oracle import gather_rows, scatter_rows, zigzag_packed_perm, zigzag_perm


def test_gather_worked_example():
    x = np.arange(8).reshape(4, 2) * 10
    got = gather_rows(x, [2, -1, 0, 3, 4])
    assert got.tolist() == [[40, 50], [0, 0], [0, 10], [60, 70], [0, 0]]
    out = np.full((4, 2), 7)
    scatter_rows(np.array([[1, 2], [3, 4], [5, 6]]), [3, -1, 0], out)
    assert out.tolist() == [[5, 6], [7, 7], [7, 7], [1, 2]]


def test_gather_of_zigzag_shards_is_the_closed_form():
    n, p = 96, 3
    lb = n // (2 * p)
    perm = zigzag_perm(n, p)
    stream = np.arange(n)[:, None] * np.array([1, -1])
    for r in range(p):
        got = gather_rows(stream, perm[r * n // p:(r + 1) * n // p])[:, 0]
        want = np.concatenate([np.arange(r * lb, (r + 1) * lb),
                               np.arange((2 * p - 1 - r) * lb, (2 * p - r) * lb)])
        assert np.array_equal(got, want)


def test_scatter_undoes_gather(rng):
    starts = [0, 24, 72, 96]
    perm, _ = zigzag_packed_perm(starts, 3)
    x = rng.standard_normal((96, 2, 5))
    back = scatter_rows(gather_rows(x, perm), perm, np.zeros_like(x))
    assert np.array_equal(back, x)
