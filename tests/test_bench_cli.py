"""bench.py's command-line contract on the CPU: more than one GPU is refused
with a message before anything touches a device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "--gpus 2" in r.stderr and r.stdout == ""


def test_incompatible_modes_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--graph", "--ring-copy"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0 and "--ring-copy" in r.stderr


def test_fixed_cost_fit_recovers_known_costs():
    """The fit behind ``--fixed-cost`` (T = L + n * (tiles * t + F)) returns the
    per-launch, per-tile and per-workgroup costs that generated its points,
    exactly without noise and closely with it."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    L, t, F = 14.0, 1.7, 9.5
    shapes = [(n, tiles) for n in (1.0, 2.0, 4.0) for tiles in (16, 32, 64, 128)]
    exact = [(n, tiles, L + n * (tiles * t + F)) for n, tiles in shapes]
    got = bench.fit_fixed_costs(exact)
    assert np.allclose(got, (L, t, F), rtol=0, atol=1e-9)
    rng = np.random.default_rng(3)
    noisy = [(n, tiles, T * (1 + 0.002 * rng.standard_normal())) for n, tiles, T in exact]
    got = bench.fit_fixed_costs(noisy)
    assert abs(got[1] - t) < 0.02 and abs(got[2] - F) < 2.0 and abs(got[0] - L) < 5.0
    # 3 us more per workgroup moves F alone
    shifted = [(n, tiles, T + n * 3.0) for n, tiles, T in exact]
    assert np.allclose(bench.fit_fixed_costs(shifted), (L, t, F + 3.0), atol=1e-9)
