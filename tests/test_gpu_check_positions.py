"""The device check of the position preconditions counts exactly the
violations a host count finds, and the binding's debug mode refuses bad
arrays before launching attention."""

import numpy as np
import pytest

from tests.helpers import to_dev_i32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mm():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from long_context_multimodal_amd import mmsp
    mmsp.lib()
    return mmsp, torch


def _host_count(pos, starts=None):
    bad = int((np.diff(pos) <= 0).sum())
    if starts is not None:
        bad += int(((starts > pos) | (starts < 0)).sum()) + int((np.diff(starts) < 0).sum())
    return bad


@pytest.mark.parametrize("n", [1, 5, 1000, 300001])
def test_counts_match_host(mm, n):
    mmsp, _ = mm
    rng = np.random.default_rng(n)
    pos = np.sort(rng.choice(4 * n + 8, n, replace=False)).astype(np.int32)
    starts = np.minimum(pos, (pos // 97) * 97).astype(np.int32)
    assert mmsp.check_positions(to_dev_i32(pos)) == 0
    assert mmsp.check_positions(to_dev_i32(pos), to_dev_i32(starts)) == 0
    if n > 2:
        bad_pos = pos.copy()
        idx = rng.choice(np.arange(1, n), size=min(n - 1, 7), replace=False)
        bad_pos[idx] = bad_pos[idx - 1]  # repeats
        bad_st = starts.copy()
        bad_st[rng.choice(n, 3, replace=False)] = pos.max() + 1
        assert mmsp.check_positions(to_dev_i32(bad_pos)) == _host_count(bad_pos)
        assert (mmsp.check_positions(to_dev_i32(pos), to_dev_i32(bad_st))
                == _host_count(pos, bad_st))


def test_debug_mode_refuses_bad_positions(mm, monkeypatch):
    mmsp, torch = mm
    monkeypatch.setattr(mmsp, "CHECK_POSITIONS", True)
    q = torch.zeros(64, 2, 64, dtype=torch.bfloat16, device="cuda")
    good = to_dev_i32(np.arange(64, dtype=np.int32))
    bad = to_dev_i32(np.r_[np.arange(32), np.arange(32)].astype(np.int32))
    mmsp.attn_fwd_chunk(q, q, q, good, good)  # passes the check
    with pytest.raises(ValueError):
        mmsp.attn_fwd_chunk(q, q, q, good, bad)
    with pytest.raises(ValueError):
        mmsp.attn_fwd_chunk(q, q, q, bad, good)
    dq = torch.zeros(64, 2, 64, dtype=torch.float32, device="cuda")
    stats = torch.zeros(2, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        mmsp.attn_bwd_chunk(q, q, q, q, stats, stats, bad, good, dq)
    torch.cuda.synchronize()
