"""Shared test helpers: bf16 transfer, tolerance checks (no method arithmetic)."""

import numpy as np

# tolerances on bf16-input attention outputs (fp32 accumulation): max-abs and
# mean-abs error against the float64 oracle
O_MAX, O_MEAN = 2e-2, 2e-3
# gradients: the absolute bounds above; the mean error divided by the oracle
# tensor's RMS; and, where the sums of absolute terms are supplied, the
# elementwise rounding bound.  P and dS are rounded to bf16 (unit roundoff
# u = 2^-9) before the gradient contractions and delta comes from the bf16 O,
# so each element errs by at most about u * (sum of |terms|); the check allows
# twice that.
BF16_U = 2.0 ** -9
G_MEAN = 2e-3


def to_dev_bf16(bits, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_dev_i32(x, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)


def to_np(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_close_abs(got, want, max_abs=O_MAX, mean_abs=O_MEAN, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    fin = np.isfinite(want)
    assert np.array_equal(np.isneginf(got), np.isneginf(want)), f"{what}: -inf pattern differs"
    assert not np.isnan(got).any(), f"{what}: NaN"
    err = np.abs(got[fin] - want[fin]) if fin.any() else np.zeros(1)
    assert err.max() <= max_abs, f"{what}: max abs err {err.max():.3e} > {max_abs}"
    assert err.mean() <= mean_abs, f"{what}: mean abs err {err.mean():.3e} > {mean_abs}"
    return float(err.max()), float(err.mean())


def assert_close_rms(got, want, bound=None, mean_rel=G_MEAN, max_abs=O_MAX, mean_abs=O_MEAN,
                     what=""):
    """Gradient check: absolute bounds, RMS-relative mean, elementwise bound."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite"
    rms = float(np.sqrt(np.mean(want * want)))
    err = np.abs(got - want)
    rel = err / max(rms, 1e-30)
    msg = (f"{what}: max abs {err.max():.3e} mean abs {err.mean():.3e} "
           f"max/rms {rel.max():.3e} mean/rms {rel.mean():.3e} (rms {rms:.3e})")
    assert err.max() <= max_abs and err.mean() <= mean_abs, msg
    assert rel.mean() <= mean_rel, msg
    if bound is not None:
        bound = np.asarray(bound, dtype=np.float64)
        lim = 2 * BF16_U * bound + 1e-6 * np.abs(want).max()
        worst = float((err / lim).max())
        assert worst <= 1.0, f"{msg}; exceeds 2u*sum|terms| by x{worst:.2f}"
    return float(rel.max()), float(rel.mean())
