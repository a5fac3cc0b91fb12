"""Shared test helpers: bf16 transfer, tolerance checks (no method arithmetic)."""

import numpy as np

# tolerances on bf16-input attention outputs (fp32 accumulation): max-abs and
# mean-abs error against the float64 oracle
O_MAX, O_MEAN = 2e-2, 2e-3
# gradients: the absolute bounds above; the mean error divided by the oracle
# tensor's RMS; and, where the sums of absolute terms are supplied, the
# elementwise rounding bound.  The backward rounds P and dS to bf16 (8
# significant bits, unit roundoff u = 2^-8) before the gradient contractions
# and takes delta from the bf16 rounding of its forward's O (whose weights
# were rounded to bf16 too), so to first order each element errs by at most
# u * (sum of |terms|) with the sums of oracle.attention_backward_magnitudes.
# The extra 1/8 covers what the first-order bound leaves out: second-order
# terms (about 3u = 1.2%), fp32 accumulation (at most 2^-24 of the sum of
# |terms| per accumulation step, a few thousand steps: about 6% of u), and the
# fp32 exponentials and LSE (about 1e-6 relative).
BF16_U = 2.0 ** -8
ROUNDING_SLACK = 1.0 + 1.0 / 8
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
    worst = None
    if bound is not None:
        bound = np.asarray(bound, dtype=np.float64)
        lim = ROUNDING_SLACK * BF16_U * bound + 1e-6 * np.abs(want).max()
        worst = float((err / lim).max())
    msg = (f"{what}: max abs {err.max():.3e} mean abs {err.mean():.3e} "
           f"max/rms {rel.max():.3e} mean/rms {rel.mean():.3e} (rms {rms:.3e})"
           + ("" if worst is None else f"; worst element at {worst:.3f} of (1+1/8) u sum|terms|"))
    print(f"[close] {msg}", flush=True)
    assert err.max() <= max_abs and err.mean() <= mean_abs, msg
    assert rel.mean() <= mean_rel, msg
    if worst is not None:
        assert worst <= 1.0, msg
    return float(rel.max()), float(rel.mean())


def oracle_ring_grads(q, ks, vs, do, q_pos, k_poss, order=None, q_start=None, scale=None,
                      chunks=None):
    """Oracle reference of one rank's ring: the forward over every chunk, then
    each chunk's gradients and their sums of absolute terms.  Delta comes from
    the oracle's own O; the forward-error term of the sums is summed over all
    chunks.  ``chunks`` limits the per-chunk gradients to those indices (the
    forward and dQ still cover every chunk).  Returns a dict with ``o, lse,
    delta, dq, mq`` and per-chunk lists ``dk, dv, mk, mv`` (None where not
    computed)."""
    import oracle
    n = len(ks)
    o, lse = oracle.ring_forward(q, list(ks), list(vs), q_pos, list(k_poss), order=order,
                                 q_start=q_start, scale=scale)
    delta = oracle.bwd_delta(o, do)
    c_all = sum(oracle.attention_abs_dp(q, ks[c], vs[c], do, lse, q_pos, k_poss[c], scale=scale,
                                        q_start=q_start) for c in range(n))
    out = {"o": o, "lse": lse, "delta": delta, "dq": 0.0, "mq": 0.0,
           "dk": [None] * n, "dv": [None] * n, "mk": [None] * n, "mv": [None] * n}
    for c in range(n):
        g = oracle.attention_backward(q, ks[c], vs[c], do, lse, delta, q_pos, k_poss[c],
                                      scale=scale, q_start=q_start)
        m = oracle.attention_backward_magnitudes(q, ks[c], vs[c], do, o, lse, q_pos, k_poss[c],
                                                 scale=scale, q_start=q_start, dp_abs=c_all)
        out["dq"] = out["dq"] + g[0]
        out["mq"] = out["mq"] + m[0]
        if chunks is None or c in chunks:
            out["dk"][c], out["dv"][c], out["mk"][c], out["mv"][c] = g[1], g[2], m[1], m[2]
    return out
