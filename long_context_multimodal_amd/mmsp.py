"""ctypes binding of ``libmmsp.so`` (the C-ABI in ``include/mmsp.h``).

Argument marshalling only: tensors are checked for dtype, device, layout and
shape, their device pointers and the current HIP stream are handed to the
library, and a nonzero status raises :class:`MMSPError`.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  torch is
used for device memory and streams.
"""

from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmmsp.so")

MMSP_OK = 0
STATUS_NAMES = {
    0: "MMSP_OK", -1: "MMSP_ERR_NULL", -2: "MMSP_ERR_SHAPE", -3: "MMSP_ERR_UNSUPPORTED",
    -4: "MMSP_ERR_DIVISIBILITY", -5: "MMSP_ERR_WORKSPACE", -6: "MMSP_ERR_HIP",
}
BALANCE_ZIGZAG, BALANCE_MODALITY = 0, 1
DTYPE_BF16, DTYPE_F32 = 0, 1
CAUSAL, ACCUMULATE = 1, 2
BWD_NO_DQ, BWD_NO_DKDV = 4, 8

# every symbol the header declares, with its ctypes signature
_VP, _I32, _I64, _U32, _F32, _SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                    ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t)
SIGNATURES = {
    "mmsp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mmsp_abi_version": (ctypes.c_int, []),
    "mmsp_device_info": (ctypes.c_int, [_I32, _VP, _VP, _VP]),
    "mmsp_shard_balance_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32]),
    "mmsp_shard_balance": (ctypes.c_int, [_VP, _I64, _I32, _I32, _I32, _VP, _VP, _VP, _SZ, _VP]),
    "mmsp_attn_fwd_chunk": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32,
                                           _F32, _U32, _VP, _VP, _VP]),
    "mmsp_lse_merge": (ctypes.c_int, [_VP, _VP, _VP, _VP, _I32, _I32, _I32, _VP, _VP]),
    "mmsp_attn_bwd_preprocess": (ctypes.c_int, [_VP, _VP, _I32, _I32, _I32, _VP, _VP, _VP]),
    "mmsp_attn_bwd_chunk": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32,
                                           _I32, _I32, _I32, _F32, _U32, _VP, _VP, _VP, _VP]),
    "mmsp_shard_balance_noalloc": (ctypes.c_int, [_VP, _I64, _I32, _I32, _I32, _VP, _VP, _VP]),
    "mmsp_shard_balance_packed": (ctypes.c_int, [_VP, _I32, _I64, _I32, _VP, _VP, _VP, _VP]),
    "mmsp_shard_gather": (ctypes.c_int, [_VP, _I64, _VP, _I64, _I64, _VP, _VP]),
    "mmsp_check_positions": (ctypes.c_int, [_VP, _VP, _I32, _VP, _VP]),
    "mmsp_shard_scatter": (ctypes.c_int, [_VP, _I64, _VP, _I64, _I64, _VP, _VP]),
    "mmsp_rope": (ctypes.c_int, [_VP, _VP, _I32, _VP, _I32, _I32, _I32, ctypes.c_double, _I32,
                                 _VP]),
    "mmsp_attn_fwd_chunk_packed": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _I32,
                                                  _I32, _I32, _I32, _I32, _F32, _U32, _VP, _VP,
                                                  _VP]),
    "mmsp_attn_bwd_chunk_packed": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                                  _VP, _SZ, _I32, _I32, _I32, _I32, _I32, _F32,
                                                  _U32, _VP, _VP, _VP, _VP]),
    "mmsp_attn_packed_plan_bytes": (_SZ, [_I32, _I32]),
    "mmsp_attn_packed_plan": (ctypes.c_int, [_VP, _VP, _VP, _I32, _I32, _VP, _SZ, _VP]),
    "mmsp_attn_packed_plans": (ctypes.c_int, [_VP, _VP, _VP, _I32, _I32, _I32, _VP, _SZ, _VP]),
    "mmsp_ring_forward": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32,
                                         _I32, _I32, _I32, _F32, _U32, _VP, _VP, _VP, _VP]),
    "mmsp_ring_backward": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32,
                                          _I32, _I32, _I32, _I32, _I32, _F32, _U32, _VP, _VP,
                                          _VP, _VP, _VP]),
}

_lib = None


class MMSPError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        name = STATUS_NAMES.get(code, str(code))
        msg = lib().mmsp_status_string(code).decode()
        super().__init__(f"{where}: {name} ({msg})")


def lib():
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m long_context_multimodal_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(code: int, where: str):
    if code != MMSP_OK:
        raise MMSPError(code, where)


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def device_info(device: int = 0):
    """``{"compute_units", "peak_clock_mhz", "l2_bytes"}`` of a device."""
    cu, clk, l2 = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().mmsp_device_info(device, ctypes.byref(cu), ctypes.byref(clk), ctypes.byref(l2)),
           "mmsp_device_info")
    return {"compute_units": cu.value, "peak_clock_mhz": clk.value / 1000.0,
            "l2_bytes": l2.value}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _on_current_device(t, name):
    """The work is enqueued on the current device's stream, so every tensor
    must live on that device."""
    import torch
    if t.device.type != "cuda":
        raise TypeError(f"{name}: expected a device tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name}: on {t.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}")


def _need(t, dtype, name, ndim=None):
    import torch
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    _on_current_device(t, name)
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")
    del torch


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _shape(t, shape, name):
    """The kernels trust the sizes they are given: every tensor they touch
    must have exactly the shape those sizes imply."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


# ---------------------------------------------------------------- a1
def shard_balance(n: int, n_ranks: int, mode: int = BALANCE_ZIGZAG, granularity: int = 0,
                  labels=None, with_inverse: bool = True, device="cuda"):
    """Rank-major shard permutation (int32[n]) and optionally its inverse."""
    import torch
    if labels is not None:
        _need(labels, torch.uint8, "labels", 1)
        if labels.numel() != n:
            raise ValueError("labels must have n entries")
    perm = torch.empty(n, dtype=torch.int32, device=device)
    inv = torch.empty(n, dtype=torch.int32, device=device) if with_inverse else None
    ws_bytes = lib().mmsp_shard_balance_workspace_bytes(n, n_ranks, mode, granularity)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=device) if ws_bytes else None
    _check(lib().mmsp_shard_balance(_ptr(labels), n, n_ranks, mode, granularity, _ptr(perm),
                                    _ptr(inv), _ptr(ws), ws_bytes, _stream()),
           "mmsp_shard_balance")
    return perm, inv


def shard_balance_noalloc(perm, n_ranks: int, mode: int = BALANCE_ZIGZAG, granularity: int = 0,
                          labels=None, inv=None):
    """``shard_balance`` into caller-given ``perm`` (and ``inv``), int32[n], with
    the library's own scratch (``mmsp_shard_balance_noalloc``): nothing is
    allocated."""
    import torch
    _need(perm, torch.int32, "perm", 1)
    n = perm.numel()
    _need(inv, torch.int32, "inv", 1)
    _shape(inv, (n,), "inv")
    _need(labels, torch.uint8, "labels", 1)
    _shape(labels, (n,), "labels")
    _check(lib().mmsp_shard_balance_noalloc(_ptr(labels), n, n_ranks, mode, granularity,
                                            _ptr(perm), _ptr(inv), _stream()),
           "mmsp_shard_balance_noalloc")
    return perm, inv


def shard_balance_packed(starts, n: int, n_ranks: int, with_inverse: bool = False,
                         with_token_start: bool = True):
    """Per-sample zigzag of packed samples (``starts`` int32[n_samples + 1] on
    the device).  Returns ``(perm, inv_perm or None, token_start or None)``."""
    import torch
    _need(starts, torch.int32, "starts", 1)
    device = starts.device
    perm = torch.empty(n, dtype=torch.int32, device=device)
    inv = torch.empty(n, dtype=torch.int32, device=device) if with_inverse else None
    first = torch.empty(n, dtype=torch.int32, device=device) if with_token_start else None
    _check(lib().mmsp_shard_balance_packed(_ptr(starts), starts.numel() - 1, n, n_ranks,
                                           _ptr(perm), _ptr(inv), _ptr(first), _stream()),
           "mmsp_shard_balance_packed")
    return perm, inv, first


CHECK_POSITIONS = os.environ.get("MMSP_CHECK_POSITIONS", "0") not in ("", "0")


def check_positions(pos, starts=None) -> int:
    """Number of violations of the position preconditions (strictly
    increasing ``pos``; ``starts`` non-decreasing, non-negative, not after
    ``pos``).  Synchronises the stream to read the count."""
    import torch
    _need(pos, torch.int32, "pos", 1)
    _need(starts, torch.int32, "starts", 1)
    if starts is not None and starts.numel() != pos.numel():
        raise ValueError("starts must have one entry per position")
    count = torch.empty(1, dtype=torch.int32, device=pos.device)
    _check(lib().mmsp_check_positions(_ptr(pos), _ptr(starts), pos.numel(), _ptr(count),
                                      _stream()), "mmsp_check_positions")
    return int(count.item())


def _debug_check(q_pos, k_pos, q_start):
    """With MMSP_CHECK_POSITIONS=1: refuse position arrays the kernels would
    read wrongly (checked on the device, one synchronisation per array)."""
    for name, p, st in (("q_pos", q_pos, q_start), ("k_pos", k_pos, None)):
        if p is not None:
            bad = check_positions(p, st)
            if bad:
                raise ValueError(f"{name}{'/q_start' if st is not None else ''}: "
                                 f"{bad} violations of the position preconditions")


def shard_gather(x, rows, out=None):
    """``out[i] = x[rows[i]]`` over the first dimension (zero rows where
    ``rows[i]`` is outside ``x``); ``rows`` int32 on the device."""
    import torch
    _need(rows, torch.int32, "rows", 1)
    _on_current_device(x, "x")
    if not x.is_contiguous() or x.dim() < 1:
        raise ValueError("x: expected a contiguous tensor of rows")
    shape = (rows.numel(),) + tuple(x.shape[1:])
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    _on_current_device(out, "out")
    if out.dtype != x.dtype or tuple(out.shape) != shape or not out.is_contiguous():
        raise ValueError(f"out: expected a contiguous {x.dtype} tensor of shape {shape}")
    row_bytes = math.prod(x.shape[1:]) * x.element_size()
    _check(lib().mmsp_shard_gather(_ptr(x), x.shape[0], _ptr(rows), rows.numel(), row_bytes,
                                   _ptr(out), _stream()), "mmsp_shard_gather")
    return out


def shard_scatter(x, rows, out):
    """``out[rows[i]] = x[i]`` over the first dimension (rows outside ``out``
    skipped; ``rows`` distinct)."""
    import torch
    _need(rows, torch.int32, "rows", 1)
    for t, n in ((x, "x"), (out, "out")):
        _on_current_device(t, n)
        if not t.is_contiguous() or t.dim() < 1:
            raise ValueError(f"{n}: expected a contiguous tensor of rows")
    if out.dtype != x.dtype or tuple(out.shape[1:]) != tuple(x.shape[1:]) or \
            rows.numel() != x.shape[0]:
        raise ValueError("x, rows and out disagree")
    row_bytes = math.prod(x.shape[1:]) * x.element_size()
    _check(lib().mmsp_shard_scatter(_ptr(x), x.shape[0], _ptr(rows), out.shape[0], row_bytes,
                                    _ptr(out), _stream()), "mmsp_shard_scatter")
    return out


# ---------------------------------------------------------------- a2
def packed_plan(q_pos, q_start, k_pos, plan=None):
    """Tile plan of the packed attention calls for these positions (int32
    tensor of ``mmsp_attn_packed_plan_bytes`` bytes, on the positions' device):
    every tile of the forward, dQ and dK/dV kernels listed heaviest first.
    Scheduling only: ``attn_fwd_chunk`` / ``attn_bwd_chunk`` give the same
    results with or without it.  ``plan`` may be given to reuse a buffer."""
    import torch
    _need(q_pos, torch.int32, "q_pos", 1)
    _need(q_start, torch.int32, "q_start", 1)
    _need(k_pos, torch.int32, "k_pos", 1)
    sq, sk = q_pos.numel(), k_pos.numel()
    if q_start.numel() != sq:
        raise ValueError("q_start must have sq entries")
    nbytes = lib().mmsp_attn_packed_plan_bytes(sq, sk)
    if nbytes == 0:
        raise ValueError("positions must not be empty")
    if plan is None:
        plan = torch.empty(nbytes // 4, dtype=torch.int32, device=q_pos.device)
    _need(plan, torch.int32, "plan", 1)
    _check(lib().mmsp_attn_packed_plan(_ptr(q_pos), _ptr(q_start), _ptr(k_pos), sq, sk,
                                       _ptr(plan), plan.numel() * 4, _stream()),
           "mmsp_attn_packed_plan")
    return plan


def packed_plans(q_pos, q_start, k_pos_all, n_chunks, plans=None):
    """Tile plans of ``n_chunks`` chunks in one launch: ``k_pos_all`` (int32)
    holds the chunks' key positions back to back, ``n_chunks * sk`` entries.
    Returns an int32 tensor ``[n_chunks, words]`` whose row c is chunk c's
    plan (as :func:`packed_plan` makes it); ``plans`` may be given to reuse a
    buffer of that shape."""
    import torch
    _need(q_pos, torch.int32, "q_pos", 1)
    _need(q_start, torch.int32, "q_start", 1)
    _need(k_pos_all, torch.int32, "k_pos_all", 1)
    sq = q_pos.numel()
    if q_start.numel() != sq:
        raise ValueError("q_start must have sq entries")
    if n_chunks < 1 or k_pos_all.numel() % n_chunks:
        raise ValueError("k_pos_all must hold n_chunks equal chunks")
    sk = k_pos_all.numel() // n_chunks
    nbytes = lib().mmsp_attn_packed_plan_bytes(sq, sk)
    if nbytes == 0:
        raise ValueError("positions must not be empty")
    if plans is None:
        plans = torch.empty((n_chunks, nbytes // 4), dtype=torch.int32, device=q_pos.device)
    _need(plans, torch.int32, "plans", 2)
    _shape(plans, (n_chunks, nbytes // 4), "plans")
    _check(lib().mmsp_attn_packed_plans(_ptr(q_pos), _ptr(q_start), _ptr(k_pos_all), n_chunks,
                                        sq, sk, _ptr(plans), plans.numel() * 4, _stream()),
           "mmsp_attn_packed_plans")
    return plans


def attn_fwd_chunk(q, k, v, q_pos=None, k_pos=None, scale=None, causal=True, o=None, lse=None,
                   accumulate=False, q_start=None, plan=None):
    """Attention of ``q[sq,hq,d]`` against one chunk ``k, v[sk,hkv,d]`` (bf16).

    Returns ``(o fp32[sq,hq,d], lse fp32[hq,sq])``; with ``accumulate`` the
    given ``(o, lse)`` are merged with this chunk's result in place.
    ``q_start`` (int32[sq], optional): first position of each query's packed
    sample (reset attention masks between samples; needs ``causal``).
    ``plan`` (optional, packed only): tile order from :func:`packed_plan`.
    """
    if plan is not None and q_start is None:
        raise ValueError("a tile plan applies to packed samples only")
    import torch
    _need(q, torch.bfloat16, "q", 3)
    _need(k, torch.bfloat16, "k", 3)
    _need(v, torch.bfloat16, "v", 3)
    sq, hq, d = q.shape
    sk, hkv, dk = k.shape
    if dk != d or tuple(v.shape) != (sk, hkv, d):
        raise ValueError("q/k/v shapes disagree")
    if causal:
        _need(q_pos, torch.int32, "q_pos", 1)
        _need(k_pos, torch.int32, "k_pos", 1)
        if q_pos.numel() != sq or k_pos.numel() != sk:
            raise ValueError("position arrays must match sq / sk")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if accumulate:
        if o is None or lse is None:
            raise ValueError("accumulate needs the running (o, lse)")
    if o is None:
        o = torch.empty((sq, hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((hq, sq), dtype=torch.float32, device=q.device)
    _need(o, torch.float32, "o", 3)
    _need(lse, torch.float32, "lse", 2)
    _shape(o, (sq, hq, d), "o")
    _shape(lse, (hq, sq), "lse")
    if CHECK_POSITIONS and causal:
        _debug_check(q_pos, k_pos, q_start)
    flags = (CAUSAL if causal else 0) | (ACCUMULATE if accumulate else 0)
    if q_start is not None:
        _need(q_start, torch.int32, "q_start", 1)
        if q_start.numel() != sq:
            raise ValueError("q_start must have sq entries")
        _need(plan, torch.int32, "plan", 1)
        _check(lib().mmsp_attn_fwd_chunk_packed(
            _ptr(q), _ptr(k), _ptr(v), _ptr(q_pos if causal else None), _ptr(q_start),
            _ptr(k_pos if causal else None), _ptr(plan), _nbytes(plan), sq, sk, hq, hkv, d,
            float(scale), flags, _ptr(o), _ptr(lse), _stream()), "mmsp_attn_fwd_chunk_packed")
        return o, lse
    _check(lib().mmsp_attn_fwd_chunk(_ptr(q), _ptr(k), _ptr(v), _ptr(q_pos if causal else None),
                                     _ptr(k_pos if causal else None), sq, sk, hq, hkv, d,
                                     float(scale), flags, _ptr(o), _ptr(lse), _stream()),
           "mmsp_attn_fwd_chunk")
    return o, lse


# ---------------------------------------------------------------- a3
def lse_merge(o_acc, lse_acc, o_part=None, lse_part=None, o_final=None):
    """Merge ``(o_part, lse_part)`` into ``(o_acc, lse_acc)`` in place.

    ``o_final`` (bf16, optional) receives the merged output rounded to bf16.
    """
    import torch
    _need(o_acc, torch.float32, "o_acc", 3)
    _need(lse_acc, torch.float32, "lse_acc", 2)
    _need(o_part, torch.float32, "o_part", 3)
    _need(lse_part, torch.float32, "lse_part", 2)
    _need(o_final, torch.bfloat16, "o_final", 3)
    sq, hq, d = o_acc.shape
    _shape(lse_acc, (hq, sq), "lse_acc")
    _shape(o_part, (sq, hq, d), "o_part")
    _shape(lse_part, (hq, sq), "lse_part")
    _shape(o_final, (sq, hq, d), "o_final")
    if (o_part is None) != (lse_part is None):
        raise ValueError("o_part and lse_part go together")
    _check(lib().mmsp_lse_merge(_ptr(o_acc), _ptr(lse_acc), _ptr(o_part), _ptr(lse_part), sq, hq,
                                d, _ptr(o_final), _stream()), "mmsp_lse_merge")
    return o_acc, lse_acc


# ---------------------------------------------------------------- a5
def attn_bwd_preprocess(o, dout, delta=None, dq_zero=None):
    """``delta[h, i] = sum_c dout[i,h,c] * o[i,h,c]`` (bf16 in, fp32 out).

    ``dq_zero`` (fp32 ``[sq,hq,d]``, optional) is zeroed in the same pass.
    """
    import torch
    _need(o, torch.bfloat16, "o", 3)
    _need(dout, torch.bfloat16, "dout", 3)
    _need(dq_zero, torch.float32, "dq_zero", 3)
    sq, hq, d = o.shape
    _shape(dout, (sq, hq, d), "dout")
    _shape(dq_zero, (sq, hq, d), "dq_zero")
    if delta is None:
        delta = torch.empty((hq, sq), dtype=torch.float32, device=o.device)
    _need(delta, torch.float32, "delta", 2)
    _shape(delta, (hq, sq), "delta")
    _check(lib().mmsp_attn_bwd_preprocess(_ptr(o), _ptr(dout), sq, hq, d, _ptr(delta),
                                          _ptr(dq_zero), _stream()),
           "mmsp_attn_bwd_preprocess")
    return delta


# ---------------------------------------------------------------- a6
def attn_bwd_chunk(q, k, v, dout, lse, delta, q_pos, k_pos, dq_acc, dk=None, dv=None,
                   scale=None, causal=True, accumulate=False, q_start=None, part="both",
                   plan=None):
    """Backward of one chunk: adds to ``dq_acc``; returns ``(dk, dv)`` fp32.
    ``q_start`` and ``plan`` as in :func:`attn_fwd_chunk`.  ``part`` = ``"dkdv"`` or ``"dq"``
    enqueues only that kernel (``dq_acc``, or ``dk``/``dv``, unused), so the
    two halves can run on two streams."""
    if part not in ("both", "dkdv", "dq"):
        raise ValueError("part must be 'both', 'dkdv' or 'dq'")
    if plan is not None and q_start is None:
        raise ValueError("a tile plan applies to packed samples only")
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _need(t, torch.bfloat16, n, 3)
    _need(lse, torch.float32, "lse", 2)
    _need(delta, torch.float32, "delta", 2)
    if part == "dkdv":
        dq_acc = None
    _need(dq_acc, torch.float32, "dq_acc", 3)
    sq, hq, d = q.shape
    sk, hkv, _ = k.shape
    _shape(k, (sk, hkv, d), "k")
    _shape(v, (sk, hkv, d), "v")
    _shape(dout, (sq, hq, d), "dout")
    _shape(lse, (hq, sq), "lse")
    _shape(delta, (hq, sq), "delta")
    _shape(dq_acc, (sq, hq, d), "dq_acc")
    if causal:
        _need(q_pos, torch.int32, "q_pos", 1)
        _need(k_pos, torch.int32, "k_pos", 1)
        if q_pos.numel() != sq or k_pos.numel() != sk:
            raise ValueError("position arrays must match sq / sk")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if part == "dq":
        dk = dv = None
    else:
        if dk is None:
            dk = torch.empty((sk, hkv, d), dtype=torch.float32, device=q.device)
        if dv is None:
            dv = torch.empty((sk, hkv, d), dtype=torch.float32, device=q.device)
    _need(dk, torch.float32, "dk", 3)
    _need(dv, torch.float32, "dv", 3)
    _shape(dk, (sk, hkv, d), "dk")
    _shape(dv, (sk, hkv, d), "dv")
    if CHECK_POSITIONS and causal:
        _debug_check(q_pos, k_pos, q_start)
    flags = (CAUSAL if causal else 0) | (ACCUMULATE if accumulate else 0)
    flags |= {"both": 0, "dkdv": BWD_NO_DQ, "dq": BWD_NO_DKDV}[part]
    if q_start is not None:
        _need(q_start, torch.int32, "q_start", 1)
        if q_start.numel() != sq:
            raise ValueError("q_start must have sq entries")
        _need(plan, torch.int32, "plan", 1)
        _check(lib().mmsp_attn_bwd_chunk_packed(
            _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta),
            _ptr(q_pos if causal else None), _ptr(q_start), _ptr(k_pos if causal else None),
            _ptr(plan), _nbytes(plan), sq, sk, hq, hkv, d, float(scale), flags, _ptr(dq_acc),
            _ptr(dk), _ptr(dv), _stream()), "mmsp_attn_bwd_chunk_packed")
        return dk, dv
    _check(lib().mmsp_attn_bwd_chunk(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                                     _ptr(delta), _ptr(q_pos if causal else None),
                                     _ptr(k_pos if causal else None), sq, sk, hq, hkv, d,
                                     float(scale), flags, _ptr(dq_acc), _ptr(dk), _ptr(dv),
                                     _stream()), "mmsp_attn_bwd_chunk")
    return dk, dv


# ---------------------------------------------------------------- a4 in the library
def _pointer_array(tensors):
    """Host array of the tensors' device pointers (kept alive by the caller)."""
    return (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])


def _ring_chunks(q, k_chunks, v_chunks, q_pos, k_pos_chunks, q_start, causal):
    """Check a ring's tensors; return (sq, hq, d, sk, hkv)."""
    import torch
    n = len(k_chunks)
    if n == 0 or len(v_chunks) != n or (causal and len(k_pos_chunks) != n):
        raise ValueError("one K, V (and, with the causal mask, position array) per chunk")
    _need(q, torch.bfloat16, "q", 3)
    sq, hq, d = q.shape
    _need(k_chunks[0], torch.bfloat16, "k[0]", 3)
    sk, hkv = k_chunks[0].shape[0], k_chunks[0].shape[1]
    for c in range(n):
        _need(k_chunks[c], torch.bfloat16, f"k[{c}]", 3)
        _need(v_chunks[c], torch.bfloat16, f"v[{c}]", 3)
        _shape(k_chunks[c], (sk, hkv, d), f"k[{c}]")
        _shape(v_chunks[c], (sk, hkv, d), f"v[{c}]")
        if causal:
            _need(k_pos_chunks[c], torch.int32, f"k_pos[{c}]", 1)
            _shape(k_pos_chunks[c], (sk,), f"k_pos[{c}]")
    if causal:
        _need(q_pos, torch.int32, "q_pos", 1)
        _shape(q_pos, (sq,), "q_pos")
    if q_start is not None:
        if not causal:
            raise ValueError("q_start needs the causal mask")
        _need(q_start, torch.int32, "q_start", 1)
        _shape(q_start, (sq,), "q_start")
    if CHECK_POSITIONS and causal:
        for c in range(n):
            _debug_check(q_pos, k_pos_chunks[c], q_start)
    return sq, hq, d, sk, hkv


def ring_forward_native(q, k_chunks, v_chunks, q_pos, k_pos_chunks, rank=0, scale=None,
                        causal=True, o=None, lse=None, o_final=None, q_start=None):
    """The whole ring forward in one library call (``mmsp_ring_forward``):
    chunk ``(rank - t) mod P`` at step ``t``, fused merge, bf16 output.
    Returns ``(o fp32, lse fp32, o_final bf16)`` like ``ring.ring_forward``."""
    import torch
    sq, hq, d, sk, hkv = _ring_chunks(q, k_chunks, v_chunks, q_pos, k_pos_chunks, q_start,
                                      causal)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty((sq, hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((hq, sq), dtype=torch.float32, device=q.device)
    if o_final is None:
        o_final = torch.empty((sq, hq, d), dtype=torch.bfloat16, device=q.device)
    _need(o, torch.float32, "o", 3)
    _need(lse, torch.float32, "lse", 2)
    _need(o_final, torch.bfloat16, "o_final", 3)
    _shape(o, (sq, hq, d), "o")
    _shape(lse, (hq, sq), "lse")
    _shape(o_final, (sq, hq, d), "o_final")
    ks, vs = _pointer_array(k_chunks), _pointer_array(v_chunks)
    kps = _pointer_array(k_pos_chunks) if causal else None
    _check(lib().mmsp_ring_forward(_ptr(q), ctypes.cast(ks, _VP), ctypes.cast(vs, _VP),
                                   _ptr(q_pos if causal else None),
                                   ctypes.cast(kps, _VP) if kps is not None else None,
                                   _ptr(q_start), len(k_chunks), rank, sq, sk, hq, hkv, d,
                                   float(scale), CAUSAL if causal else 0, _ptr(o), _ptr(lse),
                                   _ptr(o_final), _stream()), "mmsp_ring_forward")
    return o, lse, o_final


def ring_backward_native(q, k_chunks, v_chunks, dout, o_bf16, lse, q_pos, k_pos_chunks, rank=0,
                         scale=None, causal=True, dq=None, dks=None, dvs=None, delta=None,
                         q_start=None, accumulate=False):
    """The whole ring backward in one library call (``mmsp_ring_backward``):
    delta and zeroed dq, then every chunk in ring order.  Returns
    ``(dq, [dk_c], [dv_c])`` like ``ring.ring_backward``."""
    import torch
    sq, hq, d, sk, hkv = _ring_chunks(q, k_chunks, v_chunks, q_pos, k_pos_chunks, q_start,
                                      causal)
    n = len(k_chunks)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _need(dout, torch.bfloat16, "dout", 3)
    _need(o_bf16, torch.bfloat16, "o_bf16", 3)
    _need(lse, torch.float32, "lse", 2)
    _shape(dout, (sq, hq, d), "dout")
    _shape(o_bf16, (sq, hq, d), "o_bf16")
    _shape(lse, (hq, sq), "lse")
    if dq is None:
        dq = torch.empty((sq, hq, d), dtype=torch.float32, device=q.device)
    if delta is None:
        delta = torch.empty((hq, sq), dtype=torch.float32, device=q.device)
    if dks is None:
        dks = [torch.empty((sk, hkv, d), dtype=torch.float32, device=q.device) for _ in range(n)]
    if dvs is None:
        dvs = [torch.empty((sk, hkv, d), dtype=torch.float32, device=q.device) for _ in range(n)]
    _need(dq, torch.float32, "dq", 3)
    _need(delta, torch.float32, "delta", 2)
    _shape(dq, (sq, hq, d), "dq")
    _shape(delta, (hq, sq), "delta")
    if len(dks) != n or len(dvs) != n:
        raise ValueError("one dK and one dV per chunk")
    for c in range(n):
        _need(dks[c], torch.float32, f"dk[{c}]", 3)
        _need(dvs[c], torch.float32, f"dv[{c}]", 3)
        _shape(dks[c], (sk, hkv, d), f"dk[{c}]")
        _shape(dvs[c], (sk, hkv, d), f"dv[{c}]")
    ks, vs = _pointer_array(k_chunks), _pointer_array(v_chunks)
    kps = _pointer_array(k_pos_chunks) if causal else None
    dka, dva = _pointer_array(dks), _pointer_array(dvs)
    flags = (CAUSAL if causal else 0) | (ACCUMULATE if accumulate else 0)
    _check(lib().mmsp_ring_backward(_ptr(q), ctypes.cast(ks, _VP), ctypes.cast(vs, _VP),
                                    _ptr(dout), _ptr(o_bf16), _ptr(lse),
                                    _ptr(q_pos if causal else None),
                                    ctypes.cast(kps, _VP) if kps is not None else None,
                                    _ptr(q_start), n, rank, sq, sk, hq, hkv, d, float(scale),
                                    flags, _ptr(delta), _ptr(dq), ctypes.cast(dka, _VP),
                                    ctypes.cast(dva, _VP), _stream()), "mmsp_ring_backward")
    return dq, dks, dvs


# ---------------------------------------------------------------- rotary embedding
def rope(x, pos, theta: float = 1.0e7, inverse: bool = False, out=None):
    """Rotate ``x[s,h,d]`` (bf16 or fp32) at global positions ``pos`` (int32[s]).

    Returns ``out`` (a new tensor unless given; ``out=x`` rotates in place).
    """
    import torch
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("rope: x must be bf16 or fp32")
    _need(x, x.dtype, "x", 3)
    _need(pos, torch.int32, "pos", 1)
    s, h, d = x.shape
    if pos.numel() != s:
        raise ValueError("pos must have s entries")
    if out is None:
        out = torch.empty_like(x)
    _need(out, x.dtype, "out", 3)
    _shape(out, (s, h, d), "out")
    dtype = DTYPE_BF16 if x.dtype == torch.bfloat16 else DTYPE_F32
    _check(lib().mmsp_rope(_ptr(x), _ptr(out), dtype, _ptr(pos), s, h, d, float(theta),
                           1 if inverse else 0, _stream()), "mmsp_rope")
    return out
