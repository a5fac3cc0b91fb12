"""Throughput of one rank's MM-SP chunked causal attention on one MI355X.

One step is one pass of the whole per-rank hot path over one batch of
synthetic input: shard balance (positions of every rank), the forward over all
KV chunks in ring order with the LSE merge fused into each chunk's epilogue,
the bf16 output, the backward preprocess and the backward over all chunks.
Inputs are resident in HBM before the timed region starts.

Prints ONE JSON line.  ``value`` is forward+backward TFLOP/s of the step
(algorithmic FLOPs over visible (q, k) pairs only: 4*d per pair and query head
forward, 10*d backward); the forward alone is reported beside it.  The
``roofline`` object covers the dominant kernel (per-launch HIP events on the
launch stream); ``cpu_baseline`` times the float64 oracle on a bounded sample
(the first few query heads of the same workload) on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from long_context_multimodal_amd.workloads import WORKLOADS, TRAIN  # noqa: E402

METRIC = "causal attn TFLOP/s per rank shard (fwd, fwd+bwd); % of MI355X bf16 MFMA peak"
# MI355X dense bf16 MFMA peak: 256 CUs x 4096 FLOP/clk/CU x 2.4 GHz (published 2.5 PFLOP/s)
PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
PEAK_HBM_GBS = 8000.0
# sources whose text decides each kernel's memory traffic (the kernel and the
# shared tile loaders); a stored counter reading is used only while they match
KERNEL_SRC = {
    "attn_bwd_chunk": ("long_context_multimodal_amd/csrc/attn_bwd.hip",
                       "long_context_multimodal_amd/csrc/common.h"),
    "attn_fwd_chunk": ("long_context_multimodal_amd/csrc/attn_fwd.hip",
                       "long_context_multimodal_amd/csrc/common.h"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kernels_hbm_traffic_zigzag_p8_shard8192_h32_d128_fwd_bwd.txt")
# oracle work timed for the CPU baseline, at most (about 30 s at 0.1 TFLOP/s)
CPU_BASELINE_FLOP_BUDGET = 3.0e12


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class LaunchTimer:
    """HIP events around every chunk launch on the current (launch) stream."""

    def __init__(self):
        import torch
        self.torch = torch
        self.open = {}
        self.done = {"fwd": [], "bwd": [], "rope": []}
        self.enabled = False

    def start(self, kind, chunk):
        if not self.enabled:
            return
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.open[(kind, chunk)] = e

    def stop(self, kind, chunk):
        if not self.enabled:
            return
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.done[kind].append((chunk, self.open.pop((kind, chunk)), e))

    def summary(self, kind):
        ms = [(c, a.elapsed_time(b)) for c, a, b in self.done[kind]]
        return ms


def rank_positions(perm, w, rank):
    shard = w.shard
    return perm[rank * shard:(rank + 1) * shard]


def build_inputs(w, device):
    """Seeded synthetic tensors of the workload, moved to HBM."""
    import torch
    t0 = time.time()

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(device)

    qb, _ = w.q()
    q = dev(qb)
    del qb
    kb, _ = w.k()
    ks = [dev(kb[c]) for c in range(w.n_chunks)]
    del kb
    vb, _ = w.v()
    vs = [dev(vb[c]) for c in range(w.n_chunks)]
    del vb
    dout = None
    if w.backward:
        gb, _ = w.do()
        dout = dev(gb)
        del gb
    labels = torch.from_numpy(w.labels()).to(device)
    log(f"[bench] inputs of {w.name} generated and resident in {time.time() - t0:.1f}s")
    return q, ks, vs, dout, labels


def visible_pairs_per_chunk(w, perm_np, rank, first_np=None):
    """Visible (q, k) pairs per query head for every chunk (host, from positions;
    with packed samples a key must also lie at or after its query's sample start)."""
    qp = rank_positions(perm_np, w, rank)
    qs = rank_positions(first_np, w, rank) if first_np is not None else None
    out = []
    for c in range(w.n_chunks):
        kp = np.sort(perm_np[c * w.chunk:(c + 1) * w.chunk])
        n = np.searchsorted(kp, qp, side="right")
        if qs is not None:
            n = n - np.searchsorted(kp, qs, side="left")
        out.append(int(np.maximum(n, 0).sum()))
    return out


def source_sha(paths):
    """Hash of the code of the given sources: comments and whitespace are
    dropped, so a stored counter reading stays valid across comment edits and
    goes stale on any change to the code itself."""
    h = hashlib.sha256()
    for path in paths:
        text = open(os.path.join(ROOT, path), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on this workload with the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    sha = source_sha(KERNEL_SRC[kernel])
    for line in open(TRAFFIC_FILE):
        if not line.startswith(kernel + " "):
            continue
        kv = dict(tok.split("=", 1) for tok in line.split()[1:] if "=" in tok)
        if kv.get("workload") == workload and kv.get("src_sha") == sha:
            return float(kv["hbm_bytes_per_launch"])
    return None


def cpu_baseline(w, rank, perm_np, first_np=None, full=False):
    """The oracle, as it stands, on a few query heads of the workload (a
    bounded sample), or with ``full`` on every head and row, one group of
    heads at a time."""
    import oracle
    from threadpoolctl import threadpool_info
    t_gen = time.time()
    _, qv = w.q()
    _, kv = w.k()
    _, vv = w.v()
    gv = w.do()[1] if w.backward else None
    # whole GQA groups (contiguous query heads and the KV heads they read)
    g = w.hq // w.hkv
    target = 4 if w.backward else 8
    nkv = max(1, min(w.hkv, round(target / g)))
    nh = nkv * g
    qp = rank_positions(perm_np, w, rank)
    qs_all = rank_positions(first_np, w, rank) if first_np is not None else None
    kps = [perm_np[c * w.chunk:(c + 1) * w.chunk] for c in range(w.n_chunks)]
    order = [(rank - t) % w.n_chunks for t in range(w.n_chunks)]
    per_pair = (4 + (10 if w.backward else 0)) * w.d * nh
    # all rows when that is at most ~30 s of oracle work, else a seeded random
    # subset of query rows (each row's work is counted exactly)
    rows = None
    pairs_all = sum(visible_pairs_per_chunk(w, perm_np, rank, first_np))
    flops_all = per_pair * pairs_all
    if flops_all > CPU_BASELINE_FLOP_BUDGET and not full:
        n_rows = max(64, int(w.shard * CPU_BASELINE_FLOP_BUDGET / flops_all))
        rows = np.sort(np.random.default_rng(0).choice(w.shard, n_rows, replace=False))
    qr = qp if rows is None else qp[rows]
    qsr = None if qs_all is None else (qs_all if rows is None else qs_all[rows])
    log(f"[bench] cpu_baseline inputs ready in {time.time() - t_gen:.1f}s")
    groups = range(0, w.hkv, nkv) if full else [0]
    t_fwd = t_bwd = 0.0
    for kv0 in groups:
        h0 = kv0 * g
        q1 = np.ascontiguousarray(qv[:, h0:h0 + nh, :])
        k1 = [np.ascontiguousarray(kv[c][:, kv0:kv0 + nkv, :]) for c in range(w.n_chunks)]
        v1 = [np.ascontiguousarray(vv[c][:, kv0:kv0 + nkv, :]) for c in range(w.n_chunks)]
        g1 = np.ascontiguousarray(gv[:, h0:h0 + nh, :]) if gv is not None else None
        t0 = time.time()
        o, lse = oracle.ring_forward(q1, k1, v1, qp, kps, order=order, rows=rows, q_start=qs_all)
        t_fwd += time.time() - t0
        if g1 is not None:
            t1 = time.time()
            g1r = g1 if rows is None else g1[rows]
            q1r = q1 if rows is None else q1[rows]
            delta = oracle.bwd_delta(o, g1r)
            for c in order:
                oracle.attention_backward(q1r, k1[c], v1[c], g1r, lse, delta, qr, kps[c],
                                          q_start=qsr)
            t_bwd += time.time() - t1
        if full:
            log(f"[bench] cpu_baseline heads {h0}-{h0 + nh - 1}: fwd {t_fwd:.1f}s bwd {t_bwd:.1f}s")
    pairs = 0
    for c in range(w.n_chunks):
        kc = np.sort(kps[c])
        n_vis = np.searchsorted(kc, qr, side="right")
        if qsr is not None:
            n_vis = n_vis - np.searchsorted(kc, qsr, side="left")
        pairs += int(np.maximum(n_vis, 0).sum())
    flops = per_pair * pairs * len(groups)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    elapsed = t_fwd + t_bwd
    heads = f"all {w.hq} query heads" if full else f"query heads 0-{nh - 1} of {w.hq}"
    return {
        "value": round(flops / elapsed / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{heads}, "
                   + (f"all {w.shard} query rows" if rows is None else
                      f"{len(rows)} seeded random query rows of {w.shard}")
                   + f" ({flops / (per_pair / nh * w.hq) / pairs_all:.4f}"
                   f" of the step's FLOPs), all {w.n_chunks} chunks, "
                   f"forward{' + backward' if w.backward else ''}; "
                   f"fwd {t_fwd:.1f}s bwd {t_bwd:.1f}s; host affinity "
                   f"{len(os.sched_getaffinity(0))} cpus, BLAS threads {threads}"),
    }


def graph_replay(torch, step, outputs, steps):
    """Capture one step into a HIP graph and replay it.

    The graph holds the same kernels as the eager step, with the host's
    per-launch work (argument checks, marshalling, launch calls) done once at
    capture.  Before each checked replay the outputs are cleared eagerly, so a
    replay that did nothing could not match; every replay must equal the eager
    step bit for bit (the kernels are deterministic: no atomics)."""
    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in outputs]
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    match = True
    for _ in range(3):
        for t in outputs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        match = match and all(torch.equal(a, b) for a, b in zip(outputs, want))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(steps):
        graph.replay()
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / steps, match


def sdpa_context(torch, w, iters, device):
    """PyTorch-ROCm's own flash attention (forced; no fallback to the
    batched-matmul path) on one unmasked [1, hq, chunk, d] attention: the
    library a user would otherwise call, timed for comparison only."""
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    B, H, S, D = 1, w.hq, w.chunk, w.d
    if w.hkv != w.hq:
        return {"skipped": "the flash backend is timed on equal query and KV heads only"}
    try:
        q, k, v, g = (torch.randn(B, H, S, D, device=device, dtype=torch.bfloat16)
                      for _ in range(4))
        for t in (q, k, v):
            t.requires_grad_(True)
        flop = 4.0 * D * S * S * B * H
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            for _ in range(2):
                F.scaled_dot_product_attention(q, k, v).backward(g)
            torch.cuda.synchronize()
            ev[0].record()
            for _ in range(iters):
                F.scaled_dot_product_attention(q, k, v)
            ev[1].record()
            for _ in range(iters):
                F.scaled_dot_product_attention(q, k, v).backward(g)
            ev[2].record()
            torch.cuda.synchronize()
        fwd_ms = ev[0].elapsed_time(ev[1]) / iters
        fb_ms = ev[1].elapsed_time(ev[2]) / iters
        return {"what": f"torch.nn.functional.scaled_dot_product_attention, flash backend, "
                        f"[{B}, {H}, {S}, {D}] bf16, no mask",
                "torch": torch.__version__,
                "fwd_ms": round(fwd_ms, 4), "fwd_tflops": round(flop / fwd_ms / 1e9, 1),
                "bwd_ms": round(fb_ms - fwd_ms, 4),
                "bwd_tflops": round(2.5 * flop / (fb_ms - fwd_ms) / 1e9, 1)}
    except Exception as e:  # the backend may be missing on a build: context only
        return {"skipped": f"{type(e).__name__}: {str(e)[:200]}"}


def gemm_context(torch, iters, device, n=8192):
    """A library bf16 GEMM (torch.matmul, n x n x n, fp32 accumulate) run back
    to back: how much of the nominal MFMA peak a plain dense contraction
    sustains on the box (its clock under load is in the clock counters),
    timed for comparison only."""
    try:
        a = torch.randn(n, n, device=device, dtype=torch.bfloat16)
        b = torch.randn(n, n, device=device, dtype=torch.bfloat16)
        c = torch.empty(n, n, device=device, dtype=torch.bfloat16)
        reps = max(iters, 50)
        for _ in range(5):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            torch.matmul(a, b, out=c)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        return {"what": f"torch.matmul bf16 [{n}, {n}] x [{n}, {n}], {reps} calls back to back",
                "torch": torch.__version__, "ms": round(ms, 4),
                "tflops": round(2.0 * n ** 3 / ms / 1e9, 1),
                "pct_of_peak": round(100 * 2.0 * n ** 3 / ms / 1e9 / PEAK_BF16_TFLOPS, 2)}
    except Exception as e:  # context only
        return {"skipped": f"{type(e).__name__}: {str(e)[:200]}"}


def fit_fixed_costs(points):
    """Least-squares fit of T = L + n * (tiles * t + F) to ``(n, tiles, T)``
    points (n workgroups per slot, each walking ``tiles`` inner tiles):
    returns ``(L, t, F)``, the cost per launch, per inner tile and slot, and
    per workgroup."""
    a = np.array([[1.0, n * tiles, n] for n, tiles, _ in points])
    y = np.array([float(t) for *_, t in points])
    return tuple(float(x) for x in np.linalg.lstsq(a, y, rcond=None)[0])


def fixed_cost_sweep(torch, mmsp, device, batch=8, reps=3):
    """Fixed costs of the three attention kernels, per launch and per
    workgroup.  Each kernel runs back to back on inputs where every query sees
    every key (32 heads, d = 128, causal positions with all keys earlier), with
    the inner tiles a workgroup walks and the workgroups per slot varied; a
    least-squares fit of T = L + n * (tiles * t + F) gives L (per launch), t
    (per inner tile and slot) and F (per workgroup).  A slot is one workgroup
    place: one per CU for the forward, two for the backward kernels."""
    h, d = 32, 128
    cus = mmsp.device_info(0)["compute_units"]
    gen = torch.Generator(device="cpu").manual_seed(11)
    big = [torch.randn((8192, h, d), generator=gen).to(torch.bfloat16).to(device)
           for _ in range(4)]

    def timed(call):
        call()
        ts = []
        for _ in range(reps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            for _ in range(batch):
                call()
            ev[1].record()
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]) * 1000.0 / batch)
        return sorted(ts)[len(ts) // 2]

    def inputs(sq, sk):
        qp = (1 << 20) + torch.arange(sq, dtype=torch.int32, device=device)
        kp = torch.arange(sk, dtype=torch.int32, device=device)
        return (big[0][:sq], big[1][:sk], big[2][:sk], big[3][:sq], qp, kp)

    def fwd(sq, sk):
        q, k, v, _, qp, kp = inputs(sq, sk)
        o = torch.zeros((sq, h, d), dtype=torch.float32, device=device)
        lse = torch.zeros((h, sq), dtype=torch.float32, device=device)
        return timed(lambda: mmsp.attn_fwd_chunk(q, k, v, qp, kp, o=o, lse=lse, accumulate=True))

    def bwd(part, sq, sk):
        q, k, v, do, qp, kp = inputs(sq, sk)
        lse = torch.full((h, sq), 12.0, dtype=torch.float32, device=device)
        delta = torch.zeros((h, sq), dtype=torch.float32, device=device)
        dq = torch.zeros((sq, h, d), dtype=torch.float32, device=device)
        dk = torch.empty((sk, h, d), dtype=torch.float32, device=device)
        dv = torch.empty((sk, h, d), dtype=torch.float32, device=device)
        return timed(lambda: mmsp.attn_bwd_chunk(q, k, v, do, lse, delta, qp, kp, dq, dk, dv,
                                                 part=part))

    sizes = (1024, 2048, 4096, 8192)
    runs = {
        # kernel: (slots, [(sq, sk)], inner tiles a workgroup walks, workgroups, timed call)
        "attn_fwd_kernel": (cus, [(sq, sk) for sq in (2048, 4096, 8192) for sk in sizes],
                            lambda sq, sk: sk // 64, lambda sq, sk: sq // 256 * h,
                            lambda sq, sk: fwd(sq, sk)),
        "attn_bwd_dkdv_kernel": (2 * cus, [(sq, sk) for sk in (2048, 4096, 8192) for sq in sizes],
                                 lambda sq, sk: sq // 32, lambda sq, sk: sk // 128 * h,
                                 lambda sq, sk: bwd("dkdv", sq, sk)),
        "attn_bwd_dq_kernel": (2 * cus, [(sq, sk) for sq in (2048, 4096, 8192) for sk in sizes],
                               lambda sq, sk: sk // 64, lambda sq, sk: sq // 128 * h,
                               lambda sq, sk: bwd("dq", sq, sk)),
    }
    out = {"what": "unmasked chunks, 32 heads, d = 128, launches back to back; "
                   "T = L + n * (tiles * t + F), n = workgroups per slot", "kernels": {}}
    for name, (slots, shapes, tiles_of, wgs_of, run) in runs.items():
        rows, points = [], []
        for sq, sk in shapes:
            us = run(sq, sk)
            n, tiles = wgs_of(sq, sk) / slots, tiles_of(sq, sk)
            points.append((n, tiles, us))
            rows.append({"sq": sq, "sk": sk, "workgroups_per_slot": n, "tiles": tiles,
                         "us": round(us, 1)})
        sol = fit_fixed_costs(points)
        for r, (n, tiles, _) in zip(rows, points):
            r["model_us"] = round(sol[0] + n * (tiles * sol[1] + sol[2]), 1)
        out["kernels"][name] = {"slots": slots, "L_us": round(float(sol[0]), 1),
                                "t_us_per_tile": round(float(sol[1]), 3),
                                "F_us_per_workgroup": round(float(sol[2]), 1),
                                "F_in_tiles": round(float(sol[2] / sol[1]), 1), "runs": rows}
    return out


def device_record(torch, mmsp):
    """What the run was on: the peak the roofline uses is the published one
    (2.4 GHz); the clock the runtime reports and the one reached under load
    (see the clock counters) can differ."""
    props = torch.cuda.get_device_properties(0)
    info = mmsp.device_info(0)
    return {"name": props.name, "arch": props.gcnArchName,
            "compute_units": info["compute_units"],
            "peak_clock_mhz": info["peak_clock_mhz"],
            "bf16_peak_at_that_clock_tflops": round(
                info["compute_units"] * 4096 * info["peak_clock_mhz"] * 1e6 / 1e12, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=TRAIN.name, choices=sorted(WORKLOADS))
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--unfused", action="store_true", help="separate merge pass per chunk")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the oracle on the whole workload (every head and row, one group of "
                         "heads at a time) instead of the bounded sample; minutes of CPU work")
    ap.add_argument("--rope-theta", type=float, default=None,
                    help="rotate Q and every K chunk at their global positions with this rotary "
                         "base before the ring and rotate dQ/dK back after the backward "
                         "(one memory-bound pass each; the long-context stages use 1e7)")
    ap.add_argument("--ring-copy", action="store_true",
                    help="every KV chunk after the rank's own arrives by a device-to-device "
                         "copy on a second stream while the previous chunk is computed (dK/dV "
                         "copied out likewise); also times the resident ring and the copies "
                         "alone and reports the overlap loss")
    ap.add_argument("--gather", action="store_true",
                    help="also time moving the whole token stream ([N][hq][d] bf16) into the "
                         "balanced rank-major order (done once at the model input, so reported "
                         "on its own, not in the step)")
    ap.add_argument("--sdpa-context", action="store_true",
                    help="also time PyTorch's scaled_dot_product_attention (flash backend only) "
                         "on one full, unmasked chunk-sized attention [1, hq, chunk, d], forward "
                         "and forward+backward, as third-party context (not the product path)")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one step into a HIP graph and time its replays (resident "
                         "chunks only); replays are checked bit for bit against the eager step")
    ap.add_argument("--native-ring", action="store_true",
                    help="also time the step with the ring loop in the library (mmsp_ring_forward "
                         "/ mmsp_ring_backward) and check its outputs against the Python driver's")
    ap.add_argument("--gemm-context", action="store_true",
                    help="also time a library bf16 GEMM (torch.matmul, 8192^3) back to back: the dense "
                         "MFMA rate the box sustains, for comparison only")
    ap.add_argument("--no-plan", action="store_true",
                    help="packed samples: keep the kernels' built-in tile order instead of the "
                         "work-ordered tile plan made each step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device-to-device copy (HBM counter calibration)")
    ap.add_argument("--fixed-cost", action="store_true",
                    help="time the attention kernels over workgroup lengths and counts and fit "
                         "their fixed costs per launch and per workgroup (one JSON object)")
    args = ap.parse_args()
    if (args.graph or args.native_ring) and (args.ring_copy or args.rope_theta):
        print("--graph and --native-ring run the resident-chunk step without rotary passes; they "
              "do not combine with --ring-copy or --rope-theta", file=sys.stderr)
        sys.exit(2)
    if args.native_ring and args.unfused:
        print("--native-ring runs the fused merge; it does not combine with --unfused",
              file=sys.stderr)
        sys.exit(2)
    if args.graph and args.ring_copy:
        print("--graph captures the resident-chunk step; it does not combine with --ring-copy",
              file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the ring (one rank); --gpus {args.gpus} is "
              "not supported: run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_multimodal_amd import mmsp, ring

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        n = 1 << 30  # bytes read and written once per copy
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 3}))
        return
    if args.fixed_cost:
        mmsp.lib()
        print(json.dumps(fixed_cost_sweep(torch, mmsp, torch.device("cuda:0"))))
        return
    mmsp.lib()
    device = torch.device("cuda:0")
    w = WORKLOADS[args.workload]
    rank = args.rank
    q, ks, vs, dout, labels = build_inputs(w, device)

    n = w.n_tokens
    mode = {"zigzag": mmsp.BALANCE_ZIGZAG, "modality": mmsp.BALANCE_MODALITY}.get(w.layout)

    # buffers reused by every step
    sq, hq, d = q.shape
    o = torch.empty((sq, hq, d), dtype=torch.float32, device=device)
    lse = torch.empty((hq, sq), dtype=torch.float32, device=device)
    o16 = torch.empty((sq, hq, d), dtype=torch.bfloat16, device=device)
    delta = torch.empty((hq, sq), dtype=torch.float32, device=device)
    dq = torch.empty((sq, hq, d), dtype=torch.float32, device=device) if w.backward else None
    dks = [torch.empty(k.shape, dtype=torch.float32, device=device) for k in ks] \
        if w.backward else None
    dvs = [torch.empty(k.shape, dtype=torch.float32, device=device) for k in ks] \
        if w.backward else None
    contiguous_pos = torch.arange(n, dtype=torch.int32, device=device)
    starts = (torch.from_numpy(w.sample_starts()).to(device) if w.layout == "packed" else None)
    timer = LaunchTimer()
    rx = ring.ChunkReceiver(ks[0], vs[0]) if args.ring_copy else None
    theta = args.rope_theta
    q_rot = torch.empty_like(q) if theta else None
    ks_rot = [torch.empty_like(t) for t in ks] if theta else None

    def rope_in(qp, kps):
        """Rotate Q and the K chunks at their positions (each K chunk once: its
        owner rotates it before it travels)."""
        timer.start("rope", "in")
        mmsp.rope(q, qp, theta, out=q_rot)
        for c in range(w.n_chunks):
            mmsp.rope(ks[c], kps[c], theta, out=ks_rot[c])
        timer.stop("rope", "in")
        return q_rot, ks_rot

    def rope_out(qp, kps):
        """Gradients with respect to the unrotated Q and K."""
        timer.start("rope", "out")
        mmsp.rope(dq, qp, theta, inverse=True, out=dq)
        for c in range(w.n_chunks):
            mmsp.rope(dks[c], kps[c], theta, inverse=True, out=dks[c])
        timer.stop("rope", "out")
    dk_sent = [torch.empty_like(t) for t in dks] if (rx is not None and w.backward) else None
    dv_sent = [torch.empty_like(t) for t in dvs] if (rx is not None and w.backward) else None

    def balance():
        """Shard balance on the GPU: (perm, token sample starts or None, this rank's starts)."""
        first = qs = None
        if w.layout == "packed":  # every packed sample zigzagged on its own
            perm, _, first = mmsp.shard_balance_packed(starts, n, w.n_ranks)
            qs = first[rank * w.shard:(rank + 1) * w.shard]
        elif mode is None:  # single rank holding every position, contiguous chunks
            perm = contiguous_pos
        else:
            perm, _ = mmsp.shard_balance(n, w.n_ranks, mode, w.granularity,
                                         labels=labels if mode == mmsp.BALANCE_MODALITY else None,
                                         with_inverse=False)
        return perm, first, qs

    plan_bufs = [None]

    def tile_plans(qp, qs, kps):
        """Work-ordered tile plans of the step's chunks (packed samples): one
        per chunk, shared by the forward and the backward, buffers reused."""
        if qs is None:
            return None
        if args.no_plan:
            return [None] * len(kps)
        plan_bufs[0] = ring.packed_plans(qp, qs, kps, plans=plan_bufs[0])
        return plan_bufs[0]

    def step(received=args.ring_copy):
        perm, first, qs = balance()
        qp = perm[rank * w.shard:(rank + 1) * w.shard]
        kps = [perm[c * w.chunk:(c + 1) * w.chunk] for c in range(w.n_chunks)]
        plans = tile_plans(qp, qs, kps)
        qq, kk = rope_in(qp, kps) if theta else (q, ks)
        if received:
            ring.ring_forward_received(qq, kk, vs, qp, kps, rx, rank=rank, fused=not args.unfused,
                                       o=o, lse=lse, o_final=o16, timer=timer, q_start=qs,
                                       plans=plans)
            if w.backward:
                ring.ring_backward_received(qq, kk, vs, dout, o16, lse, qp, kps, rx, rank=rank,
                                            dq=dq, dks=dks, dvs=dvs, dk_sent=dk_sent,
                                            dv_sent=dv_sent, delta=delta, timer=timer,
                                            q_start=qs, plans=plans)
        else:
            ring.ring_forward(qq, kk, vs, qp, kps, rank=rank, fused=not args.unfused, o=o,
                              lse=lse, o_final=o16, timer=timer, q_start=qs, plans=plans)
            if w.backward:
                ring.ring_backward(qq, kk, vs, dout, o16, lse, qp, kps, rank=rank, dq=dq, dks=dks,
                                   dvs=dvs, delta=delta, timer=timer, q_start=qs, plans=plans)
        if theta and w.backward:
            rope_out(qp, kps)
        return perm, first

    def copies_only():
        """The copies one received step enqueues, without the compute."""
        order = ring.ring_order(rank, w.n_chunks)
        rx.start()
        for _ in range(2 if w.backward else 1):
            for t in range(1, w.n_chunks):
                rx.receive(t, ks[order[t]], vs[order[t]])
            if w.backward:
                for c in order:
                    rx.send(dk_sent[c], dks[c])
                    rx.send(dv_sent[c], dvs[c])
        rx.finish()

    log(f"[bench] warmup {args.warmup} steps")
    out = None
    for _ in range(args.warmup):
        out = step()
    torch.cuda.synchronize()
    perm, first = out if out is not None else step()
    perm_np = perm.cpu().numpy()
    first_np = first.cpu().numpy() if first is not None else None

    # timed region: barrier (one process) + synchronize on both sides; an
    # event between steps on the launch stream gives each step's own time
    timer.enabled = True
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record()
    for i in range(args.steps):
        step()
        marks[i + 1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timer.enabled = False
    ms_per_step = elapsed / args.steps * 1e3
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    log(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step")

    pairs = visible_pairs_per_chunk(w, perm_np, rank, first_np)
    fwd_flops = 4.0 * d * hq * sum(pairs)
    bwd_flops = 10.0 * d * hq * sum(pairs) if w.backward else 0.0
    total_flops = fwd_flops + bwd_flops
    value = total_flops / (ms_per_step * 1e-3) / 1e12

    def kernel_roofline(kind, per_pair):
        launches = timer.summary(kind)
        if not launches:
            return None
        tot_ms = sum(ms for _, ms in launches)
        tot_flop = sum(per_pair * d * hq * pairs[c] for c, _ in launches)
        avg_ms = tot_ms / len(launches)
        achieved = tot_flop / (tot_ms * 1e-3) / 1e12
        name = "attn_bwd_chunk" if kind == "bwd" else "attn_fwd_chunk"
        traffic = read_traffic(name, w.name)
        return {"kernel": name, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "avg_launch_ms": round(avg_ms, 4),
                "launches": len(launches),
                "algorithmic_flop_per_launch": round(tot_flop / len(launches), 1)}

    def by_chunk_class(kind, per_pair):
        """Average launch time and rate per chunk class: the rank's own chunk
        (the causal diagonal), chunks of earlier ranks and of later ranks."""
        out = {}
        for cls, pick in (("own", lambda c: c == rank), ("earlier_ranks", lambda c: c < rank),
                          ("later_ranks", lambda c: c > rank)):
            sel = [(c, ms) for c, ms in timer.summary(kind) if pick(c)]
            if not sel:
                continue
            tot_ms = sum(ms for _, ms in sel)
            flop = sum(per_pair * d * hq * pairs[c] for c, _ in sel)
            out[cls] = {"avg_launch_ms": round(tot_ms / len(sel), 4),
                        "tflops": round(flop / (tot_ms * 1e-3) / 1e12, 2) if tot_ms else None,
                        "launches": len(sel)}
        return out

    fwd_rf = kernel_roofline("fwd", 4)
    bwd_rf = kernel_roofline("bwd", 10) if w.backward else None
    fwd_ms = sum(ms for _, ms in timer.summary("fwd")) / args.steps
    bwd_ms = sum(ms for _, ms in timer.summary("bwd")) / args.steps if w.backward else 0.0
    fwd_tflops = fwd_flops / (fwd_ms * 1e-3) / 1e12 if fwd_ms > 0 else None
    if not w.backward:
        value = fwd_flops / (ms_per_step * 1e-3) / 1e12

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) rounded to bf16; frame/text label stream)",
        "config": {
            "workload": w.name,
            "description": w.note,
            "q_shard_tokens": w.shard,
            "kv_chunks": w.n_chunks,
            "kv_chunk_tokens": w.chunk,
            "hq": w.hq, "hkv": w.hkv, "head_dim": w.d,
            "layout": w.layout, "rank": rank,
            "pass": "fwd+bwd" if w.backward else "fwd",
            "merge": "separate" if args.unfused else "fused into chunk epilogue",
            "tile_order": ("built-in" if w.layout != "packed" or args.no_plan
                           else "work-ordered plan per chunk"),
            "chunks": ("received by double-buffered copies" if args.ring_copy
                       else "resident in HBM"),
            "rope_theta": theta,
        },
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_tflops, 2) if fwd_tflops else None,
        "fwd_pct_of_peak": round(100 * fwd_tflops / PEAK_BF16_TFLOPS, 2) if fwd_tflops else None,
        "fwd_ms_per_step": round(fwd_ms, 4),
        "bwd_ms_per_step": round(bwd_ms, 4),
        "algorithmic_tflop_per_step": round(total_flops / 1e12, 4),
        "visible_pairs_per_head": int(sum(pairs)),
        "roofline": bwd_rf if bwd_rf is not None else fwd_rf,
        "roofline_fwd": fwd_rf,
        "step_ms": {"min": round(step_ms[0], 4), "median": round(step_ms[len(step_ms) // 2], 4),
                    "max": round(step_ms[-1], 4)},
        "chunk_classes": {"fwd": by_chunk_class("fwd", 4),
                          **({"bwd": by_chunk_class("bwd", 10)} if w.backward else {})},
        "device": device_record(torch, mmsp),
    }
    if theta:
        rope_ms = sum(ms for _, ms in timer.summary("rope")) / args.steps
        elems = (q.numel() + sum(t.numel() for t in ks)) * 2 * 2  # bf16 read + write
        if w.backward:
            elems += (dq.numel() + sum(t.numel() for t in dks)) * 4 * 2  # fp32 in place
        result["rope"] = {"ms_per_step": round(rope_ms, 4),
                          "hbm_bytes_per_step": int(elems),
                          "GBps": round(elems / (rope_ms * 1e-3) / 1e9, 1),
                          "share_of_step_pct": round(100 * rope_ms / ms_per_step, 2)}
    if rx is not None:
        def timed(fn):
            torch.cuda.synchronize()
            t_0 = time.perf_counter()
            for _ in range(args.steps):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - t_0) / args.steps * 1e3
        rx.bytes_received = rx.bytes_sent = 0
        copy_ms = timed(copies_only)
        copy_bytes = (rx.bytes_received + rx.bytes_sent) / args.steps
        resident_ms = timed(lambda: step(received=False))
        result["ring_copy"] = {
            "what": ("each KV chunk after the rank's own is copied device-to-device into one of "
                     "two receive buffers on a second stream while the previous chunk is "
                     "computed" + ("; each chunk's dK/dV are copied out the same way"
                                   if w.backward else "")),
            "ms_per_step_received": round(ms_per_step, 4),
            "ms_per_step_resident": round(resident_ms, 4),
            "overlap_loss_pct": round(100 * (ms_per_step - resident_ms) / resident_ms, 2),
            "copy_only_ms_per_step": round(copy_ms, 4),
            "copy_bytes_per_step": int(copy_bytes),
            "copy_only_GBps": round(copy_bytes / (copy_ms * 1e-3) / 1e9, 1),
            "exposed_copy_pct": round(100 * max(0.0, ms_per_step - resident_ms) / copy_ms, 2),
        }
    if args.gather:
        stream = torch.empty((n, hq, d), dtype=torch.bfloat16, device=device).normal_()
        into = torch.empty_like(stream)
        perm_all = torch.from_numpy(perm_np.astype(np.int32)).to(device)
        for _ in range(2):
            mmsp.shard_gather(stream, perm_all, out=into)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(args.steps):
            mmsp.shard_gather(stream, perm_all, out=into)
        ev[1].record()
        torch.cuda.synchronize()
        g_ms = ev[0].elapsed_time(ev[1]) / args.steps
        g_bytes = 2 * stream.numel() * stream.element_size()  # every row read and written
        result["gather"] = {"what": "whole token stream moved into rank-major shard order",
                            "rows": n, "row_bytes": hq * d * 2, "ms": round(g_ms, 4),
                            "hbm_bytes": g_bytes,
                            "GBps": round(g_bytes / (g_ms * 1e-3) / 1e9, 1),
                            "frac_of_hbm_peak": round(g_bytes / (g_ms * 1e-3) / 8e12, 3)}
        del stream, into
    if args.sdpa_context:
        result["sdpa_context"] = sdpa_context(torch, w, args.steps, device)
    if args.gemm_context:
        result["gemm_context"] = gemm_context(torch, args.steps, device)
    if args.native_ring:
        outs = [o, lse, o16] + ([dq] + dks + dvs if w.backward else [])

        def native_step():
            perm_n, _, qs_n = balance()
            qp_n = perm_n[rank * w.shard:(rank + 1) * w.shard]
            kps_n = [perm_n[c * w.chunk:(c + 1) * w.chunk] for c in range(w.n_chunks)]
            mmsp.ring_forward_native(q, ks, vs, qp_n, kps_n, rank=rank, o=o, lse=lse,
                                     o_final=o16, q_start=qs_n)
            if w.backward:
                mmsp.ring_backward_native(q, ks, vs, dout, o16, lse, qp_n, kps_n, rank=rank,
                                          dq=dq, dks=dks, dvs=dvs, delta=delta, q_start=qs_n)

        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        want = [t.clone() for t in outs]
        for t in outs:
            t.zero_()
        native_step()
        torch.cuda.synchronize()
        n_match = all(torch.equal(a, b) for a, b in zip(outs, want))
        for _ in range(args.warmup):
            native_step()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(args.steps):
            native_step()
        ev[1].record()
        torch.cuda.synchronize()
        n_ms = ev[0].elapsed_time(ev[1]) / args.steps
        result["native_ring"] = {"ms_per_step": round(n_ms, 4),
                                 "python_driver_ms_per_step": round(ms_per_step, 4),
                                 "outputs_equal_python_driver": bool(n_match)}
        log(f"[bench] native ring {n_ms:.3f} ms/step (Python driver {ms_per_step:.3f}), "
            f"outputs equal: {n_match}")
    if args.graph:
        outs = [o, lse, o16] + ([dq] + dks + dvs if w.backward else [])
        g_ms, g_match = graph_replay(torch, step, outs, args.steps)
        result["graph"] = {"ms_per_step": round(g_ms, 4), "eager_ms_per_step": round(ms_per_step, 4),
                           "saving_pct": round(100 * (ms_per_step - g_ms) / ms_per_step, 2),
                           "replays_equal_eager": bool(g_match)}
        log(f"[bench] graph replay {g_ms:.3f} ms/step (eager {ms_per_step:.3f}), "
            f"replays equal eager: {g_match}")
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host ("
            + ("whole workload" if args.cpu_full else "bounded sample") + ")")
        result["cpu_baseline"] = cpu_baseline(w, rank, perm_np, first_np, full=args.cpu_full)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
