"""One rank's ring loop on a single GPU (host orchestration of the C-ABI calls).

"LongVILA Guide: 2M Context Multi-Modal AI Model", section "Implementation:
PyTorch Distributed Pipeline and Token Routing": at ring step ``t`` a rank
computes attention of its local queries against the KV chunk it holds, while
sending that chunk to the next ring rank and receiving the next one from the
previous rank.  The chunk present at step ``t`` on rank ``r`` therefore came
from rank ``(r - t) mod P``.  Here all ``P`` chunks are resident in HBM and
are visited in that order; the per-step output is merged exactly through the
log-sum-exp (fused into the attention epilogue, or as a separate merge pass).

The backward follows the same order: ``delta`` from the saved bf16 output,
then one backward call per chunk adding into ``dQ`` and producing that
chunk's ``dK``/``dV`` (which a multi-GPU ring would send back to the owner).
"""

from __future__ import annotations

from . import mmsp


def ring_order(rank: int, n_chunks: int):
    """Chunk index visited at each ring step by ``rank``."""
    return [(rank - t) % n_chunks for t in range(n_chunks)]


def _back_to_back(k_pos_chunks):
    """One view over all chunks' positions when they lie back to back in one
    array (slices of one balance permutation), else None."""
    import torch
    first = k_pos_chunks[0]
    n, sk = len(k_pos_chunks), first.numel()
    for c, kp in enumerate(k_pos_chunks):
        if (kp.dtype != torch.int32 or kp.device != first.device or kp.numel() != sk or
                not kp.is_contiguous() or kp.data_ptr() != first.data_ptr() + 4 * c * sk):
            return None
    if first.untyped_storage().nbytes() < 4 * (first.storage_offset() + n * sk):
        return None
    return torch.as_strided(first, (n * sk,), (1,))


def packed_plans(q_pos, q_start, k_pos_chunks, plans=None):
    """Tile plans of every chunk for packed samples (:func:`mmsp.packed_plan`),
    indexed by chunk; one set serves the forward and the backward of a step.
    When the chunks' positions lie back to back in one array, one launch makes
    them all and the result is an int32 tensor whose row c is chunk c's plan;
    otherwise a list.  ``plans`` (a result of this call) has its buffers
    reused."""
    import torch
    k_all = _back_to_back(k_pos_chunks)
    if k_all is not None:
        block = plans if isinstance(plans, torch.Tensor) else None
        return mmsp.packed_plans(q_pos, q_start, k_all, len(k_pos_chunks), plans=block)
    reuse = plans if isinstance(plans, list) else None
    return [mmsp.packed_plan(q_pos, q_start, kp, plan=None if reuse is None else reuse[c])
            for c, kp in enumerate(k_pos_chunks)]


def _plans_for(q_pos, q_start, k_pos_chunks, causal, plans):
    """The given plans, or new ones for packed samples, or none."""
    if q_start is None or not causal:
        return None
    return plans if plans is not None else packed_plans(q_pos, q_start, k_pos_chunks)


def ring_forward(q, k_chunks, v_chunks, q_pos, k_pos_chunks, rank=0, fused=True, scale=None,
                 causal=True, order=None, o_final=None, o=None, lse=None, timer=None,
                 q_start=None, plans=None):
    """Forward over all chunks in ring order.

    Returns ``(o_acc fp32[sq,hq,d], lse fp32[hq,sq], o_bf16[sq,hq,d])``.  ``o``,
    ``lse`` and ``o_final`` may be given to reuse buffers; ``timer`` (optional)
    gets ``start/stop(kind, chunk)`` calls around every chunk launch.
    ``q_start`` (optional): per-query sample starts of packed samples;
    ``plans`` (optional, per chunk) their tile plans (:func:`packed_plans`,
    made here when not given).
    """
    import torch
    n = len(k_chunks)
    order = ring_order(rank, n) if order is None else order
    plans = _plans_for(q_pos, q_start, k_pos_chunks, causal, plans)
    o_part = lse_part = None
    for step, c in enumerate(order):
        kp = k_pos_chunks[c] if causal else None
        pl = None if plans is None else plans[c]
        if timer is not None:
            timer.start("fwd", c)
        if step == 0:
            o, lse = mmsp.attn_fwd_chunk(q, k_chunks[c], v_chunks[c], q_pos, kp, scale=scale,
                                         causal=causal, o=o, lse=lse, q_start=q_start, plan=pl)
        elif fused:
            mmsp.attn_fwd_chunk(q, k_chunks[c], v_chunks[c], q_pos, kp, scale=scale,
                                causal=causal, o=o, lse=lse, accumulate=True, q_start=q_start,
                                plan=pl)
        else:
            o_part, lse_part = mmsp.attn_fwd_chunk(q, k_chunks[c], v_chunks[c], q_pos, kp,
                                                   scale=scale, causal=causal, o=o_part,
                                                   lse=lse_part, q_start=q_start, plan=pl)
            mmsp.lse_merge(o, lse, o_part, lse_part)
        if timer is not None:
            timer.stop("fwd", c)
    if o_final is None:
        o_final = torch.empty(o.shape, dtype=torch.bfloat16, device=o.device)
    mmsp.lse_merge(o, lse, None, None, o_final=o_final)
    return o, lse, o_final


def ring_backward(q, k_chunks, v_chunks, dout, o_bf16, lse, q_pos, k_pos_chunks, rank=0,
                  scale=None, causal=True, order=None, dq=None, dks=None, dvs=None, delta=None,
                  timer=None, q_start=None, plans=None):
    """Backward over all chunks in ring order from the saved output and LSE.

    Returns ``(dq fp32[sq,hq,d], [dk_c fp32], [dv_c fp32])`` indexed by chunk.
    ``q_start`` and ``plans`` as in :func:`ring_forward`.
    """
    import torch
    n = len(k_chunks)
    order = ring_order(rank, n) if order is None else order
    plans = _plans_for(q_pos, q_start, k_pos_chunks, causal, plans)
    if dq is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    delta = mmsp.attn_bwd_preprocess(o_bf16, dout, delta, dq_zero=dq)
    dks = [None] * n if dks is None else dks
    dvs = [None] * n if dvs is None else dvs
    for c in order:
        kp = k_pos_chunks[c] if causal else None
        if timer is not None:
            timer.start("bwd", c)
        dks[c], dvs[c] = mmsp.attn_bwd_chunk(q, k_chunks[c], v_chunks[c], dout, lse, delta, q_pos,
                                             kp, dq, dk=dks[c], dv=dvs[c], scale=scale,
                                             causal=causal, q_start=q_start,
                                             plan=None if plans is None else plans[c])
        if timer is not None:
            timer.stop("bwd", c)
    return dq, dks, dvs


class ChunkReceiver:
    """Double-buffered arrival of ring chunks on one GPU.

    The pages hide the ring exchange behind compute: while the attention of
    the chunk held at step ``t`` runs, the next chunk is received from the
    previous rank into a second buffer ("LongVILA Guide: 2M Context
    Multi-Modal AI Model", section "Multi-Modal Sequence Parallelism (MM-SP)
    Mechanics", item 3).  With one GPU the transfer is stood in for by a
    device-to-device copy on a second stream (default priority) from the
    chunk's resident storage into one of two receive buffers; the compute
    stream waits for the copy of its chunk, and a copy into a buffer waits for
    the compute that last read it.  In the backward the chunk's dK/dV are
    likewise copied out (sent back to the owner) on the copy stream.
    """

    def __init__(self, like_k, like_v, device=None):
        import torch
        device = like_k.device if device is None else device
        self.k = [torch.empty_like(like_k) for _ in range(2)]
        self.v = [torch.empty_like(like_v) for _ in range(2)]
        self.stream = torch.cuda.Stream(device=device)
        self.copied = [torch.cuda.Event() for _ in range(2)]
        self.consumed = [torch.cuda.Event() for _ in range(2)]
        self.used = [False, False]
        self.bytes_received = 0
        self.bytes_sent = 0

    def start(self):
        """Order the copy stream after everything already enqueued on the
        current stream.  Without it a copy could run ahead of that work: read
        chunks a preceding kernel has not finished writing (a rotary pass), or
        overwrite memory the allocator handed to the receive buffers after an
        earlier tensor was freed while kernels still reading it were queued."""
        import torch
        self.stream.wait_stream(torch.cuda.current_stream())

    def receive(self, step, k_src, v_src):
        """Enqueue the copy of the chunk for ``step`` into buffer ``step % 2``."""
        import torch
        b = step % 2
        with torch.cuda.stream(self.stream):
            if self.used[b]:
                self.stream.wait_event(self.consumed[b])
            self.k[b].copy_(k_src, non_blocking=True)
            self.v[b].copy_(v_src, non_blocking=True)
            self.copied[b].record(self.stream)
        # the sources are read on the copy stream: keep their memory from
        # being reused by the caching allocator before that read is done
        k_src.record_stream(self.stream)
        v_src.record_stream(self.stream)
        self.bytes_received += k_src.numel() * k_src.element_size() * 2

    def take(self, step):
        """Make the current stream wait for the chunk of ``step``; return its buffers."""
        import torch
        b = step % 2
        torch.cuda.current_stream().wait_event(self.copied[b])
        return self.k[b], self.v[b]

    def release(self, step):
        """Mark the end, on the current stream, of the compute reading ``step``'s buffer."""
        import torch
        b = step % 2
        self.consumed[b].record(torch.cuda.current_stream())
        self.used[b] = True

    def send(self, dst, src):
        """Copy ``src`` (written on the current stream) to ``dst`` on the copy stream."""
        import torch
        ev = torch.cuda.Event()
        ev.record(torch.cuda.current_stream())
        with torch.cuda.stream(self.stream):
            self.stream.wait_event(ev)
            dst.copy_(src, non_blocking=True)
        src.record_stream(self.stream)
        dst.record_stream(self.stream)
        self.bytes_sent += src.numel() * src.element_size()

    def finish(self):
        """Make the current stream wait for every copy enqueued so far."""
        import torch
        torch.cuda.current_stream().wait_stream(self.stream)


def ring_forward_received(q, k_chunks, v_chunks, q_pos, k_pos_chunks, receiver, rank=0,
                          fused=True, scale=None, causal=True, o_final=None, o=None, lse=None,
                          timer=None, q_start=None, plans=None):
    """``ring_forward`` in ring order, with every chunk after the rank's own
    arriving through ``receiver`` (a :class:`ChunkReceiver`) while the previous
    chunk is computed.  Same kernels and order, so the same results."""
    import torch
    n = len(k_chunks)
    order = ring_order(rank, n)
    plans = _plans_for(q_pos, q_start, k_pos_chunks, causal, plans)
    o_part = lse_part = None
    receiver.start()
    for step, c in enumerate(order):
        if step == 0:
            kc, vc = k_chunks[c], v_chunks[c]  # the rank's own chunk is local
        else:
            kc, vc = receiver.take(step)
        if step + 1 < n:  # the next chunk arrives while this one is computed
            receiver.receive(step + 1, k_chunks[order[step + 1]], v_chunks[order[step + 1]])
        kp = k_pos_chunks[c] if causal else None
        pl = None if plans is None else plans[c]
        if timer is not None:
            timer.start("fwd", c)
        if step == 0:
            o, lse = mmsp.attn_fwd_chunk(q, kc, vc, q_pos, kp, scale=scale, causal=causal, o=o,
                                         lse=lse, q_start=q_start, plan=pl)
        elif fused:
            mmsp.attn_fwd_chunk(q, kc, vc, q_pos, kp, scale=scale, causal=causal, o=o, lse=lse,
                                accumulate=True, q_start=q_start, plan=pl)
        else:
            o_part, lse_part = mmsp.attn_fwd_chunk(q, kc, vc, q_pos, kp, scale=scale,
                                                   causal=causal, o=o_part, lse=lse_part,
                                                   q_start=q_start, plan=pl)
            mmsp.lse_merge(o, lse, o_part, lse_part)
        if timer is not None:
            timer.stop("fwd", c)
        if step > 0:
            receiver.release(step)
    if o_final is None:
        o_final = torch.empty(o.shape, dtype=torch.bfloat16, device=o.device)
    mmsp.lse_merge(o, lse, None, None, o_final=o_final)
    receiver.finish()
    return o, lse, o_final


def ring_backward_received(q, k_chunks, v_chunks, dout, o_bf16, lse, q_pos, k_pos_chunks,
                           receiver, rank=0, scale=None, causal=True, dq=None, dks=None,
                           dvs=None, dk_sent=None, dv_sent=None, delta=None, timer=None,
                           q_start=None, plans=None):
    """``ring_backward`` with chunks arriving through ``receiver`` and each
    chunk's dK/dV sent (copied to ``dk_sent[c]``/``dv_sent[c]``) on the copy
    stream as soon as they are computed."""
    import torch
    n = len(k_chunks)
    order = ring_order(rank, n)
    plans = _plans_for(q_pos, q_start, k_pos_chunks, causal, plans)
    if dq is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    receiver.start()
    delta = mmsp.attn_bwd_preprocess(o_bf16, dout, delta, dq_zero=dq)
    dks = [None] * n if dks is None else dks
    dvs = [None] * n if dvs is None else dvs
    for step, c in enumerate(order):
        if step == 0:
            kc, vc = k_chunks[c], v_chunks[c]
        else:
            kc, vc = receiver.take(step)
        if step + 1 < n:
            receiver.receive(step + 1, k_chunks[order[step + 1]], v_chunks[order[step + 1]])
        kp = k_pos_chunks[c] if causal else None
        if timer is not None:
            timer.start("bwd", c)
        dks[c], dvs[c] = mmsp.attn_bwd_chunk(q, kc, vc, dout, lse, delta, q_pos, kp, dq,
                                             dk=dks[c], dv=dvs[c], scale=scale, causal=causal,
                                             q_start=q_start,
                                             plan=None if plans is None else plans[c])
        if timer is not None:
            timer.stop("bwd", c)
        if step > 0:
            receiver.release(step)
        if dk_sent is not None:
            receiver.send(dk_sent[c], dks[c])
            receiver.send(dv_sent[c], dvs[c])
    receiver.finish()
    return dq, dks, dvs
