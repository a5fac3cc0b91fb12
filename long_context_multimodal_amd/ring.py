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


def ring_forward(q, k_chunks, v_chunks, q_pos, k_pos_chunks, rank=0, fused=True, scale=None,
                 causal=True, order=None, o_final=None, o=None, lse=None, timer=None):
    """Forward over all chunks in ring order.

    Returns ``(o_acc fp32[sq,hq,d], lse fp32[hq,sq], o_bf16[sq,hq,d])``.  ``o``,
    ``lse`` and ``o_final`` may be given to reuse buffers; ``timer`` (optional)
    gets ``start/stop(kind, chunk)`` calls around every chunk launch.
    """
    import torch
    n = len(k_chunks)
    order = ring_order(rank, n) if order is None else order
    o_part = lse_part = None
    for step, c in enumerate(order):
        kp = k_pos_chunks[c] if causal else None
        if timer is not None:
            timer.start("fwd", c)
        if step == 0:
            o, lse = mmsp.attn_fwd_chunk(q, k_chunks[c], v_chunks[c], q_pos, kp, scale=scale,
                                         causal=causal, o=o, lse=lse)
        elif fused:
            mmsp.attn_fwd_chunk(q, k_chunks[c], v_chunks[c], q_pos, kp, scale=scale,
                                causal=causal, o=o, lse=lse, accumulate=True)
        else:
            o_part, lse_part = mmsp.attn_fwd_chunk(q, k_chunks[c], v_chunks[c], q_pos, kp,
                                                   scale=scale, causal=causal, o=o_part,
                                                   lse=lse_part)
            mmsp.lse_merge(o, lse, o_part, lse_part)
        if timer is not None:
            timer.stop("fwd", c)
    if o_final is None:
        o_final = torch.empty(o.shape, dtype=torch.bfloat16, device=o.device)
    mmsp.lse_merge(o, lse, None, None, o_final=o_final)
    return o, lse, o_final


def ring_backward(q, k_chunks, v_chunks, dout, o_bf16, lse, q_pos, k_pos_chunks, rank=0,
                  scale=None, causal=True, order=None, dq=None, dks=None, dvs=None, delta=None,
                  timer=None):
    """Backward over all chunks in ring order from the saved output and LSE.

    Returns ``(dq fp32[sq,hq,d], [dk_c fp32], [dv_c fp32])`` indexed by chunk.
    """
    import torch
    n = len(k_chunks)
    order = ring_order(rank, n) if order is None else order
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
                                             causal=causal)
        if timer is not None:
            timer.stop("bwd", c)
    return dq, dks, dvs
