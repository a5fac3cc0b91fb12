"""Seeded synthetic inputs shared by the tests, the bench and the oracle runs.

This module holds *no* arithmetic of the attention method: it draws random
tensors, rounds them to bfloat16 (round-to-nearest-even) and builds the
text/visual label stream.  Both the HIP path and the CPU oracle consume what it
returns; neither is imported here.

Workload shapes follow the pages: 576 visual tokens per video frame sampled at
one frame per second ("LongVILA Guide: 2M Context Multi-Modal AI Model",
section "Problem", item 1), a 2,097,152-token context over 256 ranks, i.e.
8192 tokens per rank, and 32 query heads (same page, "Multi-Modal Sequence
Parallelism (MM-SP) Mechanics" and the launcher under "Production").
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# seeds of the synthetic tensors
SEED_Q, SEED_K, SEED_V, SEED_DO, SEED_SEGMENTS = 1, 2, 3, 4, 5

FRAME_TOKENS = 576  # visual tokens per frame
TEXT_RUN = (8, 64)  # inclusive range of the text run after each frame


def bf16_round(x):
    """Round float32 values to bfloat16, nearest-even.

    Returns ``(bits, values)``: ``bits`` is ``uint16`` (the bf16 encoding) and
    ``values`` the same numbers as float32.  Inputs must be finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    hi = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    vals = (hi.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return hi, vals


def normal_bf16(seed: int, shape, scale: float = 1.0):
    """N(0, scale^2) samples drawn as float32 from ``default_rng(seed)``, rounded to bf16."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return bf16_round(x)


def frame_text_labels(n: int, seed: int = SEED_SEGMENTS) -> np.ndarray:
    """Interleaved video/text label stream (uint8, 1 = visual token, 0 = text).

    A text run of U{8..64} tokens, then repeated [576 visual][text U{8..64}]
    -- one frame per second followed by its timestamp/caption text -- until at
    least ``n`` tokens, truncated to ``n``.
    """
    rng = np.random.default_rng(seed)
    out = []
    total = 0
    run = int(rng.integers(TEXT_RUN[0], TEXT_RUN[1] + 1))
    out.append(np.zeros(run, dtype=np.uint8))
    total += run
    while total < n:
        out.append(np.ones(FRAME_TOKENS, dtype=np.uint8))
        run = int(rng.integers(TEXT_RUN[0], TEXT_RUN[1] + 1))
        out.append(np.zeros(run, dtype=np.uint8))
        total += FRAME_TOKENS + run
    return np.concatenate(out)[:n]


def tiny_labels() -> np.ndarray:
    """The 1024-token stream of the tiny case: 64 text, one 576-token frame, 384 text."""
    return np.concatenate([np.zeros(64, np.uint8), np.ones(576, np.uint8),
                           np.zeros(384, np.uint8)])


def packed_sample_starts(n: int, multiple: int, seed: int = SEED_SEGMENTS) -> np.ndarray:
    """Boundaries of video samples packed into an ``n``-token buffer.

    Each sample is a clip of U{2..40} frames of 576 visual tokens, each frame
    followed by U{8..64} text tokens, its length rounded up to a multiple of
    ``multiple`` (so every sample can be zigzagged on its own); samples are
    drawn until the buffer is full and the last one takes the remainder.
    ``n`` must be a multiple of ``multiple``.  Returns int32 ``[n_samples+1]``.
    """
    assert n % multiple == 0
    rng = np.random.default_rng(seed)
    starts = [0]
    while True:
        frames = int(rng.integers(2, 41))
        ln = sum(FRAME_TOKENS + int(rng.integers(TEXT_RUN[0], TEXT_RUN[1] + 1))
                 for _ in range(frames))
        ln = -(-ln // multiple) * multiple
        if starts[-1] + ln >= n:
            break
        starts.append(starts[-1] + ln)
    starts.append(n)
    return np.asarray(starts, dtype=np.int32)


@dataclass(frozen=True)
class Workload:
    """One synthetic per-rank workload.

    ``layout`` is ``"contiguous"`` (single rank holding every position, KV
    split into contiguous chunks), ``"zigzag"``, ``"modality"`` or
    ``"packed"`` (variable-length samples packed into the buffer, each
    zigzagged on its own); the positions themselves are produced by the
    shard-balance step, not here.
    """

    name: str
    n_tokens: int
    n_ranks: int
    hq: int
    hkv: int
    d: int
    layout: str
    granularity: int = 0
    rank: int = 0
    n_chunks_override: int = 0
    backward: bool = False
    note: str = field(default="", compare=False)

    @property
    def shard(self) -> int:
        return self.n_tokens // self.n_ranks

    @property
    def n_chunks(self) -> int:
        return self.n_chunks_override or self.n_ranks

    @property
    def chunk(self) -> int:
        return self.n_tokens // self.n_chunks

    def labels(self) -> np.ndarray:
        if self.layout == "contiguous":
            return tiny_labels() if self.n_tokens == 1024 else np.zeros(self.n_tokens, np.uint8)
        return frame_text_labels(self.n_tokens)

    def sample_starts(self) -> np.ndarray:
        """Packed layout: ``n_samples + 1`` sample boundaries (int32).  Sample
        lengths are multiples of ``2P * granularity`` (``granularity`` 0 or 1:
        just ``2P``, what the per-sample zigzag needs)."""
        return packed_sample_starts(self.n_tokens, 2 * self.n_ranks * max(1, self.granularity))

    def q(self):
        return normal_bf16(SEED_Q, (self.shard, self.hq, self.d))

    def k(self):
        return normal_bf16(SEED_K, (self.n_chunks, self.chunk, self.hkv, self.d))

    def v(self):
        return normal_bf16(SEED_V, (self.n_chunks, self.chunk, self.hkv, self.d))

    def do(self):
        return normal_bf16(SEED_DO, (self.shard, self.hq, self.d))


TINY = Workload("tiny_s1024_h4_d64_4chunks", 1024, 1, 4, 4, 64, "contiguous",
                n_chunks_override=4, backward=True,
                note="64 text + 576 visual + 384 text; KV in 4 contiguous chunks of 256")
RANK_FWD = Workload("zigzag_p8_shard8192_h32_d128", 65536, 8, 32, 32, 128, "zigzag",
                    note="rank 0 of zigzag P=8: 8192-token Q shard vs 8 KV chunks of 8192")
GQA = Workload("zigzag_p16_shard16384_hq28_hkv4_d128", 262144, 16, 28, 4, 128, "zigzag",
               note="rank 0 of zigzag P=16: 16384-token Q shard vs 16 KV chunks, GQA 28/4")
MODALITY = Workload("modality_p8_g256_n65536_h32_d128", 65536, 8, 32, 32, 128, "modality",
                    granularity=256,
                    note="frame/text stream, modality-balanced into 8 shards at g=256; rank 0")
TRAIN = Workload("zigzag_p8_shard8192_h32_d128_fwd_bwd", 65536, 8, 32, 32, 128, "zigzag",
                 backward=True,
                 note="rank 0 of zigzag P=8, forward + backward over 8 KV chunks")

# The per-GPU share after the intra-node all-to-all of the hybrid scheme: a
# 2,097,152-token context over a ring of 32 node groups (65,536 tokens each)
# whose 8 GPUs split the 32 heads, 4 per GPU ("LongVILA Guide: 2M Context
# Multi-Modal AI Model", "Multi-Modal Sequence Parallelism (MM-SP)
# Mechanics", items 1-2): long rows, few heads, 32 ring steps.
ULYSSES = Workload("ulysses_p32_shard65536_h4_d128", 2097152, 32, 4, 4, 128, "zigzag",
                   note="rank 0 of a zigzag ring of 32 over 2,097,152 tokens, 4 heads per GPU: "
                        "65,536-token Q shard vs 32 KV chunks of 65,536")
ULYSSES_TRAIN = Workload("ulysses_p32_shard65536_h4_d128_fwd_bwd", 2097152, 32, 4, 4, 128,
                         "zigzag", backward=True,
                         note="as ulysses_p32_shard65536_h4_d128, forward + backward")

# Packed video samples (reset attention masks between them: same page,
# "Critical Operational Best Practices"), per-sample zigzag over 8 ranks.
PACKED = Workload("packed_p8_n65536_h32_d128", 65536, 8, 32, 32, 128, "packed",
                  note="video clips of 2-40 frames packed into 65,536 tokens, each zigzagged "
                       "over 8 ranks; rank 0 (reset masks between samples)")
PACKED_TRAIN = Workload("packed_p8_n65536_h32_d128_fwd_bwd", 65536, 8, 32, 32, 128, "packed",
                        backward=True, note="as packed_p8_n65536_h32_d128, forward + backward")

# The same clips with every length rounded up to a multiple of 2P x 64, so
# each per-rank piece is a whole number of 64-token tiles and no tile holds
# two samples (about 4% padding tokens at this length mix).
PACKED_ALIGNED_TRAIN = Workload("packed_aligned64_p8_n65536_h32_d128_fwd_bwd", 65536, 8, 32, 32,
                                128, "packed", granularity=64, backward=True,
                                note="as packed_p8_n65536_h32_d128_fwd_bwd with clip lengths "
                                     "rounded up to multiples of 1024 (tile-aligned pieces)")

WORKLOADS = {w.name: w for w in (TINY, RANK_FWD, GQA, MODALITY, TRAIN, ULYSSES, ULYSSES_TRAIN,
                                 PACKED, PACKED_TRAIN, PACKED_ALIGNED_TRAIN)}
