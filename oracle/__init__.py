"""CPU oracle for per-rank MM-SP chunked causal attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only the tests, the smoke check of ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` may call it.  It is a plain, slow, obviously-correct numpy
float64 restatement of what the hot path computes, written from the source
pages (cited per function) and sharing no code with the HIP library.

Sources (web pages, cited by title and section):

* "LongVILA Guide: 2M Context Multi-Modal AI Model" -- section
  "Implementation: PyTorch Distributed Pipeline and Token Routing"
  (the ``LongVILAMultiModalAttention.forward`` ring loop: scaled dot-product
  scores divided by the square root of the head dimension, a softmax, and a
  per-ring-step accumulation into an output accumulator); section
  "Multi-Modal Sequence Parallelism (MM-SP) Mechanics" (ring of KV chunks,
  one attention call per chunk); section "Problem" item 2 (modality
  imbalance between ranks).
* "Ultra-Large Multimodal LLM Inference ..." section 4, "Load Balancing for
  Tensor Parallelism" (dispatch by modality token density).
* "LongVILA - ... (Jason's Study)" section "What it is" (2M context trained
  without gradient checkpointing, so the backward consumes the saved
  forward statistics).

Modules:

* :mod:`oracle.attention` -- causal attention of a query shard against one
  KV chunk, returning ``(O, LSE)``.  Pinned (closed forms, brute force).
* :mod:`oracle.merge`     -- log-sum-exp merge of chunk results and the
  ring-order driver.  Pinned (split-then-merge equals unsplit).
* :mod:`oracle.backward`  -- gradients of the chunk attention from the final
  LSE.  Pinned (central finite differences, softmax invariants).
* :mod:`oracle.rope`      -- rotary position embedding at global positions
  (theta = 1e7 in the 2M stage).  Pinned (hand-worked values, norms,
  relative-position invariance, inverse).
* :mod:`oracle.balance`   -- zigzag and modality-balanced shard
  permutations.  Pinned by closed form, invariants and brute force; the
  exact modality assignment rule is this project's definition because the
  pages state only the problem (see :mod:`oracle.balance`).
"""

from .attention import attention_forward, visible_pairs  # noqa: F401
from .merge import lse_merge, ring_forward  # noqa: F401
from .backward import (attention_abs_dp, attention_backward,  # noqa: F401
                       attention_backward_magnitudes, bwd_delta)
from .rope import rope, rope_angles, rope_bf16  # noqa: F401
from .balance import (  # noqa: F401
    zigzag_perm,
    zigzag_packed_perm,
    modality_perm,
    inverse_perm,
    causal_work_per_rank,
    visual_per_rank,
    gather_rows,
    scatter_rows,
)
