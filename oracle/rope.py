"""Oracle: rotary position embedding at global token positions (float64).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

"LongVILA Guide: 2M Context Multi-Modal AI Model", section "Three-Stage
Long-Context Alignment Curriculum", stage 2: the rotary position embedding's
base frequency theta is raised from 10,000 to 10,000,000 before the 2M-token
stage.  The page gives no formula; the reading used here is the common
half-split form of rotary embeddings: for head dimension ``d`` and pair index
``i < d/2``, the pair ``(x[i], x[i + d/2])`` of a query or key at position
``p`` is rotated by the angle ``p * theta**(-2 i / d)``:

    y[i]       = x[i] cos(a) - x[i + d/2] sin(a)
    y[i + d/2] = x[i + d/2] cos(a) + x[i] sin(a)

Positions are the tokens' global positions (the balanced shard's ``q_pos`` /
``k_pos``), so every rank rotates its tokens exactly as an unsharded model
would.  The inverse (rotation by ``-a``) is the transpose, which maps
gradients with respect to rotated queries/keys back to the unrotated ones.

Rotated queries and keys enter attention as bf16 (as a model feeds them to
its attention kernel): ``rope_bf16`` rounds the float64 rotation to float32
and then to bf16, both round-to-nearest-even.
"""

from __future__ import annotations

import numpy as np


def rope_angles(pos, d: int, theta: float) -> np.ndarray:
    """``[S, d/2]`` angles ``pos * theta**(-2 i / d)`` in float64."""
    pos = np.asarray(pos, dtype=np.float64)
    i = np.arange(d // 2, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * i / d)
    return pos[:, None] * inv_freq[None, :]


def rope(x, pos, theta: float, inverse: bool = False) -> np.ndarray:
    """Rotate ``x[S, H, d]`` (any float type) at positions ``pos[S]``; float64 out."""
    x = np.asarray(x, dtype=np.float64)
    s, h, d = x.shape
    assert d % 2 == 0 and np.asarray(pos).shape == (s,)
    a = rope_angles(pos, d, theta)
    c = np.cos(a)[:, None, :]
    sn = np.sin(a)[:, None, :]
    if inverse:
        sn = -sn
    x1 = x[..., : d // 2]
    x2 = x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * sn, x2 * c + x1 * sn], axis=-1)


def rope_bf16(x, pos, theta: float):
    """Rotation rounded float64 -> float32 -> bf16 (RNE).  Returns ``(bits, values)``
    like the seeded input generators: ``uint16`` encodings and their float32 values."""
    y = rope(x, pos, theta).astype(np.float32)
    u = y.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    hi = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    vals = (hi.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return hi, vals
