"""Partial rotary position embedding (oracle side).

"DeepSeek V4 infrastructure" (volanea.com), "Compression only works if the
attention path is engineered end to end": the attention uses *partial* rotary
positional embeddings; "DeepSeek V4: How They Crushed the Million-Token Memory
Problem" (sameershanbhag.com), "Two kinds of memory instead of one": the RoPE
dimensions are the ones kept in BF16.  The pages give no formula.  Reading: the
last D_r dims of a D-dim vector are rotated with the half-split pairing, dims
(i, i + D_r/2) by the angle pos * base^(-2i/D_r); angles, cosines and sines in fp64.
"""
from __future__ import annotations

import numpy as np


def inv_freq(D_r: int, base: float) -> np.ndarray:
    i = np.arange(D_r // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / D_r)


def rotate(x_rope: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate the RoPE slice ``x_rope`` [..., D_r] at position(s) ``pos`` (broadcast
    over the leading dims).  Returns fp64."""
    x = np.asarray(x_rope, np.float64)
    D_r = x.shape[-1]
    h = D_r // 2
    theta = np.asarray(pos, np.float64)[..., None] * inv_freq(D_r, base)
    c, s = np.cos(theta), np.sin(theta)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def apply(x: np.ndarray, pos, D_r: int, base: float) -> np.ndarray:
    """[x_nope ; R(pos) x_rope] for a full D-dim vector (fp64)."""
    x = np.asarray(x, np.float64)
    if D_r == 0:
        return x.copy()
    return np.concatenate([x[..., :-D_r], rotate(x[..., -D_r:], pos, base)], axis=-1)
