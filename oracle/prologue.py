"""Query and key-value normalization ahead of attention (oracle side).

"DeepSeek V4 infrastructure" (volanea.com), "Compression only works if the
attention path is engineered end to end": the attention path normalizes the
queries and the key-value vectors.  The page gives no formula.  Reading: a
root-mean-square normalization with a learned per-dimension scale gamma, over the
D dims of every query head vector and of every new key-value token,

    y_d = gamma_d * x_d / sqrt(mean_e(x_e^2) + eps),

evaluated in fp64 and rounded once into the storage format.  A normalized token is
what the sliding-window ring holds (token u of sequence b at slot b * W_cap +
u mod W_cap), so the window branch and the pooling both read it.  The indexer's
vectors are not normalized.
"""
from __future__ import annotations

import numpy as np

from . import quant


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """fp64 normalization of the last axis of ``x`` (any leading shape)."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(gamma, np.float64) * x / np.sqrt(ms + float(eps))


def encode(y: np.ndarray, fmt: str):
    """Storage codes of fp64 values: (BF16 bits as uint16, or binary32 bits as uint32),
    plus the flags of values within 1e-12 relative of a rounding boundary."""
    if fmt == "f32":
        v, fragile = quant.f32_round(y)
        return v.astype(np.float32).view(np.uint32), fragile
    return quant.bf16_encode(y, return_fragile=True)


def append_ring(ring: np.ndarray, seq: np.ndarray, pos: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """A copy of ``ring`` [B, W_cap, ...] with row i placed at (seq[i], pos[i] mod W_cap)."""
    out = np.array(ring, copy=True)
    W_cap = out.shape[1]
    for i in range(len(seq)):
        out[int(seq[i]), int(pos[i]) % W_cap] = rows[i]
    return out
