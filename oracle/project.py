"""Grouped output projection after attention (oracle side).

"DeepSeek V4 infrastructure" (volanea.com), "Compression only works if the
attention path is engineered end to end": CSA's attention ends in a grouped output
projection.  The page gives no formula.  Reading: the H heads are split into G
consecutive groups of H/G heads; group g's head outputs, concatenated in head order
(K_g = (H/G) * D values), are multiplied by the group's own weight matrix, and the
G results are concatenated:

    y[n, g, c] = sum_{k < K_g} o[n, g*(H/G) + k // D, k % D] * W[g, c, k]

(W stored as [G, d_g, K_g]: output unit c of group g holds its K_g input weights
contiguously).  Evaluated in fp64 from the stored BF16 values.
"""
from __future__ import annotations

import numpy as np


def grouped_out_proj(o: np.ndarray, W: np.ndarray) -> np.ndarray:
    """o [Nq, H, D], W [G, d_g, K_g] (fp64 values) -> y [Nq, G, d_g] (fp64)."""
    o = np.asarray(o, np.float64)
    W = np.asarray(W, np.float64)
    Nq, H, D = o.shape
    G, d_g, K_g = W.shape
    assert H % G == 0 and K_g == (H // G) * D
    x = o.reshape(Nq, G, K_g)                    # group g: heads g*H/G .. (g+1)*H/G - 1, in order
    y = np.empty((Nq, G, d_g))
    for g in range(G):
        y[:, g, :] = x[:, g, :] @ W[g].T
    return y
