"""Top-k selection of compressed entries (oracle side).

"DeepSeek V4: How They Crushed the Million-Token Memory Problem"
(sameershanbhag.com), "Two kinds of memory instead of one": the indexer keeps
only the top-k most relevant compressed blocks.

Reading: among the visible entries j (those whose block is complete at the query,
j < floor((t+1)/m)), keep the min(k, V) with the largest score; equal scores go to
the lower index (+0 and -0 are equal).  The output is the chosen set in ascending
order, padded with -1 to length k.
"""
from __future__ import annotations

import numpy as np


def n_visible(t: int, m: int) -> int:
    """Entries whose whole block lies at or before position t."""
    return (int(t) + 1) // int(m)


def select(scores: np.ndarray, k: int) -> np.ndarray:
    """Ascending indices of the top-k of ``scores`` [V] (ties: lower index), -1 padded."""
    s = np.asarray(scores)
    V = s.shape[0]
    j = np.arange(V)
    order = np.lexsort((j, -s.astype(np.float64)))      # by -score, then index
    keep = np.sort(order[:min(k, V)])
    out = np.full(k, -1, np.int64)
    out[:keep.size] = keep
    return out


def kth_gap(scores: np.ndarray, k: int):
    """(k-th largest, (k+1)-th largest) scores, for reporting near-ties."""
    s = np.sort(np.asarray(scores, np.float64))[::-1]
    if s.size <= k:
        return None
    return s[k - 1], s[k]
