"""Shared-KV multi-query attention with one softmax (oracle side).

"DeepSeek V4 infrastructure" (volanea.com), "Compression only works if the
attention path is engineered end to end": CSA attends with shared key-value
multi-query attention over compressed entries picked by the indexer, plus a
sliding-window branch and an attention sink.  "DeepSeek V4: How They Crushed the
Million-Token Memory Problem" (sameershanbhag.com), "Two kinds of memory instead of
one": HCA attends densely over all its compressed entries, and both keep a
separate sliding window of recent uncompressed tokens.

Readings:
  * every query head uses the same key/value vectors, and a key is also its value
    (the whole stored D-dim entry, RoPE slice included);
  * the attention set of query t is its selected CSA entries (all visible HCA
    entries) plus the raw window tokens u in [max(0, t-n_win+1), t] with their RoPE
    slice rotated at u; entries overlapping the window are not removed;
  * the sink is one extra logit sigma_h per head with a zero value, not scaled by tau:
        l_a = tau * q_hat . kappa_a,  M = max(sigma, max_a l_a)
        o   = sum_a e^(l_a - M) kappa_a / (e^(sigma - M) + sum_a e^(l_a - M))
        lse = M + log(e^(sigma - M) + sum_a e^(l_a - M)).
"""
from __future__ import annotations

import numpy as np

from . import rope


def attend(q_hat: np.ndarray, keys: np.ndarray, sink: np.ndarray, tau: float):
    """o [H, D], lse [H] for rotated queries q_hat [H, D] over keys=values [A, D]."""
    q = np.asarray(q_hat, np.float64)
    K = np.asarray(keys, np.float64)
    sig = np.asarray(sink, np.float64)
    if K.shape[0] == 0:
        return np.zeros_like(q), sig.copy()
    logits = tau * (q @ K.T)                                  # [H, A]
    M = np.maximum(sig, logits.max(axis=1))
    e = np.exp(logits - M[:, None])
    es = np.exp(sig - M)
    den = es + e.sum(axis=1)
    o = (e @ K) / den[:, None]
    return o, M + np.log(den)


def window_positions(t: int, n_win: int) -> np.ndarray:
    return np.arange(max(0, int(t) - n_win + 1), int(t) + 1, dtype=np.int64)


def window_keys(ring: np.ndarray, seq: int, t: int, n_win: int, W_cap: int, D_r: int,
                base: float) -> np.ndarray:
    """Rotated window tokens [n, D] of sequence ``seq`` at query position t, read from a
    ring of decoded raw rows [B, W_cap, D] (token u at slot u mod W_cap)."""
    u = window_positions(t, n_win)
    x = np.asarray(ring[seq][u % W_cap], np.float64)
    return rope.apply(x, u, D_r, base)


def query_hat(q: np.ndarray, t: int, D_r: int, base: float) -> np.ndarray:
    """[q_nope ; R(t) q_rope] for every head of one query [H, D]."""
    return rope.apply(q, t, D_r, base)
