"""Lightning-indexer scores (oracle side).

"DeepSeek V4: How They Crushed the Million-Token Memory Problem"
(sameershanbhag.com), "Two kinds of memory instead of one": the lightning indexer
runs in FP4 and scores with ReLU-scored multi-head dot products, then keeps the
top-k compressed blocks.  "DeepSeek V4 infrastructure" (volanea.com), "Compression
only works if the attention path is engineered end to end": a lightweight indexer
selects the relevant blocks from auxiliary indexing data.

Reading: for query t, indexer head h and visible entry j,
    d[t,h,j] = q_I[t,h] . k_I[j]          (no RoPE, no scale)
    I[t,j]   = sum_h w[t,h] * max(d[t,h,j], 0)
with per-(query, head) weights w >= 0.

Quantized operands (FP8 with per-tensor scale 1, or MXFP4): every head dot is an
exact binary32 number (products of the element grids are exact and the sums stay
within 24 bits), so d is computed exactly here and checked to be so.  The head
sum is then defined in binary32, one rounding per head (a fused multiply-add into
the running sum), in one canonical order:
    S_u <- fl32(w_h * max(d_h, +0) + S_u), from S_u = +0,
           over h = 32T + 8(i//4) + 4u + i%4, T ascending, then i = 0..15   (u = 0, 1)
    I    = fl32(S_0 + S_1)
f32 operands (the tiny workload): everything in fp64, sequential over dims, then
over heads ascending, un-fused.
"""
from __future__ import annotations

import numpy as np


def head_dots_exact(q_vals: np.ndarray, k_vals: np.ndarray, grain_q, grain_k) -> np.ndarray:
    """d[h, j] for decoded quantized operands q [H_I, d_I], k [V, d_I].

    ``grain_q`` [H_I] / ``grain_k`` [V] are the finest spacing of each row's value
    grid (2^-9 for FP8 E4M3; half the smallest block scale for MXFP4).  Every
    product is then a multiple of grain_q*grain_k, and every partial sum of the dot,
    in any order, is a binary32 number while sum_i |q_i k_i| < 2^24 grain_q grain_k.
    That condition is asserted, so the fp64 value below is the exact dot, and
    binary32 hardware reaches it in any accumulation order.
    """
    q = np.asarray(q_vals, np.float64)
    k = np.asarray(k_vals, np.float64)
    d = q @ k.T
    if d.size:
        absum = np.abs(q) @ np.abs(k).T
        bound = np.float64(2.0 ** 24) * np.outer(np.asarray(grain_q, np.float64),
                                                np.asarray(grain_k, np.float64))
        assert np.all(absum < bound), "head dot not exact in binary32"
        assert np.all(d.astype(np.float32).astype(np.float64) == d)
    return d


def fp8_grain(n_rows: int) -> np.ndarray:
    """Finest value spacing of E4M3FN rows (per-tensor scale 1): the subnormal step."""
    return np.full(n_rows, 2.0 ** -9)


def mxfp4_grain(scales: np.ndarray) -> np.ndarray:
    """Finest value spacing of MXFP4 rows: E2M1 step 0.5 times the row's smallest
    block scale (scales [..., d/32] E8M0 bytes)."""
    s = np.asarray(scales).astype(np.float64).min(axis=-1)
    return np.exp2(s - 127.0) * 0.5


def fma_f32(a, b, c) -> np.ndarray:
    """fl32(a * b + c) with a single rounding (round to nearest even), elementwise,
    for binary32 a, b, c.  a * b is exact in binary64 (24 + 24 significand bits);
    the binary64 sum s = fl64(a*b + c) and its error e (a*b + c = s + e exactly,
    Knuth's TwoSum) then decide the result: s rounds to binary32 like the exact sum
    unless s lies exactly halfway between two binary32 neighbours and e != 0, when
    the exact sum is on the side of e."""
    p = np.asarray(a, np.float32).astype(np.float64) * np.asarray(b, np.float32).astype(np.float64)
    c64 = np.asarray(c, np.float32).astype(np.float64)
    p, c64 = np.broadcast_arrays(p, c64)
    s = p + c64
    bv = s - p
    e = (p - (s - bv)) + (c64 - bv)
    r = s.astype(np.float32)
    r64 = r.astype(np.float64)
    up = np.nextafter(r, np.float32(np.inf))
    dn = np.nextafter(r, np.float32(-np.inf))
    hi = np.where(r64 > s, r, up)                 # the binary32 neighbours bracketing s
    lo = np.where(r64 < s, r, dn)
    tie = (r64 != s) & (s - lo.astype(np.float64) == hi.astype(np.float64) - s)
    out = np.where(tie & (e > 0), hi, np.where(tie & (e < 0), lo, r))
    return out.astype(np.float32)


def score_canonical_f32(d: np.ndarray, w: np.ndarray) -> np.ndarray:
    """I[j] (float32) from exact head dots d [H_I, V] and weights w [H_I], in the
    canonical order above.  H_I must be a multiple of 32."""
    H_I, V = d.shape
    assert H_I % 32 == 0
    w32 = np.asarray(w, np.float32)
    relu = np.where(d > 0, d, 0.0).astype(np.float32)
    S = []
    for u in range(2):
        acc = np.zeros(V, np.float32)
        for T in range(H_I // 32):
            for i in range(16):
                h = 32 * T + 8 * (i // 4) + 4 * u + i % 4
                acc = fma_f32(w32[h], relu[h], acc)
        S.append(acc)
    return np.add(S[0], S[1], dtype=np.float32)


def score_f64(q: np.ndarray, k: np.ndarray, w: np.ndarray) -> np.ndarray:
    """I[j] (fp64) for f32 operands q [H_I, d_I], k [V, d_I], w [H_I]: dots summed
    sequentially over dims, terms summed sequentially over heads, no fused ops."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    w = np.asarray(w, np.float64)
    H_I, d_I = q.shape
    V = k.shape[0]
    acc = np.zeros(V)
    for h in range(H_I):
        dh = np.zeros(V)
        for i in range(d_I):
            dh = dh + q[h, i] * k[:, i]
        acc = acc + w[h] * np.where(dh > 0, dh, 0.0)
    return acc
