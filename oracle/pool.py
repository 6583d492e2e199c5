"""Softmax-gated pooling of the shared-KV stream into compressed entries (oracle side).

"DeepSeek Releases V4 with Million-Token Context Optimized for AI Agents"
(botbeat.news), "Summary": CSA compresses KV entries 4x by softmax-gated pooling
with a learned positional bias, HCA compresses 128x.  "DeepSeek V4: How They
Crushed the Million-Token Memory Problem" (sameershanbhag.com), "Two kinds of
memory instead of one": every 4 (CSA) or 128 (HCA) tokens become one KV entry.
"Inside DeepSeek V4 ..." (jakobijn.be), "The Architecture: Hybrid Attention
(CSA + HCA)": the indexer searches over these summaries.

Readings (no formula is printed):
  * blocks are the aligned, non-overlapping groups of m tokens [jm, jm+m);
  * each token gets a scalar gate logit z = g . x + b[pos mod m] from its
    un-rotated raw vector x (all D dims);
  * the block's weights are alpha = softmax(z) over its m tokens;
  * the entry is c = sum_i alpha_i x_i, and its RoPE slice is then rotated at the
    block's last position p_j = jm + m - 1;
  * the CSA indexer key is pooled from the raw indexer-key stream with the same alpha.
"""
from __future__ import annotations

import numpy as np

from . import quant, rope


def gate_logits(x_blk: np.ndarray, gate_w: np.ndarray, gate_b: np.ndarray) -> np.ndarray:
    """z_i = g . x_i + b_i for the m tokens of one aligned block (fp64)."""
    x = np.asarray(x_blk, np.float64)
    return x @ np.asarray(gate_w, np.float64) + np.asarray(gate_b, np.float64)


def pool_weights(z: np.ndarray) -> np.ndarray:
    """Softmax over the block's m gate logits."""
    z = np.asarray(z, np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def pool_block(x_blk, gate_w, gate_b, y_blk=None):
    """(alpha, c_hat, y_hat): the weights, the pooled un-rotated KV entry and the pooled
    indexer key (None without an indexer stream)."""
    alpha = pool_weights(gate_logits(x_blk, gate_w, gate_b))
    c_hat = alpha @ np.asarray(x_blk, np.float64)
    y_hat = None if y_blk is None else alpha @ np.asarray(y_blk, np.float64)
    return alpha, c_hat, y_hat


def compress_block(x_blk, gate_w, gate_b, block_pos: int, D_r: int, base: float, y_blk=None):
    """Pre-quantization entry [c_nope ; R(p_j) c_rope] (fp64) and pooled indexer key."""
    m = x_blk.shape[0]
    _, c_hat, y_hat = pool_block(x_blk, gate_w, gate_b, y_blk)
    entry = rope.apply(c_hat, block_pos + m - 1, D_r, base)
    return entry, y_hat


def encode_entry(entry: np.ndarray, D_r: int, kv_fmt: str):
    """Encode pre-quantization entries [n, D].

    ``f32``: one f32 plane.  ``fp8``: nope dims to FP8 with a per-entry power-of-two
    scale (smallest 2^e with amax <= 448*2^e), RoPE dims to BF16, scale as f32.
    Returns a dict of planes plus a per-element ``fragile`` mask [n, D].
    """
    e = np.asarray(entry, np.float64)
    if kv_fmt == "f32":
        v, fr = quant.f32_round(e)
        return dict(f32=v.astype(np.float32), fragile=fr)
    nope, rp = e[:, :-D_r], e[:, -D_r:]
    s, s_fr = quant.entry_scale(nope)
    codes, n_fr = quant.fp8_encode(nope / s[:, None], return_fragile=True)
    bits, r_fr = quant.bf16_encode(rp, return_fragile=True)
    fragile = np.concatenate([n_fr | s_fr[:, None], r_fr], axis=1)
    return dict(nope=codes, rope=bits, scale=s.astype(np.float32), fragile=fragile, scale_fragile=s_fr)


def encode_idx(y_hat: np.ndarray, idx_fmt: str):
    """Encode pooled indexer keys [n, d_I]: f32, FP8 (per-tensor scale 1) or MXFP4."""
    y = np.asarray(y_hat, np.float64)
    if idx_fmt == "f32":
        v, fr = quant.f32_round(y)
        return dict(f32=v.astype(np.float32), fragile=fr)
    if idx_fmt == "fp8":
        codes, fr = quant.fp8_encode(y, return_fragile=True)
        return dict(fp8=codes, fragile=fr)
    packed, scales, fr = quant.mxfp4_encode(y, return_fragile=True)
    return dict(codes=packed, scales=scales, fragile=fr)


def kv_compress(raw: np.ndarray, block_row, block_pos, gate_w, gate_b, m: int, D_r: int,
                base: float, kv_fmt: str, raw_idx: np.ndarray | None = None,
                idx_fmt: str | None = None):
    """Pool every listed block.

    ``raw`` [R, D] (and ``raw_idx`` [R, d_I]) are decoded raw rows (fp64); block n
    uses rows block_row[n] .. block_row[n]+m-1, whose first token sits at absolute
    position block_pos[n] (a multiple of m).  Returns the encoded planes, the
    pre-quantization values and the fragile masks.
    """
    n = len(block_row)
    D = raw.shape[1]
    entries = np.zeros((n, D))
    yh = None if raw_idx is None else np.zeros((n, raw_idx.shape[1]))
    for i in range(n):
        r0, p0 = int(block_row[i]), int(block_pos[i])
        assert p0 % m == 0
        xb = raw[r0:r0 + m]
        yb = None if raw_idx is None else raw_idx[r0:r0 + m]
        entries[i], y = compress_block(xb, gate_w, gate_b, p0, D_r, base, yb)
        if yh is not None:
            yh[i] = y
    out = dict(entry=entries, kv=encode_entry(entries, D_r, kv_fmt))
    if yh is not None:
        out["y"] = yh
        out["idx"] = encode_idx(yh, idx_fmt)
    return out
