"""One pass of the hybrid compressed-attention path for one layer (oracle side).

Order of a step, for each layer ("DeepSeek Releases V4 ..." (botbeat.news),
"Summary"; "DeepSeek V4: How They Crushed the Million-Token Memory Problem"
(sameershanbhag.com), "Two kinds of memory instead of one"):
  1. pool every block that is complete and not yet in the cache;
  2. CSA only: score every visible compressed entry with the indexer and keep the
     top-k per query;
  3. attend with one softmax over the selected (CSA) or all visible (HCA) entries,
     the sliding window and the sink.

Inputs are the stored bytes a workload holds (f32 planes, or FP8/BF16/MXFP4 codes);
they are decoded exactly to fp64 here.
"""
from __future__ import annotations

import numpy as np

from . import quant, pool, indexer, topk, attend

_FP8_LUT = quant.fp8_decode(np.arange(256))


def fp8_values(codes):
    return _FP8_LUT[np.asarray(codes)]


def raw_values(ring, fmt):
    """Decoded raw rows of a window ring (f32 array or BF16 bits) as fp64."""
    return np.asarray(ring, np.float64) if fmt == "f32" else quant.bf16_decode(ring)


def pool_layer(lay, g):
    """Pool the blocks a layer lists; returns the oracle's kv_compress result."""
    W = lay.W_cap
    raw = raw_values(lay.win, lay.fmt).reshape(-1, g.D)
    p = lay.pool
    has_idx = lay.mode == "csa" and hasattr(lay, "win_idx")
    raw_idx = raw_values(lay.win_idx, lay.fmt).reshape(-1, g.d_I) if has_idx else None
    kv_fmt = "f32" if lay.fmt == "f32" else "fp8"
    res = pool.kv_compress(raw, p["block_row"], p["block_pos"], lay.gate_w, lay.gate_b, lay.m,
                           g.D_r, g.rope_base, kv_fmt, raw_idx, lay.idx_fmt if has_idx else None)
    res["out_row"] = np.asarray(p["out_row"])
    del W
    return res


class _Cache:
    """Read access to a layer's compressed cache with the step's pooled rows laid over."""

    def __init__(self, lay, g, pooled):
        self.lay, self.g = lay, g
        self.over = {int(r): i for i, r in enumerate(pooled["out_row"])}
        self.kv = pooled["kv"]
        self.idx = pooled.get("idx")

    def entries(self, rows):
        lay, g = self.lay, self.g
        rows = np.asarray(rows, np.int64)
        if lay.fmt == "f32":
            out = np.asarray(lay.cache_f32[rows], np.float64)
        else:
            out = np.concatenate([fp8_values(lay.cache_nope[rows]) * lay.cache_scale[rows, None],
                                  quant.bf16_decode(lay.cache_rope[rows])], axis=1)
        for n, r in enumerate(rows):
            i = self.over.get(int(r))
            if i is None:
                continue
            if lay.fmt == "f32":
                out[n] = self.kv["f32"][i]
            else:
                out[n] = np.concatenate([fp8_values(self.kv["nope"][i]) * float(self.kv["scale"][i]),
                                         quant.bf16_decode(self.kv["rope"][i])])
        return out

    def idx_keys(self, rows):
        """(values [n, d_I] fp64, grain [n])"""
        lay = self.lay
        rows = np.asarray(rows, np.int64)
        if lay.idx_fmt == "f32":
            v = np.asarray(lay.idx_f32[rows], np.float64)
            gr = None
        elif lay.idx_fmt == "fp8":
            v = fp8_values(lay.idx_fp8[rows])
            gr = indexer.fp8_grain(len(rows))
        else:
            v = quant.mxfp4_decode(lay.idx_codes[rows], lay.idx_scales[rows])
            gr = indexer.mxfp4_grain(lay.idx_scales[rows])
        for n, r in enumerate(rows):
            i = self.over.get(int(r))
            if i is None:
                continue
            if lay.idx_fmt == "f32":
                v[n] = self.idx["f32"][i]
            elif lay.idx_fmt == "fp8":
                v[n] = fp8_values(self.idx["fp8"][i])
            else:
                v[n] = quant.mxfp4_decode(self.idx["codes"][i], self.idx["scales"][i])
                gr[n] = indexer.mxfp4_grain(self.idx["scales"][i][None])[0]
        return v, gr


def query_values(lay, qi):
    if lay.fmt == "f32":
        return np.asarray(lay.q[qi], np.float64)
    return quant.bf16_decode(lay.q[qi])


def index_query_values(lay, qi):
    """(q_I values [H_I, d_I], grain [H_I])"""
    if lay.idx_fmt == "f32":
        return np.asarray(lay.q_I[qi], np.float64), None
    if lay.idx_fmt == "fp8":
        return fp8_values(lay.q_I[qi]), indexer.fp8_grain(lay.q_I.shape[1])
    return (quant.mxfp4_decode(lay.q_I[qi], lay.q_I_scales[qi]),
            indexer.mxfp4_grain(lay.q_I_scales[qi]))


def scores_for_query(cache: _Cache, lay, g, qi, t, b):
    V = topk.n_visible(t, lay.m)
    rows = int(lay.cache_row_start[b]) + np.arange(V)
    kv, kgr = cache.idx_keys(rows)
    qv, qgr = index_query_values(lay, qi)
    w = lay.w[qi]
    if lay.idx_fmt == "f32":
        return indexer.score_f64(qv, kv, w)
    d = indexer.head_dots_exact(qv, kv, qgr, kgr)
    return indexer.score_canonical_f32(d, w)


def run_layer(lay, g, queries=None, pooled=None):
    """Oracle step of one layer.  ``queries``: indices of the queries to evaluate
    (default all).  Returns pooled entries, idx [nq, k] (CSA), scores, o [nq, H, D]
    and lse [nq, H].

    Layer modes: "csa" and "hca" as above; "swa" is the sliding-window-only block
    ("DeepSeek V4: How They Crushed the Million-Token Memory Problem"
    (sameershanbhag.com), "Two kinds of memory instead of one": the final
    multi-token-prediction block runs sliding-window only): no compressed entries,
    nothing pooled, the set is the window tokens alone (pooled is then None)."""
    swa = lay.mode == "swa"
    if pooled is None and not swa:
        pooled = pool_layer(lay, g)
    cache = None if swa else _Cache(lay, g, pooled)
    nq_all = len(lay.q_pos)
    qs = np.arange(nq_all) if queries is None else np.asarray(queries)
    ring = raw_values(lay.win, lay.fmt)
    out_o = np.zeros((len(qs), g.H, g.D))
    out_lse = np.zeros((len(qs), g.H))
    out_idx = np.full((len(qs), g.topk), -1, np.int64) if lay.mode == "csa" else None
    out_sel = np.zeros((len(qs), g.topk)) if lay.mode == "csa" else None
    gaps = []
    for n, qi in enumerate(qs):
        t, b = int(lay.q_pos[qi]), int(lay.seq_id[qi])
        V = topk.n_visible(t, lay.m)
        if lay.mode == "csa":
            I = scores_for_query(cache, lay, g, qi, t, b)
            sel = topk.select(I, g.topk)
            out_idx[n] = sel
            out_sel[n, sel >= 0] = I[sel[sel >= 0]]
            gaps.append(topk.kth_gap(I, g.topk))
            js = sel[sel >= 0]
        elif not swa:
            js = np.arange(V)
        ent = np.zeros((0, g.D)) if swa else cache.entries(int(lay.cache_row_start[b]) + js)
        win = attend.window_keys(ring, b, t, g.n_win, lay.W_cap, g.D_r, g.rope_base)
        keys = np.concatenate([ent, win], axis=0)
        qh = attend.query_hat(query_values(lay, qi), t, g.D_r, g.rope_base)
        out_o[n], out_lse[n] = attend.attend(qh, keys, lay.sink, g.tau)
    return dict(pooled=pooled, idx=out_idx, sel_scores=out_sel, o=out_o, lse=out_lse, queries=qs,
                kth_gaps=gaps)
