"""One attention layer's device buffers and its step through the four entry points.

A step, per layer ("DeepSeek Releases V4 ..." (botbeat.news), "Summary";
"DeepSeek V4: How They Crushed the Million-Token Memory Problem"
(sameershanbhag.com), "Two kinds of memory instead of one"):
  1. hca_kv_compress pools the blocks the new tokens complete;
  2. CSA only: hca_indexer_topk scores the visible entries and keeps the top-k;
  3. hca_attn_decode / hca_attn_prefill attends with one softmax over the entries,
     the window and the sink.
All three are enqueued on the current stream with no host round trip.

``DeviceLayer.from_host`` takes any object carrying the layer's host arrays
(numpy) under the attribute names used below, uploads them once, and keeps them
resident; ``step()`` then only launches kernels.

With ``page_rows`` the compressed cache (KV entries and, for CSA, indexer keys) is
laid out in pages of that many rows, placed at seeded-random physical slots, and
addressed through one block table per layer instead of contiguous per-sequence
runs: the cache format that continuous batching needs ("DeepSeek V4
infrastructure" (volanea.com), "Compression only works if the attention path is
engineered end to end").  The host arrays stay the logical, contiguous layout;
``phys_rows`` maps their row numbers to the device rows.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import _abi as A
from .ops import (IdxCache, KVCache, hca_attn_decode, hca_attn_prefill, hca_decode_layer, hca_indexer_topk,
                  hca_kv_compress)


def _page_layout(starts: np.ndarray, n_rows: int, max_visible: int, page_rows: int, seed: int):
    """Block table and logical->physical row map of a paged cache.

    Sequence b owns logical rows [starts[b], next start) (host layout); its j-th row
    goes to page table[b, j // page_rows], row j % page_rows.  The pages of all
    sequences, plus spare ones that stay unreferenced, are shuffled over the
    physical cache.  Table slots past a sequence's pages name a spare page."""
    if page_rows < 1 or page_rows & (page_rows - 1):
        raise ValueError("page_rows must be a power of two")
    starts = np.asarray(starts, np.int64)
    order = np.argsort(starts, kind="stable")
    ends = np.empty_like(starts)
    ends[order] = np.append(starts[order][1:], n_rows)
    lens = ends - starts
    npages = (lens + page_rows - 1) // page_rows
    pitch = int(max(1, npages.max(initial=0), -(-max_visible // page_rows)))
    used = int(npages.sum())
    total = used + max(2, used // 8)
    perm = np.random.default_rng(seed).permutation(total).astype(np.int32)
    table = np.full((len(starts), pitch), perm[-1], np.int32)
    phys = np.empty(n_rows, np.int64)
    k = 0
    for b in range(len(starts)):
        table[b, :npages[b]] = perm[k:k + npages[b]]
        k += int(npages[b])
        j = np.arange(lens[b], dtype=np.int64)
        phys[starts[b] + j] = table[b, j // page_rows].astype(np.int64) * page_rows + j % page_rows
    return table, phys, total * page_rows


def _scatter_rows(x: np.ndarray, phys: np.ndarray, n_phys: int, rng) -> np.ndarray:
    """x's rows at their physical places; rows no page holds get random bytes."""
    if x.shape[0] != len(phys):
        raise ValueError(f"cache array has {x.shape[0]} rows, layout {len(phys)}")
    out = np.empty((n_phys,) + x.shape[1:], x.dtype)
    out[phys] = x
    free = np.ones(n_phys, bool)
    free[phys] = False
    junk = rng.integers(0, 256, (int(free.sum()), out[0].nbytes), dtype=np.uint8)
    out[free] = junk.view(x.dtype).reshape((-1,) + x.shape[1:])
    return out


def _t(x, device, dtype=None):
    a = np.ascontiguousarray(x)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a).to(device)
    return t if dtype is None else t.view(dtype)


class DeviceLayer:
    """Resident buffers of one layer (CSA or HCA) for a batch of queries."""

    def __init__(self):
        self.idx: Optional[torch.Tensor] = None
        self.o: Optional[torch.Tensor] = None
        self.lse: Optional[torch.Tensor] = None
        self.pages = None            # (page_table [B, pitch] int32, page_rows) when paged
        self.split_chunks = 0        # decode: > 0 = fixed split, batch-invariant outputs
        self._phys: Optional[np.ndarray] = None

    def phys_rows(self, rows) -> np.ndarray:
        """Device cache rows of the host layout's rows."""
        rows = np.asarray(rows, np.int64)
        return rows if self._phys is None else self._phys[rows]

    @classmethod
    def from_host(cls, lay, g, device="cuda", page_rows: Optional[int] = None,
                  page_seed: int = 0) -> "DeviceLayer":
        d = cls()
        d.mode = {"csa": A.MODE_CSA, "hca": A.MODE_HCA, "swa": A.MODE_SWA}[lay.mode]
        if d.mode == A.MODE_SWA:
            return cls._window_only(d, lay, g, torch.device(device))
        d.m, d.g, d.device = lay.m, g, torch.device(device)
        d.f32 = lay.fmt == "f32"
        dev = d.device
        d.max_visible = int(((lay.q_pos + 1) // lay.m).max()) if len(lay.q_pos) else 0
        rows = lambda x: x                                   # noqa: E731
        if page_rows is not None:
            table, d._phys, n_phys = _page_layout(lay.cache_row_start, int(lay.n_rows), d.max_visible,
                                                  page_rows, page_seed)
            fill = np.random.default_rng(page_seed + 1)
            rows = lambda x: _scatter_rows(x, d._phys, n_phys, fill)   # noqa: E731
            d.pages = (_t(table, dev), page_rows)
        if d.f32:
            d.cache = KVCache(f32=_t(rows(lay.cache_f32), dev))
            d.win = _t(lay.win, dev)
            d.q = _t(lay.q, dev)
        else:
            d.cache = KVCache(nope=_t(rows(lay.cache_nope), dev),
                              rope=_t(rows(lay.cache_rope), dev, torch.bfloat16),
                              scale=_t(rows(lay.cache_scale), dev))
            d.win = _t(lay.win, dev, torch.bfloat16)
            d.q = _t(lay.q, dev, torch.bfloat16)
        d.W_cap = lay.W_cap
        d.cache_row_start = None if d.pages else _t(lay.cache_row_start.astype(np.int64), dev)
        d.q_pos = _t(lay.q_pos.astype(np.int64), dev)
        d.seq_id = _t(lay.seq_id.astype(np.int32), dev)
        d.sink = _t(lay.sink.astype(np.float32), dev)
        d.gate_w = _t(lay.gate_w.astype(np.float32), dev)
        d.gate_b = _t(lay.gate_b.astype(np.float32), dev)
        p = lay.pool
        d.block_row = _t(p["block_row"].astype(np.int64), dev)
        d.block_pos = _t(p["block_pos"].astype(np.int64), dev)
        d.out_row = _t(d.phys_rows(p["out_row"]), dev)
        d.Nq = len(lay.q_pos)
        d.win_idx = None
        if d.mode == A.MODE_CSA:
            fmt = {"f32": A.F32, "fp8": A.FP8_E4M3, "mxfp4": A.MXFP4}[lay.idx_fmt]
            if fmt == A.F32:
                d.keys = IdxCache(_t(rows(lay.idx_f32), dev), fmt)
                d.qI = IdxCache(_t(lay.q_I, dev), fmt)
            elif fmt == A.FP8_E4M3:
                d.keys = IdxCache(_t(rows(lay.idx_fp8), dev), fmt)
                d.qI = IdxCache(_t(lay.q_I, dev), fmt)
            else:
                d.keys = IdxCache(_t(rows(lay.idx_codes), dev), fmt, _t(rows(lay.idx_scales), dev))
                d.qI = IdxCache(_t(lay.q_I, dev), fmt, _t(lay.q_I_scales, dev))
            d.w = _t(lay.w.astype(np.float32), dev)
            if getattr(lay, "win_idx", None) is not None:
                d.win_idx = _t(lay.win_idx, dev, None if d.f32 else torch.bfloat16)
            d.idx = torch.empty((d.Nq, g.topk), dtype=torch.int32, device=dev)
        d.o = torch.empty_like(d.q)
        d.lse = torch.empty((d.Nq, g.H), dtype=torch.float32, device=dev)
        return d

    @staticmethod
    def _window_only(d, lay, g, dev):
        """The sliding-window-only layer: ring, queries and sink; no cache."""
        d.m, d.g, d.device, d.f32 = 1, g, dev, lay.fmt == "f32"
        d.win = _t(lay.win, dev, None if d.f32 else torch.bfloat16)
        d.q = _t(lay.q, dev, None if d.f32 else torch.bfloat16)
        d.W_cap, d.max_visible, d.Nq = lay.W_cap, 0, len(lay.q_pos)
        d.cache = d.cache_row_start = None
        d.q_pos = _t(lay.q_pos.astype(np.int64), dev)
        d.seq_id = _t(lay.seq_id.astype(np.int32), dev)
        d.sink = _t(lay.sink.astype(np.float32), dev)
        d.o = torch.empty_like(d.q)
        d.lse = torch.empty((d.Nq, g.H), dtype=torch.float32, device=dev)
        return d

    # ----------------------------------------------------------------- steps
    def _pool_kw(self, debug: Optional[torch.Tensor] = None) -> dict:
        g = self.g
        csa = self.mode == A.MODE_CSA
        return dict(raw=self.win, block_row=self.block_row, block_pos=self.block_pos, out_row=self.out_row,
                    gate_w=self.gate_w, gate_b=self.gate_b, out=self.cache, m=self.m, D_r=g.D_r,
                    rope_base=g.rope_base, raw_idx=self.win_idx if csa else None,
                    out_idx=self.keys if csa else None, debug=debug)

    def _select_kw(self, score: Optional[torch.Tensor] = None, queries: Optional[slice] = None) -> dict:
        g = self.g
        qs = queries if queries is not None else slice(None)
        qI = IdxCache(self.qI.data[qs], self.qI.fmt, None if self.qI.scales is None else self.qI.scales[qs])
        return dict(q=qI, w=self.w[qs], keys=self.keys, cache_row_start=self.cache_row_start,
                    seq_id=self.seq_id[qs], q_pos=self.q_pos[qs], k=g.topk, m=self.m,
                    max_visible=self.max_visible, idx=self.idx[qs],
                    score=None if score is None else score[qs], pages=self.pages)

    def _attend_kw(self) -> dict:
        g = self.g
        csa = self.mode == A.MODE_CSA
        return dict(q=self.q, cache=self.cache, cache_row_start=self.cache_row_start, win=self.win,
                    sink=self.sink, seq_id=self.seq_id, q_pos=self.q_pos, mode=self.mode, m=self.m,
                    n_win=g.n_win, D_r=g.D_r, max_visible=self.max_visible, k=g.topk if csa else 0,
                    idx=self.idx if csa else None, tau=g.tau, rope_base=g.rope_base, o=self.o,
                    lse=self.lse, pages=self.pages, split_chunks=self.split_chunks)

    def pool(self, debug: Optional[torch.Tensor] = None):
        if self.mode == A.MODE_SWA:
            return
        hca_kv_compress(**self._pool_kw(debug))

    def select(self, score: Optional[torch.Tensor] = None, prof=None, queries: Optional[slice] = None):
        """Indexer top-k of every query, or of the queries in ``queries`` (a slice)."""
        return hca_indexer_topk(**self._select_kw(score, queries), prof=prof)

    def attend(self, prefill: bool = False, prof=None):
        fn = hca_attn_prefill if prefill else hca_attn_decode
        return fn(**self._attend_kw(), prof=prof)

    def step(self, prefill: bool = False, pool: bool = True, prof_select=None, prof_attend=None,
             fused: bool = True):
        """pool -> (CSA) select -> attend.  Decode runs as one hca_decode_layer call
        (``fused`` False: the three calls one after another, the same results)."""
        csa = self.mode == A.MODE_CSA
        if prefill or not fused:
            if pool:
                self.pool()
            if csa:
                self.select(prof=prof_select)
            return self.attend(prefill, prof=prof_attend)
        return hca_decode_layer(self._attend_kw(),
                                pool=self._pool_kw() if pool and self.mode != A.MODE_SWA else None,
                                indexer=self._select_kw() if csa else None,
                                prof=prof_select if csa else prof_attend)

    def clone(self) -> "DeviceLayer":
        """An independent copy of every device buffer (same shapes and contents)."""
        c = DeviceLayer()
        for k, v in self.__dict__.items():
            if isinstance(v, torch.Tensor):
                v = v.clone()
            elif isinstance(v, tuple) and k == "pages":
                v = (v[0].clone(), v[1])
            elif isinstance(v, (KVCache, IdxCache)):
                v = type(v)(**{f: (getattr(v, f).clone() if isinstance(getattr(v, f), torch.Tensor)
                                   else getattr(v, f)) for f in v.__dataclass_fields__})
            setattr(c, k, v)
        return c
