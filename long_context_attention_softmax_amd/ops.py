"""Python boundary over the C ABI: the entry points with the C names.

Each function checks dtypes, devices and layouts of PyTorch tensors, fills the
descriptor with raw device pointers and row pitches, and calls the library on the
current HIP stream.  Outputs are written into caller tensors (or allocated here);
workspaces are allocated once per (op, device, stream) and reused (the library needs
no particular contents in them).  There is no fallback: every result comes from the
HIP kernels.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _abi as A

_WS: dict = {}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must live on the GPU")


def _pitch(t: torch.Tensor) -> int:
    """Row pitch in bytes of a tensor whose last dim is contiguous and whose leading
    dims flatten to rows."""
    if t.stride(-1) != 1:
        raise ValueError("last dim must be contiguous")
    for i in range(t.dim() - 2):
        if t.stride(i) != t.stride(i + 1) * t.shape[i + 1]:
            raise ValueError("leading dims must flatten into rows")
    return (t.stride(-2) if t.dim() >= 2 else t.shape[-1]) * t.element_size()


def _set_pages(d, pages) -> None:
    """pages = (page_table [B, pages per sequence] int32, page_rows) or None."""
    if pages is None:
        return
    table, rows = pages
    if table.dtype != torch.int32 or table.dim() != 2 or not table.is_contiguous():
        raise ValueError("page_table must be a contiguous int32 [B, pages] tensor")
    _need_cuda(table)
    d.page_table, d.page_table_pitch, d.page_rows = _ptr(table), table.shape[1], int(rows)


def _seqs(cache_row_start, pages) -> int:
    return cache_row_start.numel() if cache_row_start is not None else pages[0].shape[0]


def _i64(t: torch.Tensor, n: int, name: str) -> torch.Tensor:
    if t.dtype != torch.int64 or t.numel() < n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int64 tensor of >= {n} elements")
    return t


def _workspace(op: int, nbytes: int, device) -> Optional[torch.Tensor]:
    """The scratch buffer of ``op`` for the current stream of ``device``.  Calls that
    share a workspace must be ordered on one stream, so each (op, device, stream)
    gets its own buffer: calls on different streams never share scratch."""
    if nbytes == 0:
        return None
    dev = device.index if device.index is not None else torch.cuda.current_device()
    key = (op, dev, torch.cuda.current_stream(dev).cuda_stream)
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        _WS[key] = ws
    off = (-ws.data_ptr()) % 256
    return ws[off:]


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _events(prof) -> "ctypes._Pointer":
    """The timing hook's event pair: prof = (begin, end) torch.cuda.Event objects."""
    for e in prof:
        if e.cuda_event == 0:             # torch creates an event on its first record
            e.record()
    ev = A.new_desc(A.ProfileEvents)
    ev.begin, ev.end = prof[0].cuda_event, prof[1].cuda_event
    return ctypes.byref(ev)


@dataclass
class KVCache:
    """Compressed KV planes: ``f32`` [N, D] float, or FP8 ``nope`` [N, D_n] uint8 +
    ``rope`` [N, D_r] int16/bfloat16 bits + ``scale`` [N] float."""
    f32: Optional[torch.Tensor] = None
    nope: Optional[torch.Tensor] = None
    rope: Optional[torch.Tensor] = None
    scale: Optional[torch.Tensor] = None

    @property
    def fmt(self) -> int:
        return A.F32 if self.f32 is not None else A.FP8_E4M3

    def planes(self) -> A.KvPlanes:
        p = A.KvPlanes()
        p.fmt = self.fmt
        if self.f32 is not None:
            _need_cuda(self.f32)
            if self.f32.dtype != torch.float32:
                raise ValueError("f32 plane must be float32")
            p.f32, p.f32_pitch = _ptr(self.f32), _pitch(self.f32)
        else:
            _need_cuda(self.nope, self.rope, self.scale)
            if self.nope.dtype != torch.uint8 or self.rope.element_size() != 2 or self.scale.dtype != torch.float32:
                raise ValueError("FP8 planes: nope uint8, rope 16-bit, scale float32")
            p.nope, p.nope_pitch = _ptr(self.nope), _pitch(self.nope)
            p.rope, p.rope_pitch = _ptr(self.rope), _pitch(self.rope)
            p.scale = _ptr(self.scale)
        return p


@dataclass
class IdxCache:
    """Indexer vectors: f32 [N, d_I] float, FP8 [N, d_I] uint8, or MXFP4 packed
    [N, d_I/2] uint8 + ``scales`` [N, d_I/32] uint8."""
    data: torch.Tensor
    fmt: int
    scales: Optional[torch.Tensor] = None

    def planes(self) -> A.IdxPlanes:
        _need_cuda(self.data, self.scales)
        p = A.IdxPlanes()
        p.fmt = self.fmt
        d = self.data.reshape(-1, self.data.shape[-1])
        p.data, p.pitch = _ptr(d), _pitch(d)
        if self.scales is not None:
            s = self.scales.reshape(-1, self.scales.shape[-1])
            p.scales, p.scale_pitch = _ptr(s), _pitch(s)
        return p


def _raw_fmt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return A.F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return A.BF16
    raise ValueError("raw rows must be float32 or bfloat16 (bits)")


def hca_kv_compress(*args, **kw) -> None:
    """Pool the listed blocks of ``raw`` rows into ``out`` (and ``out_idx``)."""
    d, _keep = _kv_compress_desc(*args, **kw)
    A.check(A.lib.hca_kv_compress(ctypes.byref(d), _stream()))


def _kv_compress_desc(raw: torch.Tensor, block_row: torch.Tensor, block_pos: torch.Tensor,
                      out_row: torch.Tensor, gate_w: torch.Tensor, gate_b: torch.Tensor,
                      out: KVCache, *, m: int, D_r: int, rope_base: float = 10000.0,
                      raw_idx: Optional[torch.Tensor] = None, out_idx: Optional[IdxCache] = None,
                      debug: Optional[torch.Tensor] = None):
    """The descriptor of a pooling call, and the tensors it points into."""
    raw2 = raw.reshape(-1, raw.shape[-1])
    n = block_row.numel()
    _need_cuda(raw2, block_row, block_pos, out_row, gate_w, gate_b, raw_idx, debug)
    d = A.new_desc(A.KvCompressDesc)
    d.m, d.D, d.D_r, d.n_blocks, d.rope_base = m, raw2.shape[1], D_r, n, rope_base
    d.raw_fmt = _raw_fmt(raw2)
    d.raw, d.raw_pitch = _ptr(raw2), _pitch(raw2)
    d.block_row = _ptr(_i64(block_row, n, "block_row"))
    d.block_pos = _ptr(_i64(block_pos, n, "block_pos"))
    d.out_row = _ptr(_i64(out_row, n, "out_row"))
    if gate_w.dtype != torch.float32 or gate_b.dtype != torch.float32:
        raise ValueError("gate_w and gate_b must be float32")
    gate_w, gate_b = gate_w.contiguous(), gate_b.contiguous()
    d.gate_w, d.gate_b = _ptr(gate_w), _ptr(gate_b)
    d.out = out.planes()
    if raw_idx is not None:
        ri = raw_idx.reshape(-1, raw_idx.shape[-1])
        if _raw_fmt(ri) != d.raw_fmt:
            raise ValueError("raw_idx must have raw's dtype")
        d.d_I = ri.shape[1]
        d.raw_idx, d.raw_idx_pitch = _ptr(ri), _pitch(ri)
        d.out_idx = out_idx.planes()
    if debug is not None:
        d.debug = _ptr(debug)
    return d, (raw2, gate_w, gate_b)


def hca_indexer_query_group(Nq: int, max_visible: int, fmt: int, k: int) -> int:
    """Queries per group of an indexer call of these shapes (Nq when it runs as one
    group; the last group holds the rest)."""
    d = A.new_desc(A.IndexerTopkDesc)
    d.Nq, d.k, d.max_visible = Nq, k, max_visible
    d.q.fmt = d.keys.fmt = fmt
    return A.indexer_query_group(d)


def hca_indexer_topk(*args, prof=None, **kw) -> torch.Tensor:
    """Top-k entries per query.  q.data is [Nq, H_I, ...]; returns idx [Nq, k] int32.
    ``pages`` = (page_table, page_rows) addresses a paged key cache instead of
    cache_row_start (see include/hca.h)."""
    d, idx, _keep = _indexer_desc(*args, **kw)
    if prof is not None:
        A.check(A.lib.hca_profiled(A.OP_INDEXER_TOPK, ctypes.byref(d), _events(prof), _stream()))
    else:
        A.check(A.lib.hca_indexer_topk(ctypes.byref(d), _stream()))
    return idx


def _indexer_desc(q: IdxCache, w: torch.Tensor, keys: IdxCache, cache_row_start: Optional[torch.Tensor],
                  seq_id: torch.Tensor, q_pos: torch.Tensor, *, k: int, m: int,
                  max_visible: int, idx: Optional[torch.Tensor] = None,
                  score: Optional[torch.Tensor] = None, pages=None):
    """The descriptor of an indexer call (its workspace attached), idx, and the tensors
    the descriptor points into."""
    Nq, H_I = q.data.shape[0], q.data.shape[1]
    d_I = q.data.shape[-1] * (2 if q.fmt == A.MXFP4 else 1)
    _need_cuda(w, cache_row_start, seq_id, q_pos, idx, score)
    if idx is None:
        idx = torch.empty((Nq, k), dtype=torch.int32, device=w.device)
    d = A.new_desc(A.IndexerTopkDesc)
    d.Nq, d.B, d.H_I, d.d_I, d.k, d.m = Nq, _seqs(cache_row_start, pages), H_I, d_I, k, m
    d.max_visible = max_visible
    d.q = q.planes()
    d.keys = keys.planes()
    if w.dtype != torch.float32 or not w.is_contiguous():
        raise ValueError("w must be contiguous float32 [Nq, H_I]")
    d.w = _ptr(w)
    if cache_row_start is not None:
        d.cache_row_start = _ptr(_i64(cache_row_start, 1, "cache_row_start"))
    _set_pages(d, pages)
    if seq_id.dtype != torch.int32:
        raise ValueError("seq_id must be int32")
    d.seq_id = _ptr(seq_id)
    d.q_pos = _ptr(_i64(q_pos, Nq, "q_pos"))
    d.idx = _ptr(idx)
    d.score = _ptr(score)
    nb = A.workspace_bytes(A.OP_INDEXER_TOPK, d)
    ws = _workspace(A.OP_INDEXER_TOPK, nb, w.device)
    d.workspace, d.workspace_bytes = _ptr(ws), nb
    return d, idx, (ws,)


def _attn(prefill: bool, *args, prof=None, noalloc: bool = False, **kw) -> torch.Tensor:
    d, o, _keep = _attn_desc(prefill, *args, workspace=not noalloc, **kw)
    op = A.OP_ATTN_PREFILL if prefill else A.OP_ATTN_DECODE
    if noalloc:                           # the library's static scratch; no workspace
        if prof is not None:
            raise ValueError("the allocation-free entry point has no timing hook")
        A.check(A.lib.hca_attn_decode_noalloc(ctypes.byref(d), _stream()))
    elif prof is not None:
        A.check(A.lib.hca_profiled(op, ctypes.byref(d), _events(prof), _stream()))
    else:
        fn = A.lib.hca_attn_prefill if prefill else A.lib.hca_attn_decode
        A.check(fn(ctypes.byref(d), _stream()))
    return o


def _attn_desc(prefill: bool, q: torch.Tensor, cache: Optional[KVCache], cache_row_start: Optional[torch.Tensor],
               win: torch.Tensor, sink: torch.Tensor, seq_id: torch.Tensor, q_pos: torch.Tensor, *,
               mode: int, m: int, n_win: int, D_r: int, max_visible: int, k: int = 0,
               idx: Optional[torch.Tensor] = None, tau: float = 1.0, rope_base: float = 10000.0,
               o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               pages=None, split_chunks: int = 0, workspace: bool = True):
    """The descriptor of an attention call (with its workspace unless ``workspace`` is
    False), the output o, and the tensors the descriptor points into."""
    Nq, H, D = q.shape
    _need_cuda(q, cache_row_start, win, sink, seq_id, q_pos, idx, o, lse)
    io = A.F32 if q.dtype == torch.float32 else A.BF16
    if io == A.BF16 and q.dtype != torch.bfloat16:
        q = q.view(torch.bfloat16)
    if o is None:
        o = torch.empty_like(q)
    d = A.new_desc(A.AttnDesc)
    d.Nq, d.H, d.D, d.D_r = Nq, H, D, D_r
    d.B = _seqs(cache_row_start, pages) if (cache_row_start is not None or pages) else win.shape[0]
    d.mode, d.m, d.k, d.n_win, d.win_cap = mode, m, k, n_win, win.shape[-2]
    d.tau, d.io_fmt, d.rope_base, d.max_visible = tau, io, rope_base, max_visible
    d.split_chunks = split_chunks
    if not q.is_contiguous():
        raise ValueError("q must be contiguous [Nq, H, D]")
    d.q = _ptr(q)
    if cache is not None:                  # None: the window-only mode reads no cache
        d.cache = cache.planes()
    if cache_row_start is not None:
        d.cache_row_start = _ptr(_i64(cache_row_start, 1, "cache_row_start"))
    _set_pages(d, pages)
    if idx is not None:
        if idx.dtype != torch.int32 or not idx.is_contiguous():
            raise ValueError("idx must be contiguous int32 [Nq, k]")
        d.idx = _ptr(idx)
    w2 = win.reshape(-1, win.shape[-1])
    d.win, d.win_pitch = _ptr(w2), _pitch(w2)
    sink = sink.contiguous()
    d.sink = _ptr(sink)
    d.seq_id = _ptr(seq_id)
    d.q_pos = _ptr(_i64(q_pos, Nq, "q_pos"))
    d.o = _ptr(o)
    d.lse = _ptr(lse)
    ws = None
    if workspace:
        op = A.OP_ATTN_PREFILL if prefill else A.OP_ATTN_DECODE
        nb = A.workspace_bytes(op, d)
        ws = _workspace(op, nb, q.device)
        d.workspace, d.workspace_bytes = _ptr(ws), nb
    return d, o, (q, w2, sink, ws)


def hca_decode_layer(attn: dict, pool: Optional[dict] = None, indexer: Optional[dict] = None,
                     prof=None) -> torch.Tensor:
    """One decode step of one layer in one library call (see include/hca.h): ``pool``,
    ``indexer`` and ``attn`` hold the keyword arguments of hca_kv_compress,
    hca_indexer_topk (CSA only; its idx is the one attention reads) and
    hca_attn_decode.  ``prof`` brackets the scoring launch (CSA) or the attention
    kernel (HCA, sliding window).  Returns o."""
    keep = []
    d = A.new_desc(A.DecodeLayerDesc)
    if pool is not None:
        pd, k1 = _kv_compress_desc(**pool)
        keep += [pd, k1]
        d.pool = ctypes.pointer(pd)
    if indexer is not None:
        idd, _idx, k2 = _indexer_desc(**indexer)
        keep += [idd, k2]
        d.indexer = ctypes.pointer(idd)
    ad, o, k3 = _attn_desc(False, **attn)
    keep += [ad, k3]
    d.attn = ctypes.pointer(ad)
    if prof is not None:
        A.check(A.lib.hca_profiled(A.OP_DECODE_LAYER, ctypes.byref(d), _events(prof), _stream()))
    else:
        A.check(A.lib.hca_decode_layer(ctypes.byref(d), _stream()))
    return o


def hca_attn_decode(*args, **kw) -> torch.Tensor:
    """One-softmax attention of decode queries (see include/hca.h)."""
    return _attn(False, *args, **kw)


def hca_attn_decode_noalloc(*args, **kw) -> torch.Tensor:
    """hca_attn_decode through the allocation-free entry point: the library's static
    scratch instead of a workspace (pass ``o`` and ``lse`` to allocate nothing here
    either; see include/hca.h for the size limit and the one-call-at-a-time rule)."""
    return _attn(False, *args, noalloc=True, **kw)


def hca_attn_prefill(*args, **kw) -> torch.Tensor:
    """One-softmax attention of a chunk of consecutive query positions."""
    return _attn(True, *args, **kw)


def hca_qkv_prologue(q_in: Optional[torch.Tensor], gamma_q: Optional[torch.Tensor],
                     kv_in: Optional[torch.Tensor], gamma_kv: Optional[torch.Tensor],
                     tok_seq: Optional[torch.Tensor], tok_pos: Optional[torch.Tensor],
                     win: Optional[torch.Tensor], *, eps: float = 1e-6,
                     q_out: Optional[torch.Tensor] = None, idx_in: Optional[torch.Tensor] = None,
                     win_idx: Optional[torch.Tensor] = None) -> Optional[torch.Tensor]:
    """Normalize q ([Nq, H, D], into ``q_out``, default in place) and the new tokens
    ``kv_in`` ([Nt, D]), writing each token to the ring ``win`` ([B, W_cap, D]) at
    (tok_seq, tok_pos mod W_cap); ``idx_in`` rows are copied to ``win_idx`` at the
    same slots (see include/hca.h).  Returns q_out."""
    _need_cuda(q_in, gamma_q, kv_in, gamma_kv, tok_seq, tok_pos, win, q_out, idx_in, win_idx)
    d = A.new_desc(A.QkvPrologueDesc)
    ref = q_in if q_in is not None else kv_in
    if ref is None:
        raise ValueError("nothing to do: q_in and kv_in are both None")
    d.io_fmt = A.F32 if ref.dtype == torch.float32 else A.BF16
    d.eps = float(eps)
    d.D = ref.shape[-1]
    if q_in is not None:
        if not q_in.is_contiguous() or q_in.dim() != 3:
            raise ValueError("q_in must be contiguous [Nq, H, D]")
        q_out = q_in if q_out is None else q_out
        if q_out.shape != q_in.shape or q_out.dtype != q_in.dtype or not q_out.is_contiguous():
            raise ValueError("q_out must match q_in")
        d.Nq, d.H = q_in.shape[0], q_in.shape[1]
        d.q_in, d.q_out, d.gamma_q = _ptr(q_in), _ptr(q_out), _ptr(_f32(gamma_q, d.D, "gamma_q"))
    if kv_in is not None:
        if kv_in.dim() != 2 or win.dim() != 3:
            raise ValueError("kv_in must be [Nt, D] and win [B, W_cap, D]")
        if tok_seq.dtype != torch.int32:
            raise ValueError("tok_seq must be int32")
        d.Nt, d.B, d.W_cap = kv_in.shape[0], win.shape[0], win.shape[1]
        d.kv_in, d.kv_pitch, d.gamma_kv = _ptr(kv_in), _pitch(kv_in), _ptr(_f32(gamma_kv, d.D, "gamma_kv"))
        d.tok_seq, d.tok_pos = _ptr(tok_seq.contiguous()), _ptr(_i64(tok_pos, d.Nt, "tok_pos"))
        w2 = win.reshape(-1, win.shape[-1])
        d.win, d.win_pitch = _ptr(w2), _pitch(w2)
        if idx_in is not None:
            wi = win_idx.reshape(-1, win_idx.shape[-1])
            d.d_I = idx_in.shape[-1]
            d.idx_in, d.idx_pitch, d.win_idx, d.win_idx_pitch = _ptr(idx_in), _pitch(idx_in), _ptr(wi), _pitch(wi)
    A.check(A.lib.hca_qkv_prologue(ctypes.byref(d), _stream()))
    return q_out


def _f32(t: torch.Tensor, n: int, name: str) -> torch.Tensor:
    if t is None or t.dtype != torch.float32 or t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor of {n} elements")
    return t


def hca_out_proj(o: torch.Tensor, w: torch.Tensor, *, G: int, y: Optional[torch.Tensor] = None,
                 out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Grouped output projection (see include/hca.h): o [Nq, H, D] BF16, w [G, d_g, K_g]
    BF16 with K_g = H / G * D; returns y [Nq, G, d_g] (float32 or bfloat16)."""
    _need_cuda(o, w, y)
    if o.dim() != 3 or not o.is_contiguous() or w.dim() != 3 or not w.is_contiguous():
        raise ValueError("o must be contiguous [Nq, H, D] and w contiguous [G, d_g, K_g]")
    Nq, H, D = o.shape
    d_g = w.shape[1]
    if y is None:
        y = torch.empty((Nq, G, d_g), dtype=out_dtype, device=o.device)
    if not y.is_contiguous() or y.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("y must be contiguous float32 or bfloat16 [Nq, G, d_g]")
    d = A.new_desc(A.OutProjDesc)
    d.out_fmt = A.F32 if y.dtype == torch.float32 else A.BF16
    d.Nq, d.H, d.D, d.G, d.d_g = Nq, H, D, G, d_g
    d.o, d.o_pitch = _ptr(o), H * D * 2
    d.w, d.w_pitch = _ptr(w), w.shape[2] * 2
    d.y, d.y_pitch = _ptr(y), G * d_g * y.element_size()
    A.check(A.lib.hca_out_proj(ctypes.byref(d), _stream()))
    return y
