"""Seeded generators for the five workloads (and down-scaled variants).

Recipe (every draw uses ``numpy.random.default_rng(seed)`` in the order written
in each function):

* activations (raw tokens, queries, indexer queries and keys) ~ N(0,1)/sqrt(dim),
  except the KV stream of the full-size workloads, which is N(0,1);
* gate vector ~ N(0,1)/sqrt(D), positional gate biases ~ N(0, 0.02) (std 0.02);
* indexer head weights ~ U(0,1); sink logits ~ N(0,1) (0 for the tiny case);
* compressed cache entries that the step does not pool itself are synthesized
  directly in storage format: FP8 codes of N(0,1)/s clipped to +-448 with a
  per-entry power-of-two scale s drawn from {2^-8, 2^-7, 2^-6}, BF16 RoPE dims,
  FP8 indexer keys (per-tensor scale 1) or MXFP4 keys with drawn codes/scales.

Nothing here pools, rotates, scores or quantizes by the method's rules.
"""
from __future__ import annotations

import math
from types import SimpleNamespace

import numpy as np

from .configs import Geometry, WorkloadConfig, config_by_name


# ----------------------------------------------------------------- storage casts
def fp8_codes(x: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN codes (uint8) of ``x`` via PyTorch's dtype cast.

    Values are clipped to +-448 first because the cast does not saturate.
    """
    import torch
    a = np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0)
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) of ``x`` via PyTorch's dtype cast."""
    import torch
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# probability of each E2M1 magnitude code 0..7 (values 0,.5,1,1.5,2,3,4,6)
_MX_MAG_P = np.array([0.30, 0.25, 0.17, 0.11, 0.07, 0.06, 0.03, 0.01])


def mxfp4_draw(rng: np.random.Generator, shape_rows: tuple, d: int):
    """Draw MXFP4 data directly: packed E2M1 codes [*rows, d/2] and E8M0 scales [*rows, d/32].

    Element 2i sits in the low nibble of byte i, element 2i+1 in the high nibble.
    Scale bytes are 127+e with e in {-6,-5,-4} (probabilities .25/.5/.25).
    """
    assert d % 32 == 0
    mag = rng.choice(8, size=shape_rows + (d,), p=_MX_MAG_P).astype(np.uint8)
    sign = (rng.random(shape_rows + (d,)) < 0.5).astype(np.uint8)
    code = mag | (sign << 3)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    e = rng.choice(np.array([-6, -5, -4]), size=shape_rows + (d // 32,), p=[0.25, 0.5, 0.25])
    scales = (127 + e).astype(np.uint8)
    return packed, scales


def _normal(rng, shape, std=1.0, dtype=np.float32):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(dtype, copy=False)


def _fp8_entries(rng, n: int, D_n: int, chunk: int = 1 << 16):
    """Per-entry scaled FP8 nope planes: codes [n, D_n] and pow2 scales [n]."""
    codes = np.empty((n, D_n), np.uint8)
    e = rng.choice(np.array([-8, -7, -6]), size=n, p=[0.25, 0.5, 0.25])
    scale = np.ldexp(np.ones(n, np.float32), e).astype(np.float32)
    for s in range(0, n, chunk):
        t = min(n, s + chunk)
        v = _normal(rng, (t - s, D_n))
        v *= np.ldexp(np.float32(1.0), -e[s:t]).astype(np.float32)[:, None]
        codes[s:t] = fp8_codes(v)
    return codes, scale


def _bf16_normal(rng, shape, std=1.0, chunk_rows: int = 1 << 16):
    out = np.empty(shape, np.uint16)
    flat = out.reshape(shape[0], int(np.prod(shape[1:])))
    for s in range(0, shape[0], chunk_rows):
        t = min(shape[0], s + chunk_rows)
        flat[s:t] = bf16_bits(_normal(rng, (t - s, flat.shape[1]), std))
    return out


def _fp8_normal(rng, shape, std, chunk_rows: int = 1 << 16):
    out = np.empty(shape, np.uint8)
    flat = out.reshape(shape[0], int(np.prod(shape[1:])))
    for s in range(0, shape[0], chunk_rows):
        t = min(shape[0], s + chunk_rows)
        flat[s:t] = fp8_codes(_normal(rng, (t - s, flat.shape[1]), std))
    return out


def _blocks(seq: int, first_block: int, n: int, m: int, w_cap: int, row0: int):
    """Pool list for ``n`` consecutive blocks of sequence ``seq`` whose raw tokens sit in a
    ring of capacity ``w_cap`` (token u at slot u mod w_cap) and whose entries go to cache
    rows ``row0 + i``."""
    assert w_cap % m == 0
    j = first_block + np.arange(n, dtype=np.int64)
    pos = j * m
    return dict(block_row=seq * w_cap + (pos % w_cap), block_pos=pos,
                out_row=row0 + np.arange(n, dtype=np.int64))


def _cat_blocks(parts):
    if not parts:
        return dict(block_row=np.zeros(0, np.int64), block_pos=np.zeros(0, np.int64),
                    out_row=np.zeros(0, np.int64))
    return {k: np.concatenate([p[k] for p in parts]).astype(np.int64) for k in parts[0]}


# ----------------------------------------------------------------- workloads
def tiny(seed: int = 0, L: int = 2048, n_queries: int = 16, sharp: bool = False,
         g: Geometry | None = None):
    """Tiny f32 CSA+HCA decode: one raw stream pooled by both layers; queries at the
    last ``n_queries`` positions.  ``sharp`` draws queries N(0,1) (no 1/sqrt(D))."""
    from .configs import TINY_GEOMETRY
    g = g or TINY_GEOMETRY
    rng = np.random.default_rng(seed)
    x = _normal(rng, (L, g.D), 1 / math.sqrt(g.D))
    y = _normal(rng, (L, g.d_I), 1 / math.sqrt(g.d_I))
    csa_w = _normal(rng, (g.D,), 1 / math.sqrt(g.D))
    csa_b = _normal(rng, (g.m_csa,), 0.02)
    hca_w = _normal(rng, (g.D,), 1 / math.sqrt(g.D))
    hca_b = _normal(rng, (g.m_hca,), 0.02)
    q = _normal(rng, (n_queries, g.H, g.D), 1.0 if sharp else 1 / math.sqrt(g.D))
    q_I = _normal(rng, (n_queries, g.H_I, g.d_I), 1 / math.sqrt(g.d_I))
    w = rng.random((n_queries, g.H_I), dtype=np.float32)
    sink = np.zeros(g.H, np.float32)
    q_pos = np.arange(L - n_queries, L, dtype=np.int64)
    n_csa, n_hca = L // g.m_csa, L // g.m_hca
    common = dict(fmt="f32", B=1, W_cap=L, win=x.reshape(1, L, g.D), q=q, sink=sink,
                  q_pos=q_pos, seq_id=np.zeros(n_queries, np.int32),
                  cache_row_start=np.zeros(1, np.int64))
    csa = SimpleNamespace(
        mode="csa", m=g.m_csa, n_rows=n_csa, gate_w=csa_w, gate_b=csa_b,
        cache_f32=np.zeros((n_csa, g.D), np.float32), idx_fmt="f32",
        idx_f32=np.zeros((n_csa, g.d_I), np.float32), win_idx=y.reshape(1, L, g.d_I),
        q_I=q_I, w=w, pool=_blocks(0, 0, n_csa, g.m_csa, L, 0), **common)
    hca = SimpleNamespace(
        mode="hca", m=g.m_hca, n_rows=n_hca, gate_w=hca_w, gate_b=hca_b,
        cache_f32=np.zeros((n_hca, g.D), np.float32),
        pool=_blocks(0, 0, n_hca, g.m_hca, L, 0), **common)
    return SimpleNamespace(name="tiny_f32", kind="tiny", g=g, seed=seed, B=1, L=L,
                           lengths=np.array([L], np.int64), layers=[csa, hca], x=x, y=y)


def _decode_layer(rng, g: Geometry, mode: str, lengths: np.ndarray, W_cap: int,
                  kv_std: float, idx_fmt: str = "fp8"):
    """One decode layer for B sequences whose query is the last token t = L_b - 1.

    Cache rows for sequence b start at ``cache_row_start[b]``; the sequence sees
    floor(L_b/m) entries.  When L_b is a multiple of m the newest entry is pooled by
    the step itself from the window ring, so its cache row is left zero here.
    """
    B = len(lengths)
    m = g.m_csa if mode == "csa" else g.m_hca
    n_vis = (lengths // m).astype(np.int64)
    row_start = np.concatenate([[0], np.cumsum(n_vis)[:-1]]).astype(np.int64)
    N = int(n_vis.sum())
    # draw order: cache nope+scale, cache rope, [idx keys], window ring, [idx ring],
    #             gate w, gate b, q, [q_I, w], sink
    nope, scale = _fp8_entries(rng, N, g.D_n)
    rope = _bf16_normal(rng, (N, g.D_r), 1.0)
    lay = SimpleNamespace(mode=mode, m=m, fmt="quant", B=B, W_cap=W_cap, n_rows=N,
                          cache_row_start=row_start, n_visible=n_vis)
    if mode == "csa":
        if idx_fmt == "fp8":
            lay.idx_fmt = "fp8"
            lay.idx_fp8 = _fp8_normal(rng, (N, g.d_I), 1 / math.sqrt(g.d_I))
        else:
            lay.idx_fmt = "mxfp4"
            lay.idx_codes, lay.idx_scales = mxfp4_draw(rng, (N,), g.d_I)
    lay.win = _bf16_normal(rng, (B, W_cap, g.D), kv_std)
    if mode == "csa":
        lay.win_idx = _bf16_normal(rng, (B, W_cap, g.d_I), 1 / math.sqrt(g.d_I))
    lay.gate_w = _normal(rng, (g.D,), 1 / math.sqrt(g.D))
    lay.gate_b = _normal(rng, (m,), 0.02)
    lay.q = _bf16_normal(rng, (B, g.H, g.D), 1 / math.sqrt(g.D))
    if mode == "csa":
        if idx_fmt == "fp8":
            lay.q_I = _fp8_normal(rng, (B, g.H_I, g.d_I), 1 / math.sqrt(g.d_I))
        else:
            lay.q_I, lay.q_I_scales = mxfp4_draw(rng, (B, g.H_I), g.d_I)
        lay.w = rng.random((B, g.H_I), dtype=np.float32)
    lay.sink = _normal(rng, (g.H,), 1.0)
    lay.q_pos = (lengths - 1).astype(np.int64)
    lay.seq_id = np.arange(B, dtype=np.int32)
    parts = []
    for b in range(B):
        if lengths[b] % m == 0:
            j = int(lengths[b] // m) - 1
            parts.append(_blocks(b, j, 1, m, W_cap, int(row_start[b]) + j))
            r = int(row_start[b]) + j          # leave the pooled row empty
            nope[r] = 0
            rope[r] = 0
            scale[r] = 0
            if mode == "csa":
                if lay.idx_fmt == "fp8":
                    lay.idx_fp8[r] = 0
                else:
                    lay.idx_codes[r] = 0
                    lay.idx_scales[r] = 0
    lay.pool = _cat_blocks(parts)
    lay.cache_nope, lay.cache_rope, lay.cache_scale = nope, rope, scale
    return lay


def swa_layer(rng, g: Geometry, lengths: np.ndarray, W_cap: int, kv_std: float = 1.0, fmt: str = "quant"):
    """A sliding-window-only decode layer (the multi-token-prediction block): each
    sequence's query t = L_b - 1 attends to its last n_win raw tokens and the sink;
    there is no compressed cache and nothing to pool.
    Draw order: window ring, q, sink."""
    lengths = np.asarray(lengths, np.int64)
    B = len(lengths)
    lay = SimpleNamespace(mode="swa", m=1, fmt=fmt, B=B, W_cap=W_cap, n_rows=0,
                          cache_row_start=np.zeros(B, np.int64), n_visible=np.zeros(B, np.int64))
    if fmt == "f32":
        lay.win = _normal(rng, (B, W_cap, g.D), kv_std)
        lay.q = _normal(rng, (B, g.H, g.D), 1 / math.sqrt(g.D))
    else:
        lay.win = _bf16_normal(rng, (B, W_cap, g.D), kv_std)
        lay.q = _bf16_normal(rng, (B, g.H, g.D), 1 / math.sqrt(g.D))
    lay.sink = _normal(rng, (g.H,), 1.0)
    lay.q_pos = (lengths - 1).astype(np.int64)
    lay.seq_id = np.arange(B, dtype=np.int32)
    lay.pool = _cat_blocks([])
    return lay


def csa_decode(seed: int = 1, B: int = 8, L: int = 131072, g: Geometry | None = None,
               idx_fmt: str = "fp8"):
    from .configs import FULL_GEOMETRY
    g = g or FULL_GEOMETRY
    rng = np.random.default_rng(seed)
    lengths = np.full(B, L, np.int64)
    lay = _decode_layer(rng, g, "csa", lengths, g.n_win, 1.0, idx_fmt)
    return SimpleNamespace(name="csa_decode", kind="csa_decode", g=g, seed=seed, B=B,
                           lengths=lengths, layers=[lay])


def hca_decode(seed: int = 2, B: int = 4, L: int = 1048576, g: Geometry | None = None):
    from .configs import FULL_GEOMETRY
    g = g or FULL_GEOMETRY
    rng = np.random.default_rng(seed)
    lengths = np.full(B, L, np.int64)
    lay = _decode_layer(rng, g, "hca", lengths, max(g.n_win, g.m_hca), 1.0)
    return SimpleNamespace(name="hca_decode", kind="hca_decode", g=g, seed=seed, B=B,
                           lengths=lengths, layers=[lay])


def ragged_lengths(seed: int, B: int, lo: int, hi: int, round_every4: bool = False):
    """L_b = floor(exp(U(ln lo, ln hi))); optionally every 4th rounded down to a multiple
    of 128 so that HCA pooling triggers in the step."""
    rng = np.random.default_rng([seed, 0x5EED])
    L = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=B))).astype(np.int64)
    L = np.clip(L, lo, hi)
    if round_every4:
        L[::4] = np.maximum(128, (L[::4] // 128) * 128)
    return L


def ragged_pair(seed: int = 4, B: int = 32, lo: int = 4096, hi: int = 1048576,
                round_every4: bool = False, g: Geometry | None = None, idx_fmt: str = "fp8"):
    """A CSA layer then an HCA layer, each a decode step for B ragged sequences.
    The two layers get independent inputs.  ``idx_fmt`` is the CSA indexer's storage
    ("fp8", or "mxfp4" for the FP4 indexer the pages describe)."""
    from .configs import FULL_GEOMETRY
    g = g or FULL_GEOMETRY
    lengths = ragged_lengths(seed, B, lo, hi, round_every4)
    rng = np.random.default_rng(seed)
    W_cap = max(g.n_win, g.m_hca)
    csa = _decode_layer(rng, g, "csa", lengths, W_cap, 1.0, idx_fmt)
    hca = _decode_layer(rng, g, "hca", lengths, W_cap, 1.0)
    return SimpleNamespace(name="ragged_pair", kind="ragged_pair", g=g, seed=seed, B=B,
                           lengths=lengths, layers=[csa, hca])


def csa_prefill(seed: int = 3, prefix: int = 1048576, T: int = 4096, g: Geometry | None = None,
                with_hca: bool = True):
    """A T-token chunk appended to a ``prefix``-token sequence (one sequence).

    The CSA layer's cache holds prefix/4 synthesized entries plus T/4 rows that the
    chunk's pooling fills; its MXFP4 indexer keys likewise.  The window ring (capacity
    T + n_win) holds the last n_win-1 prefix tokens and the chunk.  The HCA layer gets
    its own chunk of raw tokens and prefix/128 synthesized entries plus T/128 rows to pool.
    """
    from .configs import FULL_GEOMETRY
    g = g or FULL_GEOMETRY
    assert prefix % g.m_hca == 0 and T % g.m_hca == 0
    rng = np.random.default_rng(seed)
    W_cap = T + g.n_win
    assert W_cap % g.m_hca == 0
    Np, Nc = prefix // g.m_csa, T // g.m_csa
    N = Np + Nc
    # draw order: prefix nope+scale, prefix rope, prefix idx keys, window ring (tail+chunk),
    #             chunk idx stream, gate w, gate b, q, q_I, w, sink, then the HCA layer
    nope = np.zeros((N, g.D_n), np.uint8)
    scale = np.zeros(N, np.float32)
    rope = np.zeros((N, g.D_r), np.uint16)
    nope[:Np], scale[:Np] = _fp8_entries(rng, Np, g.D_n)
    rope[:Np] = _bf16_normal(rng, (Np, g.D_r), 1.0)
    idx_codes = np.zeros((N, g.d_I // 2), np.uint8)
    idx_scales = np.zeros((N, g.d_I // 32), np.uint8)
    idx_codes[:Np], idx_scales[:Np] = mxfp4_draw(rng, (Np,), g.d_I)
    win = np.zeros((1, W_cap, g.D), np.uint16)
    tail = g.n_win - 1
    pos_tail = np.arange(prefix - tail, prefix, dtype=np.int64)
    pos_chunk = np.arange(prefix, prefix + T, dtype=np.int64)
    win[0, pos_tail % W_cap] = _bf16_normal(rng, (tail, g.D), 1.0)
    win[0, pos_chunk % W_cap] = _bf16_normal(rng, (T, g.D), 1.0)
    win_idx = np.zeros((1, W_cap, g.d_I), np.uint16)
    win_idx[0, pos_chunk % W_cap] = _bf16_normal(rng, (T, g.d_I), 1 / math.sqrt(g.d_I))
    gate_w = _normal(rng, (g.D,), 1 / math.sqrt(g.D))
    gate_b = _normal(rng, (g.m_csa,), 0.02)
    q = _bf16_normal(rng, (T, g.H, g.D), 1 / math.sqrt(g.D))
    q_I, q_I_scales = mxfp4_draw(rng, (T, g.H_I), g.d_I)
    w = rng.random((T, g.H_I), dtype=np.float32)
    sink = _normal(rng, (g.H,), 1.0)
    common = dict(B=1, W_cap=W_cap, q_pos=pos_chunk, seq_id=np.zeros(T, np.int32),
                  cache_row_start=np.zeros(1, np.int64), fmt="quant")
    csa = SimpleNamespace(
        mode="csa", m=g.m_csa, n_rows=N, n_visible=np.array([N], np.int64),
        cache_nope=nope, cache_rope=rope, cache_scale=scale, idx_fmt="mxfp4",
        idx_codes=idx_codes, idx_scales=idx_scales, win=win, win_idx=win_idx,
        gate_w=gate_w, gate_b=gate_b, q=q, q_I=q_I, q_I_scales=q_I_scales, w=w, sink=sink,
        pool=_blocks(0, Np, Nc, g.m_csa, W_cap, Np), **common)
    layers = [csa]
    if with_hca:
        Hp, Hc = prefix // g.m_hca, T // g.m_hca
        hn = np.zeros((Hp + Hc, g.D_n), np.uint8)
        hs = np.zeros(Hp + Hc, np.float32)
        hr = np.zeros((Hp + Hc, g.D_r), np.uint16)
        hn[:Hp], hs[:Hp] = _fp8_entries(rng, Hp, g.D_n)
        hr[:Hp] = _bf16_normal(rng, (Hp, g.D_r), 1.0)
        hwin = np.zeros((1, W_cap, g.D), np.uint16)
        hwin[0, pos_tail % W_cap] = _bf16_normal(rng, (tail, g.D), 1.0)
        hwin[0, pos_chunk % W_cap] = _bf16_normal(rng, (T, g.D), 1.0)
        hgw = _normal(rng, (g.D,), 1 / math.sqrt(g.D))
        hgb = _normal(rng, (g.m_hca,), 0.02)
        hsink = _normal(rng, (g.H,), 1.0)
        hca = SimpleNamespace(
            mode="hca", m=g.m_hca, n_rows=Hp + Hc, n_visible=np.array([Hp + Hc], np.int64),
            cache_nope=hn, cache_rope=hr, cache_scale=hs, win=hwin, gate_w=hgw, gate_b=hgb,
            q=q, sink=hsink, pool=_blocks(0, Hp, Hc, g.m_hca, W_cap, Hp), **common)
        layers.append(hca)
    return SimpleNamespace(name="csa_prefill", kind="csa_prefill", g=g, seed=seed, B=1,
                           prefix=prefix, T=T, lengths=np.array([prefix + T], np.int64),
                           layers=layers)


def make(cfg: WorkloadConfig | str, **overrides):
    """Build the workload of a named config (``overrides`` replace its size params)."""
    if isinstance(cfg, str):
        cfg = config_by_name(cfg)
    p = dict(cfg.params)
    p.update(overrides)
    fn = {"tiny": tiny, "csa_decode": csa_decode, "hca_decode": hca_decode,
          "csa_prefill": csa_prefill, "ragged_pair": ragged_pair}[cfg.kind]
    if cfg.kind == "tiny":
        return fn(seed=cfg.seed, g=cfg.geometry, **p)
    return fn(seed=cfg.seed, g=cfg.geometry, **p)
