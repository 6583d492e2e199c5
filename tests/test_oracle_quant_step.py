"""Pins of the oracle's quantized step readers (oracle/step.py).

A quantized layer stores each compressed entry as FP8 E4M3 codes times a per-entry
power-of-two scale for the non-RoPE dims and BF16 for the (already rotated) RoPE
dims, and its indexer keys and queries as FP8 (per-tensor scale 1) or MXFP4 ("DeepSeek
V4: How They Crushed the Million-Token Memory Problem" (sameershanbhag.com), "Two
kinds of memory instead of one": FP8 for most KV entries, BF16 for the RoPE dims, FP4
for the indexer).  The step reads these planes through ``_Cache.entries``,
``_Cache.idx_keys``, ``index_query_values`` and the quantized branch of
``scores_for_query``, with the rows pooled in the step laid over the cache.

Pinned here, independently of the oracle's own decoders:
* by hand: two- and three-row layers whose decoded values are written out as
  numbers (scale multiplied, not divided; nope dims first, RoPE dims last; MXFP4
  element 2i in the low nibble; E8M0 scale per 32 elements; the grain of each row;
  the pooled row replacing the cached one), and an indexer score worked by hand;
* differentially: a quantized layer and an f32 twin holding the same values
  (decoded here with PyTorch's FP8 cast, BF16 bit shifts and an E2M1 table) give
  the same top-k, the same selected scores and the same output.  The f32 path is
  pinned by brute force elsewhere; indexer operands are drawn so that every score
  is exact, hence the canonical binary32 head sum and the f32 path's fp64 sum agree;
* against the mathematics: with k >= V and the window covering the whole
  sequence, a quantized layer's output equals a dense softmax over the explicit
  concatenation of its decoded entries and rotated tokens, plus the sink column.
"""
from dataclasses import replace
from types import SimpleNamespace

import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import step
from synth.gen import _blocks, _cat_blocks, bf16_bits

# ------------------------------------------------------------ independent decoders
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def fp8_val(codes):
    c = torch.from_numpy(np.ascontiguousarray(np.asarray(codes, np.uint8)))
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def bf16_val(bits):
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def mx_val(packed, scales):
    p = np.asarray(packed, np.uint8)
    nib = np.stack([p & 15, p >> 4], axis=-1).reshape(p.shape[:-1] + (2 * p.shape[-1],))
    v = np.where(nib & 8, -1.0, 1.0) * _E2M1[nib & 7]
    s = np.exp2(np.asarray(scales, np.float64) - 127.0)
    return v * np.repeat(s, 32, axis=-1)


def fp8_code(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ------------------------------------------------------------------ by hand
def _hand_layer(idx_fmt):
    """Three cache rows (D = 8: 6 nope + 2 RoPE dims; d_I = 32)."""
    lay = SimpleNamespace(mode="csa", m=4, fmt="quant", idx_fmt=idx_fmt)
    # E4M3 codes: 0x38 = 1.0, 0xC4 = -3.0, 0x01 = 2^-9 (smallest subnormal), 0x40 = 2.0
    lay.cache_nope = np.array([[0x38] * 6, [0xC4] * 6, [0x01] * 6], np.uint8)
    lay.cache_scale = np.array([2.0 ** -7, 2.0 ** -6, 2.0 ** -8], np.float32)
    # BF16 bits: 0x3F80 = 1.0, 0xC040 = -3.0, 0x3E00 = 0.125, 0x4000 = 2.0
    lay.cache_rope = np.array([[0x3F80, 0xC040], [0x3E00, 0x3F80], [0x4000, 0x3E00]], np.uint16)
    if idx_fmt == "fp8":
        lay.idx_fp8 = np.zeros((3, 32), np.uint8)
        lay.idx_fp8[0, :] = 0x38                       # 1.0
        lay.idx_fp8[1, :16] = 0x30                     # 0.5
        lay.idx_fp8[1, 16:] = 0xB8                     # -1.0
        lay.idx_fp8[2, 0] = 0x01                       # 2^-9
    else:
        # byte 0x21: element 2i = code 1 (0.5), element 2i + 1 = code 2 (1.0);
        # byte 0x9A: element 2i = code 0xA (-1.0), element 2i + 1 = code 9 (-0.5)
        lay.idx_codes = np.array([[0x21] * 16, [0x9A] * 16, [0x00] * 16], np.uint8)
        lay.idx_scales = np.array([[128], [125], [130]], np.uint8)     # 2, 2^-2, 2^3
    return lay


def test_entries_by_hand_scale_multiplies_and_planes_in_order():
    lay = _hand_layer("fp8")
    pooled = dict(out_row=np.array([], np.int64), kv=dict())
    c = step._Cache(lay, None, pooled)
    got = c.entries([2, 0, 1])
    want = np.array([
        [2.0 ** -17] * 6 + [2.0, 0.125],
        [2.0 ** -7] * 6 + [1.0, -3.0],
        [-3.0 / 64] * 6 + [0.125, 1.0],
    ])
    assert np.array_equal(got, want)


def test_entries_pooled_row_replaces_cached_row():
    lay = _hand_layer("fp8")
    pooled = dict(out_row=np.array([1]),
                  kv=dict(nope=np.array([[0x40] * 6], np.uint8), scale=np.array([0.25], np.float32),
                          rope=np.array([[0x4000, 0xC040]], np.uint16)))
    c = step._Cache(lay, None, pooled)
    got = c.entries([0, 1, 2])
    assert np.array_equal(got[1], [0.5] * 6 + [2.0, -3.0])
    assert np.array_equal(got[0], [2.0 ** -7] * 6 + [1.0, -3.0])
    assert np.array_equal(got[2], [2.0 ** -17] * 6 + [2.0, 0.125])


def test_idx_keys_fp8_by_hand():
    lay = _hand_layer("fp8")
    pooled = dict(out_row=np.array([2]), kv=dict(), idx=dict(fp8=np.full((1, 32), 0x40, np.uint8)))
    v, gr = step._Cache(lay, None, pooled).idx_keys([0, 1, 2])
    assert np.array_equal(v[0], np.ones(32))
    assert np.array_equal(v[1], [0.5] * 16 + [-1.0] * 16)
    assert np.array_equal(v[2], np.full(32, 2.0))           # the pooled row
    assert np.array_equal(gr, np.full(3, 2.0 ** -9))


def test_idx_keys_mxfp4_by_hand_nibble_order_scale_and_grain():
    lay = _hand_layer("mxfp4")
    pooled = dict(out_row=np.array([], np.int64), kv=dict())
    v, gr = step._Cache(lay, None, pooled).idx_keys([0, 1, 2])
    assert np.array_equal(v[0], np.tile([1.0, 2.0], 16))            # (0.5, 1.0) x 2
    assert np.array_equal(v[1], np.tile([-0.25, -0.125], 16))       # (-1.0, -0.5) x 2^-2
    assert np.array_equal(v[2], np.zeros(32))
    # grain: half the E2M1 step ... the row's scale times 0.5
    assert np.array_equal(gr, [1.0, 2.0 ** -3, 4.0])
    # the pooled row replaces the cached one, grain included
    pooled = dict(out_row=np.array([0]), kv=dict(),
                  idx=dict(codes=np.full((1, 16), 0x77, np.uint8), scales=np.array([[120]], np.uint8)))
    v, gr = step._Cache(lay, None, pooled).idx_keys([0, 1])
    assert np.array_equal(v[0], np.full(32, 6.0 * 2.0 ** -7))
    assert np.array_equal(gr, [2.0 ** -8, 2.0 ** -3])


def test_index_query_values_by_hand():
    lay = SimpleNamespace(idx_fmt="fp8", q_I=np.array([[[0x38] * 32, [0xB0] * 32]], np.uint8))
    v, gr = step.index_query_values(lay, 0)
    assert np.array_equal(v, [[1.0] * 32, [-0.5] * 32]) and np.array_equal(gr, [2.0 ** -9] * 2)
    lay = SimpleNamespace(idx_fmt="mxfp4", q_I=np.array([[[0x21] * 16, [0x9A] * 16]], np.uint8),
                          q_I_scales=np.array([[[127], [129]]], np.uint8))
    v, gr = step.index_query_values(lay, 0)
    assert np.array_equal(v[0], np.tile([0.5, 1.0], 16))
    assert np.array_equal(v[1], np.tile([-4.0, -2.0], 16))
    assert np.array_equal(gr, [0.5, 2.0])


@pytest.mark.parametrize("idx_fmt", ["fp8", "mxfp4"])
def test_score_worked_by_hand(idx_fmt):
    """32 indexer heads, d_I = 32: head h's query is 1 at dim h (0 elsewhere), so
    d[h, j] = k_j[h] and I_j = sum_h w_h max(k_j[h], 0).  Keys: k_0 = all 0.5 ->
    I = 0.5 * sum w; k_1 = all -1 -> I = 0; k_2 = 2 at even dims, -2 at odd dims
    -> I = 2 * sum of w over even heads.  With w_h = 1/32: 0.5, 0 and 1.0."""
    H_I, d_I = 32, 32
    g = SimpleNamespace(H_I=H_I, d_I=d_I)
    k_vals = np.array([[0.5] * 32, [-1.0] * 32, [2.0, -2.0] * 16])
    q_vals = np.eye(32)
    lay = SimpleNamespace(mode="csa", m=4, fmt="quant", idx_fmt=idx_fmt, cache_row_start=np.array([0]),
                          w=np.full((1, H_I), 1 / 32, np.float32))
    if idx_fmt == "fp8":
        lay.idx_fp8 = fp8_code(k_vals)
        lay.q_I = fp8_code(q_vals)[None]
    else:
        # E2M1 codes: 0.5 -> 1, 1.0 -> 2, scale byte 127 (1.0)
        def pack(vals, scale):
            mag = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
            c = np.array([[mag[abs(x) / scale] | (8 if x < 0 else 0) for x in row] for row in vals], np.uint8)
            return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
        lay.idx_codes = pack(k_vals, 1.0)
        lay.idx_scales = np.full((3, 1), 127, np.uint8)
        lay.q_I = pack(q_vals, 1.0)[None]
        lay.q_I_scales = np.full((1, 32, 1), 127, np.uint8)
    cache = step._Cache(lay, g, dict(out_row=np.array([], np.int64), kv=dict()))
    I = step.scores_for_query(cache, lay, g, 0, t=11, b=0)      # V = 3
    assert I.dtype == np.float32
    assert np.array_equal(I, np.array([0.5, 0.0, 1.0], np.float32))


# ---------------------------------------------------- differential: f32 twin
_R = np.array([0.0, 0.125, -0.125, 0.25, -0.25, 0.375, -0.375, 0.5, -0.5])


def _quant_layer(rng, g, mode, lengths, W_cap, idx_fmt="fp8"):
    """A quantized decode layer (one query per sequence at t = L - 1).  Indexer keys,
    queries and weights come from sets whose every score is an exact binary32 number
    (dyadic values with few bits), so any summation order gives the same score.  A
    sequence with L % m == 0 pools its last block in the step; that block's tokens are
    all equal (and the index-stream values from the same exact set, with a 0.5 in
    every 32-element block, which fixes the MXFP4 block scale at 2^-3), so the pooled
    index key is exact too.  FP8 operands stay below 0.5 in magnitude, so every dot
    is exact by the oracle's own bound (sum |q_i k_i| < 64)."""
    B = len(lengths)
    m = g.m_csa if mode == "csa" else g.m_hca
    n_vis = lengths // m
    row0 = np.concatenate([[0], np.cumsum(n_vis)[:-1]]).astype(np.int64)
    N = int(n_vis.sum())
    lay = SimpleNamespace(mode=mode, m=m, fmt="quant", B=B, W_cap=W_cap, n_rows=N,
                          cache_row_start=row0, n_visible=n_vis)
    codes = rng.integers(0, 256, (N, g.D_n)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38                       # no NaN codes
    lay.cache_nope = codes
    lay.cache_scale = np.exp2(rng.integers(-8, -5, N)).astype(np.float32)
    lay.cache_rope = bf16_bits(rng.standard_normal((N, g.D_r)))
    lay.win = bf16_bits(rng.standard_normal((B, W_cap, g.D)))
    lay.q = bf16_bits(rng.standard_normal((B, g.H, g.D)) / np.sqrt(g.D))
    lay.sink = rng.standard_normal(g.H).astype(np.float32)
    lay.gate_w = (rng.standard_normal(g.D) / np.sqrt(g.D)).astype(np.float32)
    lay.gate_b = (rng.standard_normal(m) * 0.02).astype(np.float32)
    lay.q_pos = (lengths - 1).astype(np.int64)
    lay.seq_id = np.arange(B, dtype=np.int32)
    if mode == "csa":
        lay.idx_fmt = idx_fmt
        if idx_fmt == "fp8":
            lay.idx_fp8 = fp8_code(rng.choice(_R, (N, g.d_I)))
            lay.q_I = fp8_code(rng.choice(_R, (B, g.H_I, g.d_I)))
        else:
            def draw(shape):
                c = rng.integers(0, 16, shape + (g.d_I,)).astype(np.uint8)
                return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
            lay.idx_codes = draw((N,))
            lay.idx_scales = (127 - rng.integers(0, 2, (N, g.d_I // 32))).astype(np.uint8)
            lay.q_I = draw((B, g.H_I))
            lay.q_I_scales = (127 - rng.integers(0, 2, (B, g.H_I, g.d_I // 32))).astype(np.uint8)
        lay.w = (rng.integers(0, 5, (B, g.H_I)) / 4).astype(np.float32)
        y = rng.choice(_R, (B, W_cap, g.d_I))
        lay.win_idx = bf16_bits(y)
    parts = []
    for b in range(B):
        if lengths[b] % m == 0:
            j = int(lengths[b] // m) - 1
            parts.append(_blocks(b, j, 1, m, W_cap, int(row0[b]) + j))
            slots = (j * m + np.arange(m)) % W_cap
            lay.win[b, slots] = lay.win[b, slots[0]]                 # equal tokens in the block
            if mode == "csa":
                yb = rng.choice(_R, g.d_I)
                yb[::32] = 0.5
                lay.win_idx[b, slots] = bf16_bits(yb)
    lay.pool = _cat_blocks(parts)
    return lay


def _f32_twin(lay, g, pooled):
    """The same layer as f32 planes, values decoded here; the rows the step pools are
    written into the twin's cache already, and the twin pools nothing."""
    t = SimpleNamespace(**vars(lay))
    t.fmt = "f32"
    ent = np.concatenate([fp8_val(lay.cache_nope) * lay.cache_scale[:, None].astype(np.float64),
                          bf16_val(lay.cache_rope)], axis=1)
    kv = pooled["kv"]
    for i, r in enumerate(pooled["out_row"]):
        ent[r] = np.concatenate([fp8_val(kv["nope"][i]) * float(kv["scale"][i]), bf16_val(kv["rope"][i])])
    t.cache_f32 = ent.astype(np.float32)
    assert np.array_equal(t.cache_f32.astype(np.float64), ent)
    t.win = bf16_val(lay.win).astype(np.float32)
    t.q = bf16_val(lay.q).astype(np.float32)
    if lay.mode == "csa":
        t.idx_fmt = "f32"
        if lay.idx_fmt == "fp8":
            keys, q_I = fp8_val(lay.idx_fp8), fp8_val(lay.q_I)
        else:
            keys, q_I = mx_val(lay.idx_codes, lay.idx_scales), mx_val(lay.q_I, lay.q_I_scales)
        ix = pooled["idx"]
        for i, r in enumerate(pooled["out_row"]):
            keys[r] = fp8_val(ix["fp8"][i]) if lay.idx_fmt == "fp8" else mx_val(ix["codes"][i], ix["scales"][i])
        t.idx_f32 = keys.astype(np.float32)
        t.q_I = q_I.astype(np.float32)
        t.win_idx = bf16_val(lay.win_idx).astype(np.float32)
    t.pool = _cat_blocks([])
    return t


def _geom(**kw):
    return replace(synth.FULL_GEOMETRY, H=4, D=64, D_r=16, H_I=kw.pop("H_I", 64), d_I=64,
                   topk=kw.pop("topk", 8), n_win=kw.pop("n_win", 16), m_hca=kw.pop("m_hca", 32), **kw)


@pytest.mark.parametrize("mode,idx_fmt,H_I", [("csa", "fp8", 64), ("csa", "mxfp4", 64), ("csa", "fp8", 32),
                                             ("hca", None, 64)])
def test_quantized_layer_equals_f32_twin(mode, idx_fmt, H_I):
    g = _geom(H_I=H_I)
    lengths = np.array([96, 130, 257, 64, 200], np.int64)    # 96, 64 (CSA, HCA) and 200 (CSA) pool
    lay = _quant_layer(np.random.default_rng(7), g, mode, lengths, 32, idx_fmt)
    assert len(lay.pool["out_row"]) >= 2
    rq = step.run_layer(lay, g)
    twin = _f32_twin(lay, g, rq["pooled"])
    rf = step.run_layer(twin, g)
    if mode == "csa":
        assert np.array_equal(rq["idx"], rf["idx"])
        # the canonical binary32 sum reached the exact score of every selected entry
        assert np.array_equal(rq["sel_scores"].astype(np.float64), rf["sel_scores"])
        # every visible entry's score, the pooled rows' included, is the same number
        cq = step._Cache(lay, g, rq["pooled"])
        cf = step._Cache(twin, g, rf["pooled"])
        for n, (t, b) in enumerate(zip(lay.q_pos, lay.seq_id)):
            Iq = step.scores_for_query(cq, lay, g, n, int(t), int(b))
            If = step.scores_for_query(cf, twin, g, n, int(t), int(b))
            assert Iq.dtype == np.float32 and np.array_equal(Iq.astype(np.float64), If)
    np.testing.assert_allclose(rq["o"], rf["o"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(rq["lse"], rf["lse"], rtol=1e-13, atol=1e-13)


def _rot(x, pos, D_r, base=1e4):
    """Complex-exponential RoPE (half-split pairs), written independently."""
    h = D_r // 2
    z = (x[..., -D_r:-h] + 1j * x[..., -h:]) * np.exp(
        1j * np.asarray(pos, np.float64)[..., None] * base ** (-np.arange(h) * 2 / D_r))
    return np.concatenate([x[..., :-D_r], z.real, z.imag], axis=-1)


@pytest.mark.parametrize("mode", ["csa", "hca"])
def test_quantized_layer_dense_equivalence(mode):
    """k >= V and a window of the whole sequence: one softmax over every visible
    decoded entry (the pooled one included) and every token 0..t rotated at its own
    position, plus the sink."""
    L = 64
    g = _geom(topk=4096, n_win=4096, m_hca=16)
    lengths = np.array([L, L - 3], np.int64)
    lay = _quant_layer(np.random.default_rng(8), g, mode, lengths, L, "fp8")
    res = step.run_layer(lay, g)
    kv = res["pooled"]["kv"]
    for b, Lb in enumerate(lengths):
        t = int(Lb - 1)
        V = (t + 1) // lay.m
        rows = lay.cache_row_start[b] + np.arange(V)
        ent = np.concatenate([fp8_val(lay.cache_nope[rows]) * lay.cache_scale[rows, None].astype(np.float64),
                              bf16_val(lay.cache_rope[rows])], axis=1)
        for i, r in enumerate(res["pooled"]["out_row"]):
            if r in rows:
                ent[r - rows[0]] = np.concatenate([fp8_val(kv["nope"][i]) * float(kv["scale"][i]),
                                                   bf16_val(kv["rope"][i])])
        toks = _rot(bf16_val(lay.win[b, :t + 1]), np.arange(t + 1), g.D_r)
        K = np.concatenate([ent, toks])
        qh = _rot(bf16_val(lay.q[b]), np.full(g.H, t), g.D_r)
        logits = np.concatenate([g.tau * (qh @ K.T), lay.sink[:, None].astype(np.float64)], axis=1)
        p = scipy.special.softmax(logits, axis=1)
        np.testing.assert_allclose(res["o"][b], p[:, :-1] @ K, rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(res["lse"][b], scipy.special.logsumexp(logits, axis=1), rtol=1e-12)
        if mode == "csa":
            assert list(res["idx"][b][:V]) == list(range(V))
