"""Pins of the oracle's indexer, top-k, attention and step composition (CPU only).

Indexer: pure-Python brute force, exact rational dots, correctly rounded sums,
one-hot weights, all-negative dots, the exactness guard.  Top-k: full stable sort,
k >= V, planted ties, signed zeros, visibility.  Attention: dense masked softmax over
the explicit concatenation (scipy), standard causal MQA (torch SDPA) at m = 1 with no
window and no sink, sink limits, equal logits, head permutation.  Causality: future
tokens and incomplete blocks leave outputs bit-identical.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import attend, indexer, quant, step, topk
from synth.configs import Geometry


# ------------------------------------------------------------------ indexer
def test_score_f64_matches_python_brute_force():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 32)).astype(np.float32)
    k = rng.standard_normal((40, 32)).astype(np.float32)
    w = rng.random(4).astype(np.float32)
    got = indexer.score_f64(q, k, w)
    for j in range(40):
        acc = 0.0
        for h in range(4):
            d = 0.0
            for i in range(32):
                d = d + float(q[h, i]) * float(k[j, i])
            acc = acc + float(w[h]) * (d if d > 0 else 0.0)
        assert got[j] == acc


def _fp8_operands(seed, H, V, d=128):
    rng = np.random.default_rng(seed)
    qc = synth.fp8_codes(rng.standard_normal((H, d)) / math.sqrt(d))
    kc = synth.fp8_codes(rng.standard_normal((V, d)) / math.sqrt(d))
    return step.fp8_values(qc), step.fp8_values(kc)


def test_head_dots_exact_against_rationals():
    qv, kv = _fp8_operands(1, 4, 6)
    d = indexer.head_dots_exact(qv, kv, indexer.fp8_grain(4), indexer.fp8_grain(6))
    for h in range(4):
        for j in range(6):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qv[h], kv[j]))
            assert Fraction(float(d[h, j])) == exact


def test_head_dots_exact_mxfp4_against_rationals():
    rng = np.random.default_rng(2)
    qc, qs = synth.mxfp4_draw(rng, (3,), 128)
    kc, ks = synth.mxfp4_draw(rng, (5,), 128)
    qv, kv = quant.mxfp4_decode(qc, qs), quant.mxfp4_decode(kc, ks)
    d = indexer.head_dots_exact(qv, kv, indexer.mxfp4_grain(qs), indexer.mxfp4_grain(ks))
    for h in range(3):
        for j in range(5):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qv[h], kv[j]))
            assert Fraction(float(d[h, j])) == exact


def test_exactness_guard_fires():
    q = np.full((1, 128), 448.0)
    k = np.full((1, 128), 448.0)
    with pytest.raises(AssertionError):
        indexer.head_dots_exact(q, k, indexer.fp8_grain(1), indexer.fp8_grain(1))


def test_canonical_sum_close_to_exact_sum():
    qv, kv = _fp8_operands(3, 64, 300)
    d = indexer.head_dots_exact(qv, kv, indexer.fp8_grain(64), indexer.fp8_grain(300))
    w = np.random.default_rng(4).random(64).astype(np.float32)
    got = indexer.score_canonical_f32(d, w)
    for j in range(300):
        terms = [float(np.float32(w[h]) * np.float32(max(d[h, j], 0.0))) for h in range(64)]
        exact = math.fsum(terms)
        assert abs(float(got[j]) - exact) <= 64 * 2 ** -24 * max(abs(exact), 1e-30)
    # permuting heads (with their weights) only reorders the rounding
    perm = np.random.default_rng(5).permutation(64)
    got_p = indexer.score_canonical_f32(d[perm], w[perm])
    np.testing.assert_allclose(got_p, got, rtol=64 * 2 ** -24)


def test_canonical_sum_one_hot_and_negative():
    qv, kv = _fp8_operands(6, 64, 50)
    d = indexer.head_dots_exact(qv, kv, indexer.fp8_grain(64), indexer.fp8_grain(50))
    for h in (0, 17, 63):
        w = np.zeros(64, np.float32)
        w[h] = 1.0
        got = indexer.score_canonical_f32(d, w)
        assert np.array_equal(got, np.maximum(d[h], 0).astype(np.float32))
    got = indexer.score_canonical_f32(-np.abs(d) - 1e-3, np.ones(64, np.float32))
    assert np.all(got == 0) and not np.any(np.signbit(got))


def _round_f32(x: Fraction) -> Fraction:
    """The binary32 value nearest to x (ties to even), by exact rational arithmetic."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1                                   # now 2^e <= x < 2^(e+1)
    e = max(e, -126)                             # subnormals share the smallest step
    step = Fraction(2) ** (e - 23)
    q = x / step
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * step


def test_fma_f32_against_exact_rounding():
    rng = np.random.default_rng(9)
    a = rng.random(400).astype(np.float32) * np.float32(2.0) ** rng.integers(-30, 5, 400).astype(np.float32)
    b = (rng.standard_normal(400) * 2.0 ** rng.integers(-30, 5, 400)).astype(np.float32)
    c = (rng.standard_normal(400) * 2.0 ** rng.integers(-30, 5, 400)).astype(np.float32)
    # a double-rounding trap: c + a*b = 1 + 2^-23 + 2^-24 - 2^-60 rounds to 1 + 2^-24
    # in binary64, exactly halfway; the single rounding must go down to 1 + 2^-23
    a[0], b[0], c[0] = np.float32(1 + 2.0 ** -18), np.float32(2.0 ** -24 * (1 - 2.0 ** -18)), np.float32(1 + 2.0 ** -23)
    got = indexer.fma_f32(a, b, c)
    assert float(got[0]) == 1 + 2.0 ** -23
    assert float(np.float32(np.float64(a[0]) * np.float64(b[0]) + np.float64(c[0]))) != 1 + 2.0 ** -23
    for i in range(400):
        want = _round_f32(Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i])))
        assert Fraction(float(got[i])) == want, i


def test_canonical_sum_order_by_hand():
    # heads enter S_0 / S_1 in the 32x32 output-layout order, one rounding per head
    rng = np.random.default_rng(10)
    d = (rng.standard_normal((64, 7)) * 4).astype(np.float32)
    w = rng.random(64).astype(np.float32)
    got = indexer.score_canonical_f32(d.astype(np.float64), w)
    for j in range(7):
        S = [Fraction(0), Fraction(0)]
        for u in range(2):
            for T in range(2):
                for i in range(16):
                    h = 32 * T + 8 * (i // 4) + 4 * u + i % 4
                    r = max(Fraction(float(d[h, j])), Fraction(0))
                    S[u] = _round_f32(Fraction(float(w[h])) * r + S[u])
        assert Fraction(float(got[j])) == _round_f32(S[0] + S[1])


# ------------------------------------------------------------------- top-k
def test_topk_against_stable_sort():
    rng = np.random.default_rng(7)
    for V, k in [(100, 16), (1000, 512), (5, 16), (512, 512), (0, 4)]:
        s = rng.integers(0, 40, V).astype(np.float32)     # many planted ties
        got = topk.select(s, k)
        order = sorted(range(V), key=lambda j: (-float(s[j]), j))[:min(k, V)]
        want = sorted(order) + [-1] * (k - min(k, V))
        assert list(got) == want


def test_topk_signed_zero_ties_and_lower_index():
    s = np.array([0.0, -0.0, 0.0, 1.0, -0.0], np.float32)
    assert list(topk.select(s, 3)) == [0, 1, 3]
    s = np.array([2.0, 5.0, 5.0, 5.0, 1.0], np.float32)
    assert list(topk.select(s, 2)) == [1, 2]


def test_visibility_rule():
    assert [topk.n_visible(t, 4) for t in range(9)] == [0, 0, 0, 1, 1, 1, 1, 2, 2]
    assert topk.n_visible(127, 128) == 1 and topk.n_visible(126, 128) == 0
    assert topk.n_visible(131071, 4) == 32768


# --------------------------------------------------------------- attention
def _tiny(**kw):
    g = Geometry(H=4, D=32, D_r=8, H_I=4, d_I=16, topk=kw.pop("topk", 8),
                 n_win=kw.pop("n_win", 16), m_csa=kw.pop("m_csa", 4), m_hca=kw.pop("m_hca", 32),
                 tau=kw.pop("tau", 1.0))
    return synth.tiny(seed=kw.pop("seed", 11), L=kw.pop("L", 256), n_queries=kw.pop("nq", 8),
                      g=g, **kw)


def _rot(x, pos, D_r, base=1e4):
    """Independent complex-exponential RoPE for the brute force."""
    h = D_r // 2
    z = (x[..., -D_r:-h] + 1j * x[..., -h:]) * np.exp(
        1j * np.asarray(pos, np.float64)[..., None] * base ** (-np.arange(h) * 2 / D_r))
    return np.concatenate([x[..., :-D_r], z.real, z.imag], axis=-1)


@pytest.mark.parametrize("layer,tau", [(0, 1.0), (1, 1.0), (0, 0.37), (1, 2.5)])
def test_attention_equals_dense_softmax_when_everything_visible(layer, tau):
    w = _tiny(topk=4096, n_win=4096, L=256, tau=tau)
    lay = w.layers[layer]
    lay.sink = np.linspace(-1, 1, w.g.H).astype(np.float32)
    res = step.run_layer(lay, w.g)
    ent = res["pooled"]["kv"]["f32"].astype(np.float64)
    for n, t in enumerate(lay.q_pos):
        V = (t + 1) // lay.m
        toks = _rot(w.x[: t + 1].astype(np.float64), np.arange(t + 1), w.g.D_r)
        K = np.concatenate([ent[:V], toks])
        qh = _rot(lay.q[n].astype(np.float64), np.full(w.g.H, t), w.g.D_r)
        logits = np.concatenate([tau * (qh @ K.T), lay.sink[:, None].astype(np.float64)], axis=1)
        p = scipy.special.softmax(logits, axis=1)
        np.testing.assert_allclose(res["o"][n], p[:, :-1] @ K, rtol=1e-11, atol=1e-14)
        if layer == 0:
            assert list(res["idx"][n][:V]) == list(range(V))


def test_textbook_causal_mqa_at_m1_no_window_no_sink():
    w = _tiny(m_csa=1, topk=4096, n_win=0, L=64, nq=6)
    lay = w.layers[0]
    lay.sink = np.full(w.g.H, -np.inf)
    res = step.run_layer(lay, w.g)
    toks = _rot(w.x.astype(np.float64), np.arange(64), w.g.D_r)
    for n, t in enumerate(lay.q_pos):
        qh = _rot(lay.q[n].astype(np.float64), np.full(w.g.H, t), w.g.D_r)
        Q = torch.from_numpy(qh)[None]                       # [1, H, D]
        K = torch.from_numpy(toks[: t + 1])[None, None].expand(1, w.g.H, t + 1, w.g.D)
        o = torch.nn.functional.scaled_dot_product_attention(
            Q[:, :, None, :], K.contiguous(), K.contiguous(), scale=1.0)[0, :, 0].numpy()
        np.testing.assert_allclose(res["o"][n], o, rtol=2e-6, atol=1e-8)


def test_sink_limits_and_equal_logits():
    w = _tiny()
    lay = w.layers[1]
    lay.sink = np.full(w.g.H, 1e4, np.float32)
    res = step.run_layer(lay, w.g)
    assert np.all(res["o"] == 0) and np.allclose(res["lse"], 1e4)
    # zero queries: equal logits -> mean of the attention set
    lay.sink = np.full(w.g.H, -np.inf)
    lay.q = np.zeros_like(lay.q)
    res = step.run_layer(lay, w.g)
    ent = res["pooled"]["kv"]["f32"].astype(np.float64)
    for n, t in enumerate(lay.q_pos):
        V = (t + 1) // lay.m
        win = _rot(w.x[t - 15: t + 1].astype(np.float64), np.arange(t - 15, t + 1), w.g.D_r)
        K = np.concatenate([ent[:V], win])
        np.testing.assert_allclose(res["o"][n], np.tile(K.mean(0), (w.g.H, 1)), rtol=1e-12)


def test_head_permutation():
    w = _tiny(sharp=True)
    lay = w.layers[0]
    lay.sink = np.linspace(-2, 2, w.g.H).astype(np.float32)
    r1 = step.run_layer(lay, w.g)
    perm = np.array([2, 0, 3, 1])
    lay.q = lay.q[:, perm].copy()
    lay.sink = lay.sink[perm].copy()
    r2 = step.run_layer(lay, w.g)
    np.testing.assert_allclose(r2["o"], r1["o"][:, perm], rtol=1e-13)
    assert np.array_equal(r2["idx"], r1["idx"])
    # permuting indexer heads with their weights keeps the selection
    lay.q_I = lay.q_I[:, perm].copy()
    lay.w = lay.w[:, perm].copy()
    r3 = step.run_layer(lay, w.g)
    assert np.array_equal(r3["idx"], r1["idx"])


def test_causality_future_and_incomplete_block():
    w = synth.tiny(seed=0)
    r1 = [step.run_layer(lay, w.g) for lay in w.layers]
    t_idx = 1                           # query at t = 2033: block 508 (2032..2035) incomplete
    assert w.layers[0].q_pos[t_idx] == 2033
    rng = np.random.default_rng(99)
    w.x[2034:] += rng.standard_normal(w.x[2034:].shape).astype(np.float32)
    w.y[2034:] += rng.standard_normal(w.y[2034:].shape).astype(np.float32)
    r2 = [step.run_layer(lay, w.g) for lay in w.layers]
    for a, b in zip(r1, r2):
        assert np.array_equal(a["o"][t_idx], b["o"][t_idx])
        assert np.array_equal(a["o"][0], b["o"][0])
        assert not np.array_equal(a["o"][-1], b["o"][-1])
    assert np.array_equal(r1[0]["idx"][: t_idx + 1], r2[0]["idx"][: t_idx + 1])


def test_window_contents():
    assert list(attend.window_positions(5, 3)) == [3, 4, 5]
    assert list(attend.window_positions(1, 128)) == [0, 1]
    assert list(attend.window_positions(7, 0)) == []
