"""Pins of the oracle's RoPE and softmax-gated pooling (CPU only).

RoPE: hand-worked example (tests/golden), R(0) = I, norm preservation, the complex
exponential form, and the relative-position property.  Pooling: weights sum to 1,
scipy's softmax, closed forms (block mean, one dominant bias), m = 1 identity,
permutation invariance, and the FP8 entry encoding bounds.
"""
import os

import numpy as np
import scipy.special

from oracle import pool, quant, rope

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_rope_worked_example():
    for line in open(os.path.join(GOLD, "rope_worked_example.txt")):
        if line.startswith("#") or not line.strip():
            continue
        head, xs, ys = line.split("|")
        D_r, base, pos = head.split()
        x = np.array([float(v) for v in xs.split()])
        y = np.array([float(v) for v in ys.split()])
        got = rope.rotate(x, int(pos), float(base))
        assert int(D_r) == x.size
        np.testing.assert_allclose(got, y, rtol=0, atol=1e-15)


def test_rope_identity_norm_and_complex_form():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 64))
    assert np.array_equal(rope.rotate(x, 0, 1e4), x)
    pos = rng.integers(0, 2 ** 20, 50)
    y = rope.rotate(x, pos[:, None].squeeze(-1), 1e4)
    h = 32
    np.testing.assert_allclose(x[:, :h] ** 2 + x[:, h:] ** 2, y[:, :h] ** 2 + y[:, h:] ** 2,
                               rtol=1e-12)
    z = (x[:, :h] + 1j * x[:, h:]) * np.exp(1j * pos[:, None] * 1e4 ** (-np.arange(h) * 2 / 64))
    np.testing.assert_allclose(y[:, :h], z.real, atol=1e-12)
    np.testing.assert_allclose(y[:, h:], z.imag, atol=1e-12)


def test_rope_relative_property():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    t, p = 1000, 37
    ref = rope.rotate(q, t, 1e4) @ rope.rotate(k, p, 1e4)
    for shift in (1, 999, 123456):
        got = rope.rotate(q, t + shift, 1e4) @ rope.rotate(k, p + shift, 1e4)
        np.testing.assert_allclose(got, ref, rtol=1e-9)
    # and it does depend on t - p
    other = rope.rotate(q, t + 1, 1e4) @ rope.rotate(k, p, 1e4)
    assert abs(other - ref) > 1e-6


def test_rope_apply_leaves_nope_dims():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(128)
    y = rope.apply(x, 77, 32, 1e4)
    assert np.array_equal(y[:96], x[:96])
    assert not np.allclose(y[96:], x[96:])


def test_pool_weights_sum_to_one_and_match_scipy():
    rng = np.random.default_rng(3)
    for m in (1, 4, 128):
        x = rng.standard_normal((m, 64))
        g = rng.standard_normal(64) / 8
        b = rng.standard_normal(m) * 0.02
        z = pool.gate_logits(x, g, b)
        np.testing.assert_allclose(z, [x[i] @ g + b[i] for i in range(m)], rtol=1e-13)
        a = pool.pool_weights(z)
        assert abs(a.sum() - 1.0) < 1e-15
        np.testing.assert_allclose(a, scipy.special.softmax(z), rtol=1e-13)


def test_pool_closed_forms():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4, 16))
    # zero gate, equal biases -> block mean
    _, c, _ = pool.pool_block(x, np.zeros(16), np.full(4, 0.3))
    np.testing.assert_allclose(c, x.mean(axis=0), rtol=1e-14)
    # one dominant positional bias selects that token
    for i in range(4):
        b = np.zeros(4)
        b[i] = 800.0
        _, c, y = pool.pool_block(x, np.zeros(16), b, y_blk=x[:, :3])
        np.testing.assert_allclose(c, x[i], rtol=1e-14)
        np.testing.assert_allclose(y, x[i, :3], rtol=1e-14)


def test_pool_m1_is_identity_with_rope_at_own_position():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 32))
    for p in (0, 5, 1 << 20):
        e, _ = pool.compress_block(x, rng.standard_normal(32), rng.standard_normal(1), p, 8, 1e4)
        np.testing.assert_allclose(e[:24], x[0, :24], rtol=1e-15)
        np.testing.assert_allclose(e[24:], rope.rotate(x[0, 24:], p, 1e4), rtol=1e-14)


def test_pool_rope_at_block_end_and_alpha_shared_with_index_stream():
    rng = np.random.default_rng(6)
    m, p0 = 4, 4 * 1000
    x, y = rng.standard_normal((m, 64)), rng.standard_normal((m, 16))
    g, b = rng.standard_normal(64) / 8, rng.standard_normal(m)
    e, yh = pool.compress_block(x, g, b, p0, 16, 1e4, y_blk=y)
    z = x @ g + b
    a = np.exp(z - z.max()) / np.exp(z - z.max()).sum()
    c = a @ x
    h = 8
    zc = (c[48:56] + 1j * c[56:]) * np.exp(1j * (p0 + m - 1) * 1e4 ** (-np.arange(h) * 2 / 16))
    np.testing.assert_allclose(e[:48], c[:48], rtol=1e-13)
    np.testing.assert_allclose(e[48:56], zc.real, atol=1e-13)
    np.testing.assert_allclose(e[56:], zc.imag, atol=1e-13)
    np.testing.assert_allclose(yh, a @ y, rtol=1e-13)


def test_pool_permutation_invariance():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((128, 32))
    g, b = rng.standard_normal(32) / 6, rng.standard_normal(128) * 0.02
    perm = rng.permutation(128)
    _, c1, _ = pool.pool_block(x, g, b)
    _, c2, _ = pool.pool_block(x[perm], g, b[perm])
    np.testing.assert_allclose(c1, c2, rtol=1e-12)


def test_encode_entry_fp8_bounds():
    rng = np.random.default_rng(8)
    e = rng.standard_normal((200, 512)) * np.exp(rng.uniform(-5, 5, (200, 1)))
    enc = pool.encode_entry(e, 64, "fp8")
    s = enc["scale"].astype(np.float64)
    dec = quant.fp8_decode(enc["nope"]) * s[:, None]
    # the scale is minimal: the largest code magnitude lies in [224, 448]
    top = np.abs(quant.fp8_decode(enc["nope"])).max(axis=1)
    assert np.all((top >= 224) & (top <= 448))
    # each element within half a step of its binade
    a = np.abs(e[:, :448] / s[:, None])
    step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(a, 1e-300))), -6) - 3)
    assert np.all(np.abs(dec - e[:, :448]) <= 0.5 * step * s[:, None] * (1 + 1e-12))
    np.testing.assert_allclose(quant.bf16_decode(enc["rope"]), e[:, 448:], rtol=2 ** -8)
