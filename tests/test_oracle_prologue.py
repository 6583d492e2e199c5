"""Pins of the oracle's query / key-value normalization (oracle/prologue.py):
a worked example computed by hand (tests/golden/rmsnorm_worked_example.txt),
the closed form of the output's mean square, scale and sign invariance, and the
ring placement the window branch reads back."""
import os

import numpy as np

from oracle import attend, prologue, quant

GOLD = os.path.join(os.path.dirname(__file__), "golden", "rmsnorm_worked_example.txt")


def test_worked_examples():
    n = 0
    for line in open(GOLD):
        if line.startswith("#") or not line.strip():
            continue
        eps, x, gamma, y = [p.split() for p in line.split("|")]
        got = prologue.rms_norm(np.array(x, float), np.array(gamma, float), float(eps[0]))
        assert np.allclose(got, np.array(y, float), rtol=1e-15, atol=0)
        n += 1
    assert n == 2


def test_mean_square_closed_form_and_invariances():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(5, 512)) * rng.uniform(0.01, 10, size=(5, 1))
    one = np.ones(512)
    for eps in (0.0, 1e-6, 0.5):
        y = prologue.rms_norm(x, one, eps)
        ms = np.mean(x * x, axis=1)
        assert np.allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-13)
    g = rng.uniform(0.5, 2, 512)
    y = prologue.rms_norm(x, g, 0.0)
    assert np.allclose(prologue.rms_norm(7.25 * x, g, 0.0), y, rtol=1e-14)
    assert np.array_equal(prologue.rms_norm(-x, g, 0.0), -y)
    assert np.allclose(y / g, prologue.rms_norm(x, one, 0.0), rtol=1e-14)   # gamma scales each dim


def test_encode_and_ring_placement():
    rng = np.random.default_rng(1)
    y = rng.normal(size=(3, 16))
    bits, fr = prologue.encode(y, "bf16")
    assert np.array_equal(quant.bf16_decode(bits), quant.bf16_round(y)[0])
    f, _ = prologue.encode(y, "f32")
    assert np.array_equal(f.view(np.float32), y.astype(np.float32))
    ring = np.zeros((2, 8, 16))
    out = prologue.append_ring(ring, np.array([1, 0, 1]), np.array([9, 3, 18]), y)
    # the window reader finds token u of sequence b at slot u mod W_cap
    assert np.array_equal(attend.window_keys(out, 1, 18, 1, 8, 0, 1e4)[0], y[2])
    assert np.array_equal(attend.window_keys(out, 0, 3, 1, 8, 0, 1e4)[0], y[1])
    assert np.array_equal(out[1, 1], y[0]) and np.count_nonzero(out) == 3 * 16
