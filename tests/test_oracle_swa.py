"""Pins of the oracle's window-only layer (the multi-token-prediction block).

* With no compressed entry visible (t < m - 1), an HCA layer attends to exactly the
  window and the sink, so the window-only layer over the same ring, queries and sink
  must give the same result (the HCA path is pinned by the attention and RoPE pins).
* Closed form: a one-token window and a sink logit far below every other leaves one
  softmax weight of 1, so o is that token rotated at its own position (the query's
  position) and lse is its logit.
"""
from dataclasses import replace
from types import SimpleNamespace

import numpy as np

import synth
from oracle import rope, step


def _swa_from(lay):
    return SimpleNamespace(mode="swa", m=1, fmt=lay.fmt, B=lay.B, W_cap=lay.W_cap, n_rows=0,
                           cache_row_start=np.zeros(lay.B, np.int64), win=lay.win, q=lay.q,
                           sink=lay.sink, q_pos=lay.q_pos, seq_id=lay.seq_id, pool=None)


def test_window_only_equals_hca_with_nothing_visible():
    from synth.gen import _decode_layer
    g = synth.FULL_GEOMETRY
    lens = np.array([100, 127, 60], np.int64)          # t = L - 1 < 127: no HCA entry visible
    hca = _decode_layer(np.random.default_rng(3), g, "hca", lens, 128, 1.0)
    ref = step.run_layer(hca, g)
    got = step.run_layer(_swa_from(hca), g)
    assert got["pooled"] is None and got["idx"] is None
    assert np.array_equal(got["o"], ref["o"]) and np.array_equal(got["lse"], ref["lse"])


def test_window_only_single_token_closed_form():
    g = replace(synth.TINY_GEOMETRY, n_win=1)
    lens = np.array([7, 33], np.int64)
    lay = synth.swa_layer(np.random.default_rng(4), g, lens, 8, fmt="f32")
    lay.sink = np.full(g.H, -1e4, np.float32)
    res = step.run_layer(lay, g)
    for n, L in enumerate(lens):
        t = int(L - 1)
        x = np.asarray(lay.win[n, t % 8], np.float64)
        k = rope.apply(x[None], np.array([t]), g.D_r, g.rope_base)[0]
        assert np.allclose(res["o"][n], np.broadcast_to(k, (g.H, g.D)), rtol=0, atol=1e-12)
        qh = rope.apply(np.asarray(lay.q[n], np.float64), t, g.D_r, g.rope_base)
        assert np.allclose(res["lse"][n], g.tau * (qh @ k), rtol=1e-12, atol=1e-12)
