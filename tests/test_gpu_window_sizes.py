"""GPU parity with other window sizes than the workloads' 128: one token, exactly
one 64-slot chunk, and 300 tokens (five chunks, the last partly filled) in CSA and
HCA decode; 256 tokens (four chunks) in a prefill.  Bars as in the other parity tests."""
from dataclasses import replace

import numpy as np
import pytest

import synth
from gpu_helpers import run_and_compare

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("n_win", [1, 64, 300])
def test_decode_window_sizes(gpu, n_win):
    from synth.gen import _decode_layer
    g = replace(synth.FULL_GEOMETRY, n_win=n_win)
    lens = np.array([8192, 4099, 20000, 256, 100], np.int64)
    W = -(-max(n_win, 128) // 128) * 128            # a multiple of m: no block wraps the ring
    for mode in ("csa", "hca"):
        lay = _decode_layer(np.random.default_rng(130 + n_win), g, mode, lens, W, 1.0)
        _print(f"n_win={n_win} {mode} decode")
        run_and_compare(lay, g)


def test_prefill_window_256(gpu):
    # the prefill generator needs T and T + n_win to be multiples of 128
    g = replace(synth.FULL_GEOMETRY, n_win=256)
    w = synth.csa_prefill(seed=131, prefix=4096, T=128, g=g)
    _print("n_win=256 prefill (CSA, HCA): four window chunks")
    for lay in w.layers:
        run_and_compare(lay, g, prefill=True)
