"""GPU parity with small top-k: k = 1 (the single best entry), k = 7 (odd) and
k = 64 in decode, and k = 1 in a 256-query prefill (the many-query select path).
Bars as in the other parity tests (top-k sets and selected scores bit-exact)."""
from dataclasses import replace

import numpy as np
import pytest

import synth
from gpu_helpers import run_and_compare

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("k", [1, 7, 64])
def test_decode_small_k(gpu, k):
    from synth.gen import _decode_layer
    g = replace(synth.FULL_GEOMETRY, topk=k)
    lens = np.array([8192, 4099, 30000, 12, 200], np.int64)       # V from 3 to 7500
    lay = _decode_layer(np.random.default_rng(140 + k), g, "csa", lens, 128, 1.0)
    _print(f"decode k={k}")
    run_and_compare(lay, g)


def test_prefill_top1(gpu):
    g = replace(synth.FULL_GEOMETRY, topk=1)
    w = synth.csa_prefill(seed=141, prefix=8192, T=256, g=g)
    _print("prefill k=1, 256 queries")
    run_and_compare(w.layers[0], g, prefill=True)
