"""GPU parity of attention with fewer than 64 query heads (16, 32, 48: the head
groups past H idle): CSA and HCA decode, a prefill, and the batch-invariant split.
Bars as in the other parity tests."""
from dataclasses import replace

import numpy as np
import pytest

import synth
from gpu_helpers import run_and_compare

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("H", [16, 32, 48])
def test_decode_fewer_heads(gpu, H):
    from synth.gen import _decode_layer
    g = replace(synth.FULL_GEOMETRY, H=H)
    lens = np.array([8192, 4099, 20000, 1024, 777], np.int64)
    for mode in ("csa", "hca"):
        lay = _decode_layer(np.random.default_rng(120 + H), g, mode, lens, 128, 1.0)
        _print(f"H={H} {mode} decode")
        run_and_compare(lay, g)


def test_prefill_and_split_fewer_heads(gpu):
    from long_context_attention_softmax_amd.layer import DeviceLayer
    g = replace(synth.FULL_GEOMETRY, H=16)
    w = synth.csa_prefill(seed=121, prefix=8192, T=256, g=g)
    _print("H=16 prefill (CSA, HCA)")
    for lay in w.layers:
        run_and_compare(lay, g, prefill=True)
    from synth.gen import _decode_layer
    g48 = replace(synth.FULL_GEOMETRY, H=48)
    lay = _decode_layer(np.random.default_rng(122), g48, "hca", np.array([65536, 300000, 5000], np.int64), 128, 1.0)
    dev = DeviceLayer.from_host(lay, g48)
    dev.split_chunks = 3
    _print("H=48 hca decode, split_chunks=3")
    run_and_compare(lay, g48, dev=dev)
