"""GPU parity with 32 indexer heads (one 32-head tile; the workloads use 64): FP8
decode, MXFP4 decode (the decode tiling), MXFP4 decode over a paged cache, and an
MXFP4 prefill (256 queries: the XCD-major tiling).  Bars as in the other parity
tests (top-k sets and selected scores bit-exact, output per-row error <= 2e-2)."""
from dataclasses import replace

import numpy as np
import pytest

import synth
from gpu_helpers import run_and_compare

pytestmark = pytest.mark.gpu

G32 = replace(synth.FULL_GEOMETRY, H_I=32)


def _print(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("idx_fmt,page_rows", [("fp8", None), ("fp8", 32), ("mxfp4", None), ("mxfp4", 64)])
def test_decode_32_indexer_heads(gpu, idx_fmt, page_rows):
    from synth.gen import _decode_layer
    lens = np.array([8192, 4099, 30001, 1023, 5000], np.int64)
    lay = _decode_layer(np.random.default_rng(110), G32, "csa", lens, 128, 1.0, idx_fmt)
    _print(f"H_I=32 decode {idx_fmt} page_rows={page_rows}")
    run_and_compare(lay, G32, page_rows=page_rows)


@pytest.mark.parametrize("page_rows", [None, 128])
def test_prefill_32_indexer_heads(gpu, page_rows):
    w = synth.csa_prefill(seed=111, prefix=8192, T=256, g=G32)
    _print(f"H_I=32 prefill, 256 queries, page_rows={page_rows}")
    run_and_compare(w.layers[0], G32, prefill=True, page_rows=page_rows)
