"""GPU parity of the paged compressed cache: the same workloads as the contiguous
parity tests, with KV entries and indexer keys scattered over shuffled pages and
addressed through a block table (cache_row_start passed as NULL).  Bars are the
contiguous ones (pooled codes and top-k sets bit-exact, output per-row relative
error <= 2e-2 BF16/FP8, <= 1e-5 f32), and since only addresses change, the paged
step must also reproduce the contiguous step's idx, o and lse bit for bit."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import run_and_compare, to_np

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("page_rows", [1, 8])
def test_paged_tiny_f32(gpu, page_rows):
    w = synth.tiny(seed=0)
    for lay in w.layers:
        _print(f"paged tiny f32 page_rows={page_rows} layer={lay.mode}")
        run_and_compare(lay, w.g, page_rows=page_rows)


@pytest.mark.parametrize("idx_fmt,page_rows", [("fp8", 32), ("fp8", 256), ("mxfp4", 64)])
def test_paged_csa_decode_ragged(gpu, idx_fmt, page_rows):
    # lengths that leave partial last pages and a V that is not a multiple of 32
    lens = np.array([8192, 4099, 20001, 1023, 5000, 4100], np.int64)
    g = synth.FULL_GEOMETRY
    from synth.gen import _decode_layer
    lay = _decode_layer(np.random.default_rng(31), g, "csa", lens, 128, 1.0, idx_fmt)
    _print(f"paged csa decode {idx_fmt} page_rows={page_rows} lengths={lens.tolist()}")
    run_and_compare(lay, g, page_rows=page_rows)


@pytest.mark.parametrize("page_rows", [1, 16])
def test_paged_hca_decode(gpu, page_rows):
    w = synth.hca_decode(seed=13, B=2, L=65536)
    _print(f"paged hca decode B=2 L=65536 page_rows={page_rows}")
    run_and_compare(w.layers[0], w.g, page_rows=page_rows)


def test_paged_prefill_small(gpu):
    w = synth.csa_prefill(seed=15, prefix=16384, T=256)
    csa, hca = w.layers
    _print("paged prefill CSA (MXFP4 indexer, 256 queries) page_rows=128")
    run_and_compare(csa, w.g, prefill=True, page_rows=128)
    _print("paged prefill HCA page_rows=4")
    run_and_compare(hca, w.g, prefill=True, page_rows=4)


@pytest.mark.parametrize("idx_fmt", ["fp8", "mxfp4"])
def test_paged_step_bit_identical_to_contiguous(gpu, idx_fmt):
    from long_context_attention_softmax_amd.layer import DeviceLayer
    w = synth.ragged_pair(seed=14, B=6, lo=1024, hi=65536, round_every4=True, idx_fmt=idx_fmt)
    for lay in w.layers:
        _print(f"paged vs contiguous ragged pair {idx_fmt} layer={lay.mode}")
        outs = []
        for pr in (None, 64):
            dev = DeviceLayer.from_host(lay, w.g, page_rows=pr)
            dev.step()
            torch.cuda.synchronize()
            idx = to_np(dev.idx).copy() if dev.idx is not None else None
            outs.append((idx, to_np(dev.o).copy(), to_np(dev.lse).copy()))
        for a, b in zip(*outs):
            assert (a is None and b is None) or np.array_equal(a, b)


@pytest.mark.parametrize("idx_fmt", ["fp8", "mxfp4"])
def test_paged_with_fixed_split_bit_identical(gpu, idx_fmt):
    """Paging and the batch-invariant split together: the paged step with split_chunks
    reproduces the contiguous step with the same split bit for bit."""
    from long_context_attention_softmax_amd.layer import DeviceLayer
    w = synth.ragged_pair(seed=21, B=5, lo=2048, hi=200000, round_every4=True, idx_fmt=idx_fmt)
    for lay in w.layers:
        _print(f"paged + split_chunks=2 vs contiguous + split_chunks=2, {idx_fmt}, layer={lay.mode}")
        outs = []
        for pr in (None, 32):
            dev = DeviceLayer.from_host(lay, w.g, page_rows=pr)
            dev.split_chunks = 2
            dev.step()
            torch.cuda.synchronize()
            idx = to_np(dev.idx).copy() if dev.idx is not None else None
            outs.append((idx, to_np(dev.o).copy(), to_np(dev.lse).copy()))
        for a, b in zip(*outs):
            assert (a is None and b is None) or np.array_equal(a, b)
