"""GPU parity of the layer variants: the window-only layer of the
multi-token-prediction block (HCA_MODE_SWA: sliding window and sink, no compressed
cache), in decode, prefill, the f32 path and the batch-invariant split.  Bars as in
the other parity tests: output per-row relative error <= 2e-2 (BF16) / 1e-5 (f32)."""
from dataclasses import replace

import numpy as np
import pytest

import synth
from gpu_helpers import run_and_compare

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


def test_window_only_decode_bf16(gpu):
    g = synth.FULL_GEOMETRY
    lens = np.array([1, 50, 128, 129, 4096, 1 << 20, 777], np.int64)   # windows shorter than n_win too
    lay = synth.swa_layer(np.random.default_rng(61), g, lens, 128)
    _print(f"window-only decode lengths={lens.tolist()}")
    run_and_compare(lay, g)


def test_window_only_f32(gpu):
    g = synth.TINY_GEOMETRY
    lens = np.array([3, 40, 300], np.int64)
    lay = synth.swa_layer(np.random.default_rng(62), g, lens, max(g.n_win, 8), fmt="f32")
    _print(f"window-only f32 lengths={lens.tolist()} n_win={g.n_win}")
    run_and_compare(lay, g)


def test_window_only_prefill(gpu):
    from synth.gen import _bf16_normal
    g = synth.FULL_GEOMETRY
    L, T, W_cap = 5000, 256, 512            # 256 queries of one sequence; the ring holds T + n_win tokens
    rng = np.random.default_rng(63)
    lay = synth.swa_layer(rng, g, np.array([L], np.int64), W_cap)
    lay.q_pos = np.arange(L - T, L, dtype=np.int64)
    lay.seq_id = np.zeros(T, np.int32)
    lay.q = _bf16_normal(rng, (T, g.H, g.D), 1 / np.sqrt(g.D))
    _print("window-only prefill, 256 queries")
    run_and_compare(lay, g, prefill=True)


def test_window_only_fixed_split_invariant(gpu):
    from long_context_attention_softmax_amd.layer import DeviceLayer
    from test_gpu_batch_invariant import _check_invariant
    g = replace(synth.FULL_GEOMETRY)
    lens = np.array([1, 70, 128, 500, 1 << 16], np.int64)
    lay = synth.swa_layer(np.random.default_rng(64), g, lens, 128)
    dev = DeviceLayer.from_host(lay, g)
    dev.split_chunks = 1
    _print("window-only, split_chunks=1: parity, then each query alone vs reversed batch")
    run_and_compare(lay, g, dev=dev)
    _check_invariant(dev, [list(range(dev.Nq))[::-1]])


@pytest.mark.parametrize("split", [0, 1])
def test_window_only_empty_set(gpu, split):
    """n_win = 0 in the window-only mode: every set is empty, so o = 0 and lse = the
    sink (the oracle's attention over no keys).  split_chunks = 1 asks for the fixed
    split, but with every set empty no query has a run and the launch takes the
    default plan; test_hca_empty_and_nonempty_sets_mixed runs the split itself with
    empty sets beside non-empty ones."""
    from long_context_attention_softmax_amd.layer import DeviceLayer
    g = replace(synth.FULL_GEOMETRY, n_win=0)
    lens = np.array([1, 300, 5000], np.int64)
    lay = synth.swa_layer(np.random.default_rng(65), g, lens, 16)
    dev = DeviceLayer.from_host(lay, g)
    dev.split_chunks = split
    _print(f"window-only with n_win=0, split_chunks={split}")
    ref, _, err = run_and_compare(lay, g, dev=dev)
    assert np.all(ref["o"] == 0) and err == 0.0


@pytest.mark.parametrize("split", [0, 1, 2])
def test_hca_empty_and_nonempty_sets_mixed(gpu, split):
    """An HCA layer with no window (n_win = 0) whose queries at t < m - 1 see no entry
    (empty set: o = 0, lse = the sink) next to queries that see a few entries.  With
    split_chunks 1 or 2 every non-empty set is one run (split_runs = 1, so no combine
    is launched): the empty sets must still be written."""
    from long_context_attention_softmax_amd.layer import DeviceLayer
    from synth.gen import _decode_layer
    g = replace(synth.FULL_GEOMETRY, n_win=0)
    lens = np.array([100, 1000, 127, 5000, 1, 3000], np.int64)       # V = 0, 7, 0, 39, 0, 23
    lay = _decode_layer(np.random.default_rng(66), g, "hca", lens, 128, 1.0)
    dev = DeviceLayer.from_host(lay, g)
    dev.split_chunks = split
    _print(f"HCA n_win=0, mixed empty sets, split_chunks={split} (one 64-entry chunk per set at most)")
    dev.o.fill_(1.0)                        # stale contents must be overwritten
    dev.lse.fill_(-7.0)
    ref, _, err = run_and_compare(lay, g, dev=dev)
    empty = (lens - 1 + 1) // g.m_hca == 0
    assert np.all(ref["o"][empty] == 0)
    got_o = dev.o.float().cpu().numpy()
    assert np.all(got_o[empty] == 0)
    got_lse = dev.lse.cpu().numpy()
    assert np.array_equal(got_lse[empty], np.broadcast_to(lay.sink.astype(np.float32), got_lse[empty].shape))
