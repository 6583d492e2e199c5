"""Batch-invariant decode (fixed split): with split_chunks > 0 a query's top-k set,
output and lse must be the same bits whatever other queries share the launch and in
whatever order, and must still match the oracle within the usual bars (top-k sets
and selected scores bit-exact, output per-row relative error <= 2e-2)."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import run_and_compare, to_np

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


def _subset(dev, rows):
    """The same layer and caches, with the decode batch cut down (or repeated,
    reordered) to the query rows ``rows`` of ``dev``."""
    import copy
    from long_context_attention_softmax_amd.ops import IdxCache
    r = torch.as_tensor(np.asarray(rows, np.int64), device=dev.device)
    s = copy.copy(dev)
    s.Nq = len(rows)
    s.q = dev.q.index_select(0, r).contiguous()
    s.seq_id = dev.seq_id.index_select(0, r).contiguous()
    s.q_pos = dev.q_pos.index_select(0, r).contiguous()
    s.o = torch.empty_like(s.q)
    s.lse = torch.empty((s.Nq, dev.lse.shape[1]), dtype=dev.lse.dtype, device=dev.device)
    if dev.idx is not None:
        s.w = dev.w.index_select(0, r).contiguous()
        sc = dev.qI.scales.index_select(0, r).contiguous() if dev.qI.scales is not None else None
        s.qI = IdxCache(dev.qI.data.index_select(0, r).contiguous(), dev.qI.fmt, sc)
        s.idx = torch.empty((s.Nq, dev.idx.shape[1]), dtype=dev.idx.dtype, device=dev.device)
    return s


def _run(dev):
    if dev.idx is not None:
        dev.select()
    dev.attend()
    torch.cuda.synchronize()
    idx = to_np(dev.idx).copy() if dev.idx is not None else None
    return idx, to_np(dev.o).copy(), to_np(dev.lse).copy()


def _check_invariant(dev, batches):
    """Every batch (a list of query rows of dev) gives each query the bits it gets alone."""
    alone = [_run(_subset(dev, [n])) for n in range(dev.Nq)]
    for rows in batches:
        got = _run(_subset(dev, rows))
        for i, n in enumerate(rows):
            for part, a, b in zip(("idx", "o", "lse"), got, alone[n]):
                if a is None:
                    continue
                assert np.array_equal(a[i], b[0]), f"query {n} ({part}) differs in a batch of {len(rows)}"


def _decode_layer(mode, lens, seed, idx_fmt="fp8"):
    from synth.gen import _decode_layer
    g = synth.FULL_GEOMETRY
    return _decode_layer(np.random.default_rng(seed), g, mode, np.asarray(lens, np.int64), 128, 1.0, idx_fmt), g


@pytest.mark.parametrize("mode,split", [("csa", 1), ("csa", 3), ("hca", 2), ("hca", 5)])
def test_fixed_split_parity(gpu, mode, split):
    from long_context_attention_softmax_amd.layer import DeviceLayer
    lens = [8192, 4099, 20001, 1023, 5000, 300000] if mode == "csa" else [65536, 4100, 200000, 129, 12800]
    lay, g = _decode_layer(mode, lens, 40 + split)
    dev = DeviceLayer.from_host(lay, g)
    dev.split_chunks = split
    _print(f"fixed split {mode} split_chunks={split} lengths={lens}")
    run_and_compare(lay, g, dev=dev)


@pytest.mark.parametrize("mode,split,idx_fmt", [("csa", 2, "fp8"), ("csa", 1, "mxfp4"), ("hca", 3, "fp8")])
def test_batch_composition_invariance(gpu, mode, split, idx_fmt):
    from long_context_attention_softmax_amd.layer import DeviceLayer
    lens = [4096, 9000, 131072, 5003, 70000, 4100, 1 << 20, 12345] if mode == "csa" else \
        [4096, 9000, 131072, 5120, 70000, 4100, 1 << 20, 12800]
    lay, g = _decode_layer(mode, lens, 50 + split, idx_fmt)
    dev = DeviceLayer.from_host(lay, g)
    dev.split_chunks = split
    dev.pool()                     # the step's newly completed blocks, once
    n = dev.Nq
    rng = np.random.default_rng(5)
    big = rng.integers(0, n, 300).tolist()     # 300 queries: the many-query paths of the launch plans
    _print(f"batch invariance {mode} split_chunks={split} {idx_fmt}: full, reversed, subset, 300 queries")
    _check_invariant(dev, [list(range(n)), list(range(n))[::-1], [6, 2, 0], big])


def test_full_size_ragged_pair_batch_invariant(gpu):
    from long_context_attention_softmax_amd.layer import DeviceLayer
    w = synth.make("ragged_pair_32")
    for lay in w.layers:
        dev = DeviceLayer.from_host(lay, w.g)
        dev.split_chunks = 2
        _print(f"ragged_pair_32 layer={lay.mode} split_chunks=2: every query against the oracle")
        run_and_compare(lay, w.g, dev=dev)
        _print("  each query alone, reversed batch")
        _check_invariant(dev, [list(range(dev.Nq))[::-1]])
