"""GPU parity at the full workload sizes, through the same device path and kernel
launches that bench.py times (DeviceLayer pool -> select -> attend, one call each).

Decode workloads are checked on every query (a decode step has one per sequence, so
the oracle still finishes in seconds); the 4096-token prefill chunk is checked on a
seeded sample of 128 queries that covers both ends of every 512-query block, both
ends of the first and last 8-query groups of each block (the MXFP4 scoring grid
interleaves 8-query groups over the XCDs), the first and last eight queries of the
chunk, and random ones (the oracle runs them on a thread pool).  Bars are those of the small parity tests: pooled codes and
top-k sets and selected scores bit-exact, output per-row relative error <= 2e-2.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import run_and_compare

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name,over,page_rows", [("csa_decode_128k", {}, None), ("hca_decode_1m", {}, None),
                                                 ("ragged_pair_32", {}, None),
                                                 ("ragged_pair_32", {"idx_fmt": "mxfp4"}, None),
                                                 ("ragged_pair_32", {}, 256)])
def test_full_size_decode_every_query(gpu, name, over, page_rows):
    w = synth.make(name, **over)
    for lay in w.layers:
        _print(f"{name} {over} page_rows={page_rows} layer={lay.mode} queries={len(lay.q_pos)} "
               f"lengths={[int(x) for x in w.lengths]}")
        ref, dev, err = run_and_compare(lay, w.g, page_rows=page_rows)
        assert len(ref["queries"]) == len(lay.q_pos)
        _print(f"  rel err {err:.2e}")


def _prefill_sample(nq, group, seed=7, n=128):
    """At least ``n`` seeded queries of the chunk: the first and last query of every
    512-query block (the first and last 8-query group of each block at both ends),
    the eight queries the XCD-major scoring order spreads over the eight XCDs at
    each end of the chunk, both sides of the indexer's query-group boundaries, then
    random ones."""
    fixed = []
    for b0 in range(0, nq, 512):
        fixed += [b0, b0 + 7, b0 + 8, b0 + 504, b0 + 511]
    fixed += list(range(8)) + list(range(nq - 8, nq)) + [255, 256, 2047, 2048]
    # both sides of each query-group boundary of the indexer at this size
    for g0 in range(group, nq, group):
        fixed += [g0 - 1, g0]
    got = set(q for q in fixed if 0 <= q < nq)
    rng = np.random.default_rng(seed)
    while len(got) < min(n, nq):
        got.add(int(rng.integers(0, nq)))
    return sorted(got)


def test_full_size_prefill_sampled_queries(gpu):
    w = synth.make("csa_prefill_1m")
    csa, hca = w.layers
    from long_context_attention_softmax_amd import _abi as A
    from long_context_attention_softmax_amd.ops import hca_indexer_query_group
    nq = len(csa.q_pos)
    group = hca_indexer_query_group(nq, int(((csa.q_pos + 1) // csa.m).max()), A.MXFP4, w.g.topk)
    assert 256 <= group < nq                             # the call runs in several groups
    qs = _prefill_sample(nq, group)
    _print(f"csa_prefill_1m CSA layer (MXFP4 indexer) prefix={w.prefix} T={w.T} group={group} "
           f"{len(qs)} queries: {qs}")
    ref, dev, err = run_and_compare(csa, w.g, queries=qs, prefill=True, oracle_threads=16)
    _print(f"  rel err {err:.2e}")
    qh = _prefill_sample(len(hca.q_pos), group, seed=8)
    _print(f"csa_prefill_1m HCA layer {len(qh)} queries: {qh}")
    ref, dev, err = run_and_compare(hca, w.g, queries=qh, prefill=True, oracle_threads=16)
    _print(f"  rel err {err:.2e}")
