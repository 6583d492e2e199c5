"""GPU parity at the full workload sizes, through the same device path and kernel
launches that bench.py times (DeviceLayer pool -> select -> attend, one call each).

Decode workloads are checked on every query (a decode step has one per sequence, so
the oracle still finishes in seconds); the 4096-token prefill chunk is checked on a
seeded sample of queries that covers the first and last positions, both ends of
each 8-query group the MXFP4 scoring grid interleaves over the XCDs, and queries in
different key chunks.  Bars are those of the small parity tests: pooled codes and
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


def _prefill_sample(nq, seed=7):
    fixed = [0, 1, 7, 8, 255, 256, 2047, nq - 8, nq - 1]
    rng = np.random.default_rng(seed)
    extra = rng.choice(nq, size=3, replace=False).tolist()
    return sorted(set(int(q) for q in fixed + extra if 0 <= q < nq))


def test_full_size_prefill_sampled_queries(gpu):
    w = synth.make("csa_prefill_1m")
    csa, hca = w.layers
    qs = _prefill_sample(len(csa.q_pos))
    _print(f"csa_prefill_1m CSA layer (MXFP4 indexer) prefix={w.prefix} T={w.T} queries={qs}")
    ref, dev, err = run_and_compare(csa, w.g, queries=qs, prefill=True)
    _print(f"  rel err {err:.2e}")
    qh = _prefill_sample(len(hca.q_pos), seed=8)
    _print(f"csa_prefill_1m HCA layer queries={qh}")
    ref, dev, err = run_and_compare(hca, w.g, queries=qh, prefill=True)
    _print(f"  rel err {err:.2e}")
