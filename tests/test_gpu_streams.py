"""Indexer calls that run in query groups, issued on two streams at once.

A quantized indexer call whose workspace would exceed 896 MiB is scored and
selected in query groups, the selection of one group on a second stream of the
library beside the scoring of the next, joined back to the caller's stream
through events.  Those streams and events belong to one (device, caller stream):
calls on two caller streams must not share them, or one call's event records
would release the other's waits early.  Here the same 1024-query chunk over a
1M-token prefix (three query groups) is selected on the default stream, then on
two streams concurrently, three times: every result must be the same bits.  The
single-stream result itself is checked against the oracle by the full-size
prefill test; this test covers the concurrency only.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


def test_grouped_indexer_on_two_streams(gpu):
    from long_context_attention_softmax_amd import _abi as A
    from long_context_attention_softmax_amd.layer import DeviceLayer
    from long_context_attention_softmax_amd.ops import hca_indexer_query_group
    w = synth.csa_prefill(seed=33, prefix=1 << 20, T=1024, with_hca=False)
    lay = DeviceLayer.from_host(w.layers[0], w.g)
    group = hca_indexer_query_group(lay.Nq, lay.max_visible, lay.qI.fmt, w.g.topk)
    _print(f"1024 queries over a 1M prefix: query groups of {group}")
    assert group < lay.Nq
    lay.pool()
    lay.select()
    torch.cuda.synchronize()
    ref = lay.idx.clone()
    assert int((ref >= 0).sum()) > 0
    other = lay.clone()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        lay.idx.fill_(-7)
        other.idx.fill_(-7)
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            lay.select()
        with torch.cuda.stream(sb):
            other.select()
        torch.cuda.synchronize()
        same_a, same_b = torch.equal(lay.idx, ref), torch.equal(other.idx, ref)
        _print(f"  repetition {rep}: stream A {'same' if same_a else 'DIFFERENT'}, "
               f"stream B {'same' if same_b else 'DIFFERENT'}")
        assert same_a and same_b
