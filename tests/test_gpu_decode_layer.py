"""The one-call decode step (hca_decode_layer) against the three calls it stands for.

On cloned device layers, the step through hca_decode_layer and the step as
hca_kv_compress, hca_indexer_topk (CSA) and hca_attn_decode called one after another
must agree bit for bit: the top-k lists, o, lse and every pooled row (KV entry and
index key).  Before each run the rows the step pools are overwritten with the
largest codes, so a scoring or attention workgroup that read a pooled row before the
pooling wrote it would change the result: the FP8 pooling that rides in the
scoring (CSA, FP8 keys) or attention (HCA) launch is checked for its wait, not only
for its arithmetic.  Cases: FP8 and MXFP4 indexer keys (pooling inside the scoring
launch; the MXFP4 tile that holds the new row read with coherent loads), paged caches, many blocks per launch (64
sequences, all completing a block), the pooled entry as the only entry, HCA layers
(pooling inside the attention launch, default plan and fixed split), the f32 tiny
layers (separate launches), and the profiled form."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import run_and_compare, to_np

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


def _poison(dev):
    """Largest codes in the rows this step pools."""
    rows = dev.out_row.long()
    if rows.numel() == 0:
        return
    c = dev.cache
    if c.f32 is not None:
        c.f32[rows] = 3.0e38
    else:
        c.nope[rows] = 0x7E                       # FP8 448
        c.rope.view(torch.int16)[rows] = 0x7F00   # BF16 1.7e38
        c.scale[rows] = 2.0 ** 20
    if dev.mode == 0:
        k = dev.keys
        if k.fmt == 0:
            k.data[rows] = 3.0e38
        elif k.fmt == 2:
            k.data[rows] = 0x7E
        else:
            k.data[rows] = 0x77                   # E2M1 +6 in both nibbles
            k.scales[rows] = 254                  # 2^127


def _state(dev):
    rows = dev.out_row.long()
    out = [to_np(dev.o).copy(), to_np(dev.lse).copy()]
    if dev.mode == 0:
        out.append(to_np(dev.idx).copy())
        out.append(to_np(dev.keys.data[rows]).copy())
        if dev.keys.scales is not None:
            out.append(to_np(dev.keys.scales[rows]).copy())
    c = dev.cache
    for p in (c.f32, c.nope, c.rope, c.scale):
        if p is not None:
            out.append(to_np(p[rows]).copy())
    return out


def _compare(lay, g, page_rows=None, split_chunks=0, prof=False):
    from long_context_attention_softmax_amd.layer import DeviceLayer
    base = DeviceLayer.from_host(lay, g, page_rows=page_rows)
    base.split_chunks = split_chunks
    _poison(base)
    runs = []
    for fused in (False, True):
        dev = base.clone()
        p = None
        if prof and fused:
            p = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        dev.step(fused=fused, prof_select=p, prof_attend=p)
        torch.cuda.synchronize()
        if p is not None:
            assert p[0].elapsed_time(p[1]) > 0.0
        runs.append(_state(dev))
    names = ["o", "lse", "idx", "keys", "key scales", "cache planes"]
    for i, (a, b) in enumerate(zip(*runs)):
        assert np.array_equal(a, b), f"{names[min(i, 5)]} differs between the fused and the separate step"


@pytest.mark.parametrize("idx_fmt", ["fp8", "mxfp4"])
def test_decode_layer_ragged_pair(gpu, idx_fmt):
    w = synth.ragged_pair(seed=41, B=12, lo=1024, hi=200000, round_every4=True, idx_fmt=idx_fmt)
    for lay in w.layers:
        _print(f"decode layer {lay.mode} {idx_fmt}: lengths {w.lengths.tolist()}, "
               f"{len(lay.pool['out_row'])} blocks pooled")
        _compare(lay, w.g)


@pytest.mark.parametrize("idx_fmt,page_rows", [("fp8", 64), ("mxfp4", 32)])
def test_decode_layer_paged(gpu, idx_fmt, page_rows):
    w = synth.ragged_pair(seed=42, B=9, lo=1024, hi=65536, round_every4=True, idx_fmt=idx_fmt)
    for lay in w.layers:
        _print(f"decode layer paged {lay.mode} {idx_fmt} page_rows={page_rows}")
        _compare(lay, w.g, page_rows=page_rows)


def test_decode_layer_every_sequence_pools(gpu):
    # 64 sequences at L = 8192: every query's newest entry is pooled in this step
    w = synth.csa_decode(seed=43, B=64, L=8192)
    _print("decode layer CSA B=64 L=8192: 64 blocks pooled, 64 waiting workgroups")
    _compare(w.layers[0], w.g)


def test_decode_layer_single_entry(gpu):
    # L = 4: the pooled entry is the only visible one (V = 1)
    w = synth.csa_decode(seed=44, B=3, L=4)
    _print("decode layer CSA B=3 L=4: the pooled entry is the only entry")
    _compare(w.layers[0], w.g)


def test_decode_layer_hca_and_split(gpu):
    w = synth.hca_decode(seed=45, B=3, L=65536)
    _print("decode layer HCA B=3 L=65536, default plan and split_chunks=3")
    _compare(w.layers[0], w.g)
    _compare(w.layers[0], w.g, split_chunks=3)


def test_decode_layer_tiny_f32(gpu):
    w = synth.tiny(seed=0)
    for lay in w.layers:
        _print(f"decode layer tiny f32 {lay.mode}")
        _compare(lay, w.g)


def test_decode_layer_profiled(gpu):
    w = synth.ragged_pair(seed=46, B=6, lo=4096, hi=65536, round_every4=True)
    for lay in w.layers:
        _print(f"decode layer profiled {lay.mode}")
        _compare(lay, w.g, prof=True)


@pytest.mark.parametrize("idx_fmt", ["fp8", "mxfp4"])
def test_decode_layer_matches_the_oracle(gpu, idx_fmt):
    # the fused step against the oracle directly: pooled codes, exact top-k and its
    # scores, outputs within the bars
    w = synth.ragged_pair(seed=47, B=10, lo=2048, hi=300000, round_every4=True, idx_fmt=idx_fmt)
    for lay in w.layers:
        _print(f"decode layer vs oracle {lay.mode} {idx_fmt}: {len(lay.pool['out_row'])} blocks pooled")
        run_and_compare(lay, w.g, fused=True, oracle_threads=8)
