"""GPU check of the allocation-free decode entry point (hca_attn_decode_noalloc),
called through the C ABI: on the same inputs it must give the same o and lse bits as
hca_attn_decode with a caller workspace (same kernels, same plan), on two calls in a
row, the second with a smaller batch; the default plan (partials of split queries in
the scratch) and a fixed split are both covered, as is a call whose scratch need
exceeds the static array (refused before any launch)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


def _run(dev, noalloc, n=None):
    """Attention of the first n queries of the device layer (all by default)."""
    from long_context_attention_softmax_amd import ops
    from long_context_attention_softmax_amd import _abi as A
    n = dev.Nq if n is None else n
    g = dev.g
    o = torch.full_like(dev.q[:n], 3.0)
    lse = torch.full((n, g.H), -5.0, dtype=torch.float32, device=dev.device)
    fn = ops.hca_attn_decode_noalloc if noalloc else ops.hca_attn_decode
    fn(dev.q[:n].contiguous(), dev.cache, dev.cache_row_start, dev.win, dev.sink, dev.seq_id[:n].contiguous(),
       dev.q_pos[:n].contiguous(), mode=dev.mode, m=dev.m, n_win=g.n_win, D_r=g.D_r,
       max_visible=dev.max_visible, k=g.topk if dev.mode == A.MODE_CSA else 0,
       idx=dev.idx[:n].contiguous() if dev.mode == A.MODE_CSA else None, tau=g.tau, rope_base=g.rope_base,
       o=o, lse=lse, pages=dev.pages, split_chunks=dev.split_chunks)
    torch.cuda.synchronize()
    return o.view(torch.int16).cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("split", [0, 2])
def test_noalloc_decode_matches_workspace_call(gpu, split):
    from long_context_attention_softmax_amd.layer import DeviceLayer
    # the default plan fits any 1M context; a fixed split keeps partials per run, so
    # its case has shorter contexts (up to 128K) to stay inside the static scratch
    w = synth.ragged_pair(seed=71, B=24, lo=4096, hi=1 << 20 if split == 0 else 1 << 17)
    for lay in w.layers:
        dev = DeviceLayer.from_host(lay, w.g)
        dev.split_chunks = split
        if lay.mode == "csa":
            dev.pool()
            dev.select()
        for n in (dev.Nq, 7):                      # two calls in a row, the second smaller
            _print(f"no-alloc decode: layer {lay.mode}, split_chunks={split}, {n} queries")
            o_ws, l_ws = _run(dev, False, n)
            o_na, l_na = _run(dev, True, n)
            assert np.array_equal(o_na, o_ws), "o differs from the workspace call"
            assert np.array_equal(l_na, l_ws), "lse differs from the workspace call"
            rows = o_na.view(np.uint16).reshape(-1, o_na.shape[-1])
            assert not np.any(np.all(rows == np.uint16(0x4040), axis=1)), "an output row was left unwritten"


def test_noalloc_refuses_a_call_beyond_its_scratch(gpu):
    from long_context_attention_softmax_amd import _abi as A
    from long_context_attention_softmax_amd.layer import DeviceLayer
    w = synth.hca_decode(seed=72, B=200, L=1 << 16)
    dev = DeviceLayer.from_host(w.layers[0], w.g)
    dev.split_chunks = 1                            # 200 queries x 10 runs of 64 KiB partials: > 40 MiB
    with pytest.raises(A.HcaError) as e:
        _run(dev, True)
    assert e.value.code == -6 and "scratch" in str(e.value)
