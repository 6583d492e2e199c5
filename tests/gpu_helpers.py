"""Shared helpers of the GPU parity tests: run a workload layer on the HIP path and
compare each stage with the oracle."""
from __future__ import annotations

import numpy as np
import torch

from oracle import step as ostep

TOL_QUANT = 2e-2     # per-row relative error, BF16/FP8 paths
TOL_F32 = 1e-5       # per-row relative error, f32 path
# absolute lse error, BF16/FP8 paths.  lse moves by at most the largest logit error,
# and a logit errs by the BF16 rounding (2^-9 relative) of the rotated RoPE slice of
# q and of window keys: |dl| <= 2^-8 sum_rope |q_i k_i|, about 5e-3 for queries
# N(0,1)/sqrt(512) and N(0,1) keys.  Measured: at most 2.5e-3 (sets of a few keys,
# where one logit decides lse); 2e-4 .. 5e-4 for long sets.
TOL_LSE = 5e-3


def row_rel_err(o: np.ndarray, ref: np.ndarray) -> float:
    """max over (query, head) rows of max|o - ref| / max|ref|."""
    o = np.asarray(o, np.float64).reshape(-1, o.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((np.abs(o - ref).max(axis=1) / den).max())


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_codes_equal(got, want, fragile, what):
    got, want = np.asarray(got), np.asarray(want)
    bad = got != want
    if fragile is not None:
        bad &= ~np.asarray(fragile, bool)
    n = int(bad.sum())
    assert n == 0, f"{what}: {n} mismatching codes (of {bad.size}); first at {np.argwhere(bad)[:3].tolist()}"


def check_pool(dev, pooled, lay):
    """Compare the rows the GPU pooled with the oracle's encodings."""
    if pooled is None:                     # window-only layer: nothing pooled
        return
    rows = torch.from_numpy(dev.phys_rows(pooled["out_row"])).to(dev.device)
    kv = pooled["kv"]
    if rows.numel() == 0:
        return
    if dev.f32:
        got = to_np(dev.cache.f32[rows])
        assert_codes_equal(got.view(np.uint32), kv["f32"].view(np.uint32), kv["fragile"], "pooled f32 entry")
    else:
        D_n = kv["nope"].shape[1]
        fr = kv["fragile"]
        sc_ok = ~kv["scale_fragile"]
        got_s = to_np(dev.cache.scale[rows])
        assert np.array_equal(got_s[sc_ok], kv["scale"][sc_ok]), "pooled entry scales differ"
        keep = sc_ok & (got_s == kv["scale"])
        assert_codes_equal(to_np(dev.cache.nope[rows])[keep], kv["nope"][keep], fr[keep, :D_n], "pooled FP8 nope")
        assert_codes_equal(to_np(dev.cache.rope[rows]).view(np.uint16), kv["rope"], fr[:, D_n:], "pooled BF16 rope")
    if "idx" in pooled:
        ix = pooled["idx"]
        if "f32" in ix:
            got = to_np(dev.keys.data[rows])
            assert_codes_equal(got.view(np.uint32), ix["f32"].view(np.uint32), ix["fragile"], "pooled f32 key")
        elif "fp8" in ix:
            assert_codes_equal(to_np(dev.keys.data[rows]), ix["fp8"], ix["fragile"], "pooled FP8 key")
        else:
            got_c = to_np(dev.keys.data[rows])
            got_s = to_np(dev.keys.scales[rows])
            fr = ix["fragile"]
            blk_fr = fr.reshape(fr.shape[0], -1, 32).any(axis=2)
            assert_codes_equal(got_s, ix["scales"], blk_fr, "pooled MXFP4 key scales")
            # compare element codes through their nibbles
            lo_g, hi_g = got_c & 15, got_c >> 4
            lo_w, hi_w = ix["codes"] & 15, ix["codes"] >> 4
            assert_codes_equal(lo_g, lo_w, fr[:, 0::2], "pooled MXFP4 key (even)")
            assert_codes_equal(hi_g, hi_w, fr[:, 1::2], "pooled MXFP4 key (odd)")


def oracle_layer(lay, g, queries=None, threads=1):
    """The oracle's step of one layer; with ``threads`` > 1 the queries are split
    over a thread pool (the layer is pooled once; numpy releases the GIL inside its
    large array operations) and the per-query results are joined in query order."""
    if threads <= 1 or queries is None or len(queries) < 2:
        return ostep.run_layer(lay, g, queries=queries)
    from concurrent.futures import ThreadPoolExecutor
    pooled = None if lay.mode == "swa" else ostep.pool_layer(lay, g)
    qs = [int(q) for q in queries]
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda q: ostep.run_layer(lay, g, queries=[q], pooled=pooled), qs))
    ref = dict(parts[0])
    for key in ("idx", "sel_scores", "o", "lse", "queries"):
        if ref[key] is not None:
            ref[key] = np.concatenate([p[key] for p in parts])
    ref["kth_gaps"] = [x for p in parts for x in p["kth_gaps"]]
    return ref


# the largest errors seen by run_and_compare in this process: (output, lse) per path
MAX_ERR = {"quant": [0.0, 0.0], "f32": [0.0, 0.0]}


def run_and_compare(lay, g, dev=None, queries=None, prefill=False, tol=None, check_scores=True,
                    page_rows=None, oracle_threads=1, fused=False):
    """Run the layer's step on the GPU and compare every stage with the oracle.
    ``page_rows`` lays the compressed cache out in shuffled pages of that size;
    ``fused`` runs the decode step as one hca_decode_layer call (pooling, top-k and
    attention; the selected scores still come back) instead of three calls.

    Returns (oracle result, device layer, output error)."""
    from long_context_attention_softmax_amd.layer import DeviceLayer
    from long_context_attention_softmax_amd.ops import hca_decode_layer
    dev = dev or DeviceLayer.from_host(lay, g, page_rows=page_rows)
    tol = tol if tol is not None else (TOL_F32 if dev.f32 else TOL_QUANT)
    score = None
    if dev.mode == 0:
        score = torch.zeros((dev.Nq, g.topk), dtype=torch.float64 if dev.f32 else torch.float32,
                            device=dev.device)
    if fused and not prefill:
        o = hca_decode_layer(dev._attend_kw(), pool=dev._pool_kw(),
                             indexer=dev._select_kw(score=score) if dev.mode == 0 else None)
    else:
        dev.pool()
        if dev.mode == 0:
            dev.select(score=score)
        o = dev.attend(prefill=prefill)
    torch.cuda.synchronize()
    ref = oracle_layer(lay, g, queries=queries, threads=oracle_threads)
    qs = ref["queries"]
    check_pool(dev, ref["pooled"], lay)
    if dev.mode == 0:
        got_idx = to_np(dev.idx)[qs]
        for n in range(len(qs)):
            assert np.array_equal(got_idx[n], ref["idx"][n]), \
                f"top-k set differs for query {qs[n]} (t={lay.q_pos[qs[n]]})"
        if check_scores:
            # the scores behind the selection: bit-exact on the quantized paths
            # (exact dots, one canonical head sum), fp64 on the f32 path
            got_sc = to_np(score)[qs].astype(np.float64)
            want = ref["sel_scores"]
            if dev.f32:
                np.testing.assert_allclose(got_sc, want, rtol=1e-12, atol=0)
            else:
                assert np.array_equal(got_sc, want), \
                    f"selected scores differ: max |diff| {np.abs(got_sc - want).max():.3e}"
    got_o = to_np(o)[qs]
    got_o = got_o.astype(np.float64) if dev.f32 else bf16_values(got_o)
    err = row_rel_err(got_o, ref["o"])
    assert err <= tol, f"output rel err {err:.3e} > {tol}"
    lse = to_np(dev.lse)[qs]
    lse_err = float(np.abs(lse - ref["lse"]).max()) if lse.size else 0.0
    path = "f32" if dev.f32 else "quant"
    MAX_ERR[path] = [max(MAX_ERR[path][0], err), max(MAX_ERR[path][1], lse_err)]
    print(f"  parity ({path}): output rel err {err:.3e}, lse abs err {lse_err:.3e}", flush=True)
    # lse: float32 storage on the f32 path; TOL_LSE on the BF16 path
    if dev.f32:
        assert np.allclose(lse, ref["lse"], rtol=1e-6, atol=1e-6)
    else:
        assert lse_err <= TOL_LSE, f"lse abs err {lse_err:.3e} > {TOL_LSE}"
    return ref, dev, err
