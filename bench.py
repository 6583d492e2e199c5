#!/usr/bin/env python3
"""Throughput of the hybrid compressed-attention hot path on one MI355X.

One step = one pass of the whole path over one batch: for each layer, pool the
blocks the new token completes, score + top-k with the lightning indexer (CSA),
and attend with one softmax over the entries, the window and the sink.

Primary workload (``value``): the ragged interleaved CSA+HCA decode layer pair -
32 sequences with seeded log-uniform context lengths in [4096, 1048576], 64 query
heads, D = 512 (448 FP8 + 64 BF16 RoPE), FP8 indexer 64x128, top-512, window 128.
``value`` is decoded tokens per second (one token per sequence per step through
both layers).  Secondary fields of the same line: CSA decode at 128K (8 x 131072),
HCA decode at 1M (4 x 1048576) and the MXFP4 prefill indexer of a 4096-token chunk
after a 1M prefix (TFLOP/s of the scoring kernel).

Inputs are seeded synthetic data shaped like those workloads, resident in HBM
before timing; each workload is replicated until the replicas exceed 1 GiB and the
steps rotate through them, so the 256 MiB last-level cache cannot serve them.
``roofline`` reports the dominant kernel (the CSA indexer scoring launch, which also
carries the step's pooling) against
the 8 TB/s HBM peak, timed by HIP events recorded around it on its own stream.
``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of the primary
workload on this machine's host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attn tokens/s and HBM GB/s at 1M ctx (CSA+HCA); prefill indexer TFLOPs"
HBM_PEAK_GBPS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
FP4_PEAK_TFLOPS = 10100.0
ENTRY_BYTES = 448 + 128 + 4          # FP8 nope + BF16 rope + f32 scale
TOKEN_BYTES = 512 * 2                # raw BF16 window token
KEY_BYTES = 128                      # FP8 indexer key
KEY_BYTES_FP4 = 64 + 4               # MXFP4 indexer key: 128 E2M1 codes + 4 E8M0 block scales
QO_BYTES = 2 * 64 * 512 * 2          # BF16 q and o
QI_W_BYTES = 64 * 128 + 64 * 4       # FP8 indexer query + f32 head weights
QI_W_BYTES_FP4 = 64 * KEY_BYTES_FP4 + 64 * 4   # MXFP4 indexer query + f32 head weights


# ---------------------------------------------------------------- byte models
def csa_bytes(lengths, k=512, n_win=128, key_bytes=KEY_BYTES, qiw_bytes=QI_W_BYTES):
    """Algorithmic HBM bytes of one CSA decode step (query at t = L - 1), each
    byte once: indexer keys of the visible entries, the k gathered entries, the
    window tokens, q/o, q_I/w, and the pooled entry + key (write) plus the raw
    indexer-key tokens it reads when the new token completes a block."""
    total = 0
    keys = 0
    for L in lengths:
        V = L // 4
        keys += V * key_bytes + qiw_bytes
        total += V * key_bytes + qiw_bytes + min(k, V) * ENTRY_BYTES
        total += min(n_win, L) * TOKEN_BYTES + QO_BYTES
        if L % 4 == 0:
            total += ENTRY_BYTES + key_bytes + 4 * 128 * 2
    return total, keys


def hca_bytes(lengths, n_win=128):
    total = 0
    ent = 0
    for L in lengths:
        V = L // 128
        ent += V * ENTRY_BYTES
        total += V * ENTRY_BYTES + min(n_win, L) * TOKEN_BYTES + QO_BYTES
        if L % 128 == 0:
            total += ENTRY_BYTES
    return total, ent


def prefill_indexer_flops(prefix, T, H_I=64, d_I=128):
    t = prefix + np.arange(T, dtype=np.int64)
    pairs = int(((t + 1) // 4).sum())
    return pairs * H_I * d_I * 2, pairs


# ------------------------------------------------ committed counter evidence
def committed_traffic(summary="profiles/hbm_counters.ragged_pair_32.md"):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None when a source the kernel is compiled
    from has changed since those counters were taken (or no summary exists).  The
    summary lists its sources as ``kernel_source`` / ``kernel_source_sha256`` pairs
    (comma-separated, in the same order)."""
    import hashlib
    try:
        text = open(os.path.join(ROOT, summary)).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        k, _, v = line.strip().partition(": ")
        if k in ("kernel_source", "kernel_source_sha256", "traffic_bytes_per_launch"):
            fields[k] = v.strip()
    try:
        srcs = [x.strip() for x in fields["kernel_source"].split(",")]
        shas = [x.strip() for x in fields["kernel_source_sha256"].split(",")]
        if len(srcs) != len(shas):
            return None
        for src, sha in zip(srcs, shas):
            if hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest() != sha:
                return None
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


# ------------------------------------------------------- rocprofv3 summaries
def rocprof_summary(path):
    """Markdown table of a rocprofv3 CSV: a ``*_kernel_stats.csv`` (--kernel-trace
    --stats) gives calls and durations per kernel; a ``*_counter_collection.csv``
    (--pmc) gives each counter's mean per dispatch, per kernel."""
    import csv
    from collections import defaultdict
    rows = list(csv.DictReader(open(path)))
    lines = []
    if path.endswith("kernel_stats.csv"):
        tot = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
        lines += ["| kernel | calls | avg us | min us | max us | share |", "|---|---:|---:|---:|---:|---:|"]
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
            lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{100 * float(r['TotalDurationNs']) / tot:.1f}% |")
    elif path.endswith("counter_collection.csv"):
        val = defaultdict(lambda: defaultdict(float))
        disp = defaultdict(set)
        counters = []
        for r in rows:
            k, c = r["Kernel_Name"], r["Counter_Name"]
            val[k][c] += float(r["Counter_Value"])
            disp[k].add(r["Dispatch_Id"])
            if c not in counters:
                counters.append(c)
        lines += ["| kernel | dispatches | " + " | ".join(counters) + " |",
                  "|---|---:|" + "---:|" * len(counters)]
        for k, v in val.items():
            n = len(disp[k])
            lines.append(f"| `{k}` | {n} | " + " | ".join(f"{v[c] / n:,.0f}" for c in counters) + " |")
    else:
        raise SystemExit(f"{path}: expected a rocprofv3 *_kernel_stats.csv or *_counter_collection.csv")
    return "\n".join(lines)


# ---------------------------------------------------------------- GPU timing
PROF_EVERY = 8     # steps of the timed region whose profiled kernel gets its own event pair


class Timed:
    """K timed steps rotating over the replica sets.  The profiled kernel (the scoring
    kernel, or attention) is bracketed by HIP events on every PROF_EVERY-th timed step
    only: each event pair adds queue packets that cost the step several microseconds,
    so bracketing every step would time the instrumentation along with the path."""

    def __init__(self, name, layer_sets, prefill=False):
        self.name, self.sets, self.prefill = name, layer_sets, prefill

    def run(self, steps, warmup, prof_layer=0, prof_kind="select"):
        import torch
        R = len(self.sets)
        for i in range(warmup):
            for lay in self.sets[i % R]:
                lay.step(prefill=self.prefill)
        sampled = list(range(0, steps, PROF_EVERY))
        evs = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in sampled}
        for a, b in evs.values():  # create the handles before passing them to the library
            a.record()
            b.record()
        # step-time distribution: an event between consecutive blocks of `block` steps
        block = max(1, steps // 20)
        marks = [torch.cuda.Event(enable_timing=True) for _ in range((steps + block - 1) // block + 1)]
        torch.cuda.synchronize()
        marks[0].record()
        for i in range(steps):
            for li, lay in enumerate(self.sets[i % R]):
                p = evs.get(i) if li == prof_layer else None
                lay.step(prefill=self.prefill, prof_select=p if prof_kind == "select" else None,
                         prof_attend=p if prof_kind == "attend" else None)
            if (i + 1) % block == 0 or i + 1 == steps:
                marks[(i + block) // block].record()
        torch.cuda.synchronize()
        total_ms = marks[0].elapsed_time(marks[-1])
        per = [marks[j].elapsed_time(marks[j + 1]) / min(block, steps - j * block) for j in range(len(marks) - 1)]
        self.dist = {"median": round(float(np.median(per)), 4), "p10": round(float(np.percentile(per, 10)), 4),
                     "p90": round(float(np.percentile(per, 90)), 4), "block_steps": block, "blocks": len(per)}
        kern_ms = np.array([a.elapsed_time(b) for a, b in evs.values()])
        return total_ms / steps, kern_ms


def replicate(layers, step_bytes, min_total=1 << 30, cap=64):
    reps = max(2, min(cap, math.ceil(min_total / max(step_bytes, 1))))
    sets = [layers]
    for _ in range(reps - 1):
        sets.append([l.clone() for l in layers])
    return sets


def device_layers(w, page_rows=None, split_chunks=None):
    """Resident device layers; ``page_rows`` = {"csa": rows, "hca": rows} lays each
    layer's compressed cache out in shuffled pages of that many entries;
    ``split_chunks`` = {"csa": n, "hca": n} selects the batch-invariant fixed split."""
    from long_context_attention_softmax_amd.layer import DeviceLayer
    out = []
    for l in w.layers:
        d = DeviceLayer.from_host(l, w.g, page_rows=(page_rows or {}).get(l.mode))
        d.split_chunks = (split_chunks or {}).get(l.mode, 0)
        out.append(d)
    return out


# ---------------------------------------------------------------- CPU baseline
def cpu_baseline(w, sample_every=1, repeats=5):
    """The fp64 oracle on every ``sample_every``-th sequence of the workload, both
    layers, full step (pooling, scores, top-k, attention); median of ``repeats`` runs."""
    from oracle import step as ostep
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    sel = np.arange(0, w.B, sample_every)
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        for lay in w.layers:
            qs = np.flatnonzero(np.isin(lay.seq_id, sel))
            ostep.run_layer(lay, w.g, queries=qs)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": round(len(sel) / t, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(sel)} of {w.B} sequences (every {sample_every}th; lengths "
                      f"{[int(x) for x in w.lengths[sel]]}), both layers, full step, median of {repeats} "
                      f"({t:.2f} s per pass)"}


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-secondary", action="store_true", help="time the primary workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="copy a 1 GiB buffer a few times (reference for HBM byte counters) and exit")
    ap.add_argument("--rocprof-summary", nargs="+", metavar="CSV",
                    help="print markdown tables of rocprofv3 CSV output (kernel stats or counters) and exit")
    ap.add_argument("--only", default=None, help="debug: run one workload (ragged|csa|ragged4|paged|invariant|prologue|outproj|hca|prefill)")
    args = ap.parse_args()
    if args.rocprof_summary:
        for path in args.rocprof_summary:
            print(f"{os.path.basename(path)}:\n\n{rocprof_summary(path)}\n")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(sequences are independent, so more GPUs shard the batch with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from synth.configs import config_by_name
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 4}), flush=True)
        return

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    out = {}
    secondary = {}
    only = args.only

    # ---- primary: ragged CSA+HCA layer pair ---------------------------------
    if only in (None, "ragged"):
        cfg = config_by_name("ragged_pair_32")
        t0 = time.time()
        w5 = synth.make(cfg)
        L = [int(x) for x in w5.lengths]
        cb, ckeys = csa_bytes(L)
        hb, _ = hca_bytes(L)
        log(f"[bench] ragged pair: generated in {time.time() - t0:.1f}s, {cb / 1e6:.1f} + {hb / 1e6:.1f} MB/step")
        sets = replicate(device_layers(w5), cb + hb)
        log(f"[bench] ragged pair: {len(sets)} replicas resident")
        tm = Timed("ragged", sets)
        ms, kern = tm.run(args.steps, args.warmup, prof_layer=0, prof_kind="select")
        kern_avg = float(kern.mean())
        step_bytes = cb + hb
        out.update(dict(
            value=round(w5.B / (ms * 1e-3), 1), unit="tokens/s", ms_per_step=round(ms, 4),
            step_ms=tm.dist,
            hbm_gbps=round(step_bytes / (ms * 1e-3) / 1e9, 1), bytes_per_step=step_bytes,
            config={"workload": "ragged_pair_32", "batch": w5.B, "context_lengths": L,
                    "layers": "CSA (m=4, FP8 indexer 64x128, top-512) + HCA (m=128)",
                    "heads": 64, "head_dim": 512, "window": 128, "replicas": len(sets)},
            roofline={"bound": "hbm",
                      "kernel": "score_pool_kernel<FP8> (CSA indexer scoring; the step's pooling rides in it)",
                      "achieved": round(ckeys / (kern_avg * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                      "unit": "GB/s", "frac": round(ckeys / (kern_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                      "traffic": committed_traffic(), "algorithmic_bytes_per_launch": ckeys,
                      "avg_launch_ms": round(kern_avg, 5)}))
        log(f"[bench] ragged pair: {ms:.4f} ms/step, scoring kernel {kern_avg:.4f} ms")
        del sets
        torch.cuda.empty_cache()

    if not args.no_secondary or only:
        # ---- CSA decode at 128K --------------------------------------------
        if only in (None, "csa"):
            w2 = synth.make("csa_decode_128k")
            L2 = [int(x) for x in w2.lengths]
            cb2, ck2 = csa_bytes(L2)
            sets = replicate(device_layers(w2), cb2)
            tm_csa = Timed("csa", sets)
            ms2, k2 = tm_csa.run(args.steps, args.warmup, prof_kind="select")
            secondary["csa_decode_128k"] = dict(
                tokens_per_s=round(w2.B / (ms2 * 1e-3), 1), ms_per_step=round(ms2, 4),
                hbm_gbps=round(cb2 / (ms2 * 1e-3) / 1e9, 1),
                hbm_frac=round(cb2 / (ms2 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), bytes_per_step=cb2,
                scoring_kernel_ms=round(float(k2.mean()), 5),
                scoring_kernel_gbps=round(ck2 / (float(k2.mean()) * 1e-3) / 1e9, 1), replicas=len(sets),
                step_ms=tm_csa.dist)
            log(f"[bench] csa 128k: {ms2:.4f} ms/step")
            del sets
            torch.cuda.empty_cache()
        # ---- ragged pair with the FP4 (MXFP4) indexer the pages describe -----
        if only in (None, "ragged4"):
            w6 = synth.make("ragged_pair_32", idx_fmt="mxfp4")
            L6 = [int(x) for x in w6.lengths]
            cb6, ck6 = csa_bytes(L6, key_bytes=KEY_BYTES_FP4, qiw_bytes=QI_W_BYTES_FP4)
            hb6, _ = hca_bytes(L6)
            sets = replicate(device_layers(w6), cb6 + hb6)
            ms6, k6 = Timed("ragged4", sets).run(args.steps, args.warmup, prof_layer=0, prof_kind="select")
            k6m = float(k6.mean())
            secondary["ragged_pair_32_mxfp4_indexer"] = dict(
                tokens_per_s=round(w6.B / (ms6 * 1e-3), 1), ms_per_step=round(ms6, 4),
                hbm_gbps=round((cb6 + hb6) / (ms6 * 1e-3) / 1e9, 1), bytes_per_step=cb6 + hb6,
                scoring_kernel_ms=round(k6m, 5), scoring_key_bytes=ck6,
                scoring_kernel_gbps=round(ck6 / (k6m * 1e-3) / 1e9, 1),
                scoring_hbm_frac=round(ck6 / (k6m * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), replicas=len(sets))
            log(f"[bench] ragged pair (MXFP4 indexer): {ms6:.4f} ms/step, scoring kernel {k6m:.4f} ms")
            del sets
            torch.cuda.empty_cache()
        # ---- ragged pair over a paged cache (block tables, shuffled pages) ---
        if only in (None, "paged"):
            w7 = synth.make("ragged_pair_32")
            L7 = [int(x) for x in w7.lengths]
            cb7, ck7 = csa_bytes(L7)
            hb7, _ = hca_bytes(L7)
            pages = {"csa": 256, "hca": 16}
            sets = replicate(device_layers(w7, pages), cb7 + hb7)
            ms7, k7 = Timed("paged", sets).run(args.steps, args.warmup, prof_layer=0, prof_kind="select")
            k7m = float(k7.mean())
            secondary["ragged_pair_32_paged"] = dict(
                tokens_per_s=round(w7.B / (ms7 * 1e-3), 1), ms_per_step=round(ms7, 4),
                hbm_gbps=round((cb7 + hb7) / (ms7 * 1e-3) / 1e9, 1), bytes_per_step=cb7 + hb7,
                page_rows=pages, scoring_kernel_ms=round(k7m, 5),
                scoring_kernel_gbps=round(ck7 / (k7m * 1e-3) / 1e9, 1), replicas=len(sets))
            log(f"[bench] ragged pair (paged cache): {ms7:.4f} ms/step, scoring kernel {k7m:.4f} ms")
            del sets
            torch.cuda.empty_cache()
        # ---- ragged pair, batch-invariant decode (fixed split) ---------------
        if only in (None, "invariant"):
            w8 = synth.make("ragged_pair_32")
            L8 = [int(x) for x in w8.lengths]
            cb8, _ = csa_bytes(L8)
            hb8, _ = hca_bytes(L8)
            split = {"csa": 2, "hca": 3}
            sets = replicate(device_layers(w8, split_chunks=split), cb8 + hb8)
            ms8, k8 = Timed("invariant", sets).run(args.steps, args.warmup, prof_layer=1, prof_kind="attend")
            secondary["ragged_pair_32_batch_invariant"] = dict(
                tokens_per_s=round(w8.B / (ms8 * 1e-3), 1), ms_per_step=round(ms8, 4),
                hbm_gbps=round((cb8 + hb8) / (ms8 * 1e-3) / 1e9, 1), bytes_per_step=cb8 + hb8,
                split_chunks=split, hca_attention_kernel_ms=round(float(k8.mean()), 5), replicas=len(sets))
            log(f"[bench] ragged pair (batch-invariant split): {ms8:.4f} ms/step")
            del sets
            torch.cuda.empty_cache()
        # ---- q / KV normalization prologue at the prefill chunk's size --------
        if only in (None, "prologue"):
            from long_context_attention_softmax_amd.ops import hca_qkv_prologue
            T, H, D, W = 4096, 64, 512, 4352
            gen = torch.Generator(device="cuda").manual_seed(9)
            q = torch.randn((T, H, D), generator=gen, device="cuda").to(torch.bfloat16)
            kv = torch.randn((T, D), generator=gen, device="cuda").to(torch.bfloat16)
            ring = torch.zeros((1, W, D), dtype=torch.bfloat16, device="cuda")
            gq = torch.rand(D, generator=gen, device="cuda") + 0.5
            gk = torch.rand(D, generator=gen, device="cuda") + 0.5
            seq = torch.zeros(T, dtype=torch.int32, device="cuda")
            pos = torch.arange(1 << 20, (1 << 20) + T, dtype=torch.int64, device="cuda")
            qo = torch.empty_like(q)
            pbytes = 2 * (T * H * D * 2) + 2 * (T * D * 2)             # q and tokens, read and written

            def run():
                hca_qkv_prologue(q, gq, kv, gk, seq, pos, ring, q_out=qo)
            for _ in range(args.warmup):
                run()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
            for a, b in ev:
                a.record()
                run()
                b.record()
            torch.cuda.synchronize()
            pm = float(np.mean([a.elapsed_time(b) for a, b in ev]))
            secondary["qkv_prologue_4096x64"] = dict(
                kernel_ms=round(pm, 5), bytes=pbytes, gbps=round(pbytes / (pm * 1e-3) / 1e9, 1),
                hbm_frac=round(pbytes / (pm * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                config={"queries": T, "heads": H, "D": D, "tokens": T, "io": "bf16"})
            log(f"[bench] qkv prologue 4096 x 64 heads: {pm:.4f} ms, {pbytes / (pm * 1e-3) / 1e9:.0f} GB/s")
            del q, kv, ring, qo
            torch.cuda.empty_cache()
        # ---- grouped output projection (64 heads x 512 -> 8 groups x 1024) ----
        if only in (None, "outproj"):
            from long_context_attention_softmax_amd.ops import hca_out_proj
            Hh, Dd, Gg, dg = 64, 512, 8, 1024
            Kg = Hh // Gg * Dd
            gen = torch.Generator(device="cuda").manual_seed(11)
            wts = [(torch.randn((Gg, dg, Kg), generator=gen, device="cuda") * Kg ** -0.5).to(torch.bfloat16)
                   for _ in range(4)]                                  # rotated so the cache never holds them
            res = {}
            for Nq in (32, 4096):
                o = (torch.randn((Nq, Hh, Dd), generator=gen, device="cuda") * 0.05).to(torch.bfloat16)
                y = torch.empty((Nq, Gg, dg), dtype=torch.float32, device="cuda")
                for i in range(args.warmup):
                    hca_out_proj(o, wts[i % 4], G=Gg, y=y)
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(args.steps)]
                for i, (a, b) in enumerate(ev):
                    a.record()
                    hca_out_proj(o, wts[i % 4], G=Gg, y=y)
                    b.record()
                torch.cuda.synchronize()
                pm = float(np.mean([a.elapsed_time(b) for a, b in ev]))
                wbytes = Gg * dg * Kg * 2
                flops = 2.0 * Nq * Gg * dg * Kg
                res[Nq] = pm
                key = "decode_32" if Nq == 32 else "prefill_4096"
                secondary[f"out_proj_{key}"] = dict(
                    kernel_ms=round(pm, 5), weight_bytes=wbytes,
                    gbps=round((wbytes + Nq * Hh * Dd * 2 + Nq * Gg * dg * 4) / (pm * 1e-3) / 1e9, 1),
                    tflops=round(flops / (pm * 1e-3) / 1e12, 1),
                    config={"rows": Nq, "heads": Hh, "D": Dd, "groups": Gg, "d_g": dg, "out": "f32"})
                del o, y
            log(f"[bench] out proj: decode {res[32]:.4f} ms, prefill {res[4096]:.4f} ms")
            del wts
            torch.cuda.empty_cache()
        # ---- HCA decode at 1M ----------------------------------------------
        if only in (None, "hca"):
            w3 = synth.make("hca_decode_1m")
            L3 = [int(x) for x in w3.lengths]
            hb3, _ = hca_bytes(L3)
            sets = replicate(device_layers(w3), hb3)
            tm_hca = Timed("hca", sets)
            ms3, k3 = tm_hca.run(args.steps, args.warmup, prof_kind="attend")
            secondary["hca_decode_1m"] = dict(
                tokens_per_s=round(w3.B / (ms3 * 1e-3), 1), ms_per_step=round(ms3, 4),
                hbm_gbps=round(hb3 / (ms3 * 1e-3) / 1e9, 1),
                hbm_frac=round(hb3 / (ms3 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), bytes_per_step=hb3,
                attention_kernel_ms=round(float(k3.mean()), 5), replicas=len(sets), step_ms=tm_hca.dist)
            log(f"[bench] hca 1m: {ms3:.4f} ms/step")
            del sets
            torch.cuda.empty_cache()
        # ---- prefill indexer (MXFP4) -----------------------------------------
        if only in (None, "prefill"):
            w4 = synth.make("csa_prefill_1m")
            flops, pairs = prefill_indexer_flops(w4.prefix, w4.T)
            lays = device_layers(w4)
            csa4 = lays[0]
            steps4 = max(3, min(10, args.steps // 10))
            for _ in range(2):                # warm-up: every kernel of the chunk loaded and run once
                for lay in lays:
                    lay.pool()
                csa4.select()
                csa4.attend(prefill=True)
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            s0.record()
            for i in range(steps4):
                for lay in lays:
                    lay.pool()
                csa4.select()
                csa4.attend(prefill=True)
            s1.record()
            torch.cuda.synchronize()
            chunk_ms = s0.elapsed_time(s1) / steps4
            from long_context_attention_softmax_amd import _abi as A, ops
            idx_ws = max(v.numel() for key, v in ops._WS.items() if key[0] == A.OP_INDEXER_TOPK)
            # the scoring kernel alone: the library scores many queries in groups (its
            # workspace holds two), so the chunk's queries are passed here in groups
            # of the same size, with events around each group's scoring kernel
            G = ops.hca_indexer_query_group(csa4.Nq, csa4.max_visible, csa4.qI.fmt, csa4.g.topk)
            groups = [slice(g0, min(g0 + G, csa4.Nq)) for g0 in range(0, csa4.Nq, G)]
            evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in groups]
                   for _ in range(steps4)]
            for e in evs:                     # create the events (torch makes them on first record)
                for a, b in e:
                    a.record()
                    b.record()
            for i in range(steps4):
                for sl, ev in zip(groups, evs[i]):
                    csa4.select(prof=ev, queries=sl)
            torch.cuda.synchronize()
            kms = float(np.mean([sum(a.elapsed_time(b) for a, b in e) for e in evs]))
            secondary["csa_prefill_1m"] = dict(
                indexer_scoring_tflops=round(flops / (kms * 1e-3) / 1e12, 1),
                indexer_scoring_ms=round(kms, 3),
                fp8_peak_frac=round(flops / (kms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                fp4_peak_frac=round(flops / (kms * 1e-3) / 1e12 / FP4_PEAK_TFLOPS, 4),
                scoring_flop=flops, visible_pairs=pairs, chunk_ms=round(chunk_ms, 3),
                chunk_tokens_per_s=round(w4.T / (chunk_ms * 1e-3), 1), indexer_workspace_bytes=idx_ws,
                scoring_groups=len(groups), scoring_group_queries=G)
            log(f"[bench] prefill: chunk {chunk_ms:.3f} ms, scoring {kms:.3f} ms")
            del lays, csa4
            torch.cuda.empty_cache()

    if only is None and not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(w5)

    line = {"metric": METRIC, "value": out.get("value"), "unit": out.get("unit", "tokens/s"),
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": out.get("ms_per_step"), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp8+bf16 (fp32 accumulate)", "data": "synthetic (seeded)",
            "config": out.get("config", {"workload": only}),
            "hbm_gbps": out.get("hbm_gbps"), "roofline": out.get("roofline"),
            "cpu_baseline": out.get("cpu_baseline"), "secondary": secondary}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
