"""GPU parity of a paged CSA+HCA layer pair under continuous batching.

"DeepSeek V4 infrastructure" (volanea.com), "Compression only works if the attention
path is engineered end to end": a cache format that holds up for one request can
fail under continuous, batched traffic; the path needs heterogeneous KV-cache
management and state caches for the sliding window.  Here a fixed set of sequence
slots (each with its window ring, the sliding-window state) and a pool of cache pages
per layer (CSA pages of 32 entries, HCA pages of 2: different entry kinds, different
page sizes) serve a changing batch for many decode steps:

* every step appends one token per live sequence to its ring, pools the blocks that
  token completes (opening a fresh page from the free list when the entry starts a
  page), scores and selects (CSA) and attends, all through the C ABI;
* sequences leave (their pages go back to the free list, their ring slot is freed)
  and new ones join in freed slots, on recycled pages that still hold the old
  sequence's bytes, with a prefix written into those pages.

The host keeps the logical state the oracle sees: synthesized prefix entries plus
every entry the oracle itself pooled in earlier steps (no value comes from the
GPU).  After every step: pooled codes bit-exact (fragile values +-1 code), top-k
sets exact, output per-row relative error and lse within the quantized bars.
"""
import math
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import TOL_LSE, TOL_QUANT, assert_codes_equal, bf16_values, row_rel_err, to_np
from oracle import step as ostep
from synth.gen import _bf16_normal, _fp8_entries, _fp8_normal

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


class _Layer:
    """One layer's page pool, block tables and host (logical) caches."""

    def __init__(self, mode, g, slots, page_rows, n_pages, dev, rng):
        self.mode, self.g, self.pr, self.dev = mode, g, page_rows, dev
        self.m = g.m_csa if mode == "csa" else g.m_hca
        n = n_pages * page_rows
        # the pool starts as random bytes: unreferenced rows must never be read
        self.nope = torch.from_numpy(rng.integers(0, 256, (n, g.D_n), dtype=np.uint8)).to(dev)
        self.rope = torch.from_numpy(_bf16_normal(rng, (n, g.D_r)).view(np.int16)).to(dev).view(torch.bfloat16)
        self.scale = torch.ones(n, dtype=torch.float32, device=dev)
        self.keys = (torch.from_numpy(rng.integers(0, 256, (n, g.d_I), dtype=np.uint8)).to(dev)
                     if mode == "csa" else None)
        self.pitch = 1024
        self.table = np.zeros((slots, self.pitch), np.int32)
        self.table_d = torch.zeros((slots, self.pitch), dtype=torch.int32, device=dev)
        self.free = list(rng.permutation(n_pages))
        self.pages = {}                    # slot -> list of page ids
        self.host = {}                     # slot -> dict of logical planes
        self.gate_w = (rng.standard_normal(g.D) / math.sqrt(g.D)).astype(np.float32)
        self.gate_b = (rng.standard_normal(self.m) * 0.02).astype(np.float32)
        self.sink = rng.standard_normal(g.H).astype(np.float32)
        self.opened = 0                    # pages opened by pooling during the steps

    def page_row(self, slot, j):
        return int(self.table[slot, j // self.pr]) * self.pr + j % self.pr

    def open_page(self, slot, j):
        assert j // self.pr == len(self.pages[slot])
        p = self.free.pop()
        self.pages[slot].append(p)
        self.table[slot, j // self.pr] = p
        self.table_d[slot, j // self.pr] = int(p)

    def admit(self, slot, V, rng):
        """A new sequence with V synthesized entries, on pages from the free list."""
        self.pages[slot] = []
        g = self.g
        nope, scale = _fp8_entries(rng, V, g.D_n)
        rope = _bf16_normal(rng, (V, g.D_r), 1.0)
        h = dict(nope=nope, scale=scale, rope=rope)
        if self.mode == "csa":
            h["idx"] = _fp8_normal(rng, (V, g.d_I), 1 / math.sqrt(g.d_I))
        self.host[slot] = h
        for j in range(0, V, self.pr):
            self.open_page(slot, j)
        if V:
            rows = torch.tensor([self.page_row(slot, j) for j in range(V)], device=self.dev)
            self.nope[rows] = torch.from_numpy(nope).to(self.dev)
            self.scale[rows] = torch.from_numpy(scale).to(self.dev)
            self.rope[rows] = torch.from_numpy(rope.view(np.int16)).to(self.dev).view(torch.bfloat16)
            if self.mode == "csa":
                self.keys[rows] = torch.from_numpy(h["idx"]).to(self.dev)

    def release(self, slot, rng):
        pages = self.pages.pop(slot)
        self.host.pop(slot)
        self.free.extend(rng.permutation(pages).tolist())
        self.table[slot] = 0
        self.table_d[slot] = 0


class _Batch:
    def __init__(self, g, slots, dev, seed):
        self.g, self.S, self.dev = g, slots, dev
        self.rng = np.random.default_rng(seed)
        self.W = max(g.n_win, g.m_hca)
        self.win = np.zeros((slots, self.W, g.D), np.uint16)
        self.win_idx = np.zeros((slots, self.W, g.d_I), np.uint16)
        self.win_d = torch.zeros((slots, self.W, g.D), dtype=torch.bfloat16, device=dev)
        self.win_idx_d = torch.zeros((slots, self.W, g.d_I), dtype=torch.bfloat16, device=dev)
        self.csa = _Layer("csa", g, slots, 32, 3072, dev, self.rng)
        self.hca = _Layer("hca", g, slots, 2, 1024, dev, self.rng)
        self.L = {}                        # slot -> tokens so far

    def _put_tokens(self, slot, pos):
        g = self.g
        pos = np.atleast_1d(pos)
        x = _bf16_normal(self.rng, (len(pos), g.D), 1.0)
        y = _bf16_normal(self.rng, (len(pos), g.d_I), 1 / math.sqrt(g.d_I))
        self.win[slot, pos % self.W] = x
        self.win_idx[slot, pos % self.W] = y
        idx = torch.from_numpy(pos % self.W).to(self.dev)
        self.win_d[slot, idx] = torch.from_numpy(x.view(np.int16)).to(self.dev).view(torch.bfloat16)
        self.win_idx_d[slot, idx] = torch.from_numpy(y.view(np.int16)).to(self.dev).view(torch.bfloat16)

    def admit(self, slot, L0):
        assert slot not in self.L
        self.L[slot] = L0
        for lay in (self.csa, self.hca):
            lay.admit(slot, L0 // lay.m, self.rng)
        self._put_tokens(slot, np.arange(max(0, L0 - self.W), L0))

    def release(self, slot):
        del self.L[slot]
        for lay in (self.csa, self.hca):
            lay.release(slot, self.rng)

    # ------------------------------------------------------------------ one step
    def step(self):
        g = self.g
        live = sorted(self.L)
        t = np.array([self.L[s] for s in live], np.int64)
        for s, ts in zip(live, t):
            self._put_tokens(s, ts)
            self.L[s] += 1
        q = _bf16_normal(self.rng, (len(live), g.H, g.D), 1 / math.sqrt(g.D))
        q_I = _fp8_normal(self.rng, (len(live), g.H_I, g.d_I), 1 / math.sqrt(g.d_I))
        w = self.rng.random((len(live), g.H_I), dtype=np.float32)
        errs = []
        for lay in (self.csa, self.hca):
            errs.append(self._layer_step(lay, live, t, q, q_I, w))
        return errs

    def _oracle_view(self, lay, live, t, q, q_I, w, blocks):
        """The logical layer the oracle steps: every live sequence's host cache,
        contiguous, plus an empty row for each entry pooled in this step."""
        g = self.g
        starts = np.zeros(self.S, np.int64)
        parts = {k: [] for k in lay.host[live[0]]}
        r = 0
        for s, ts in zip(live, t):
            h = lay.host[s]
            starts[s] = r
            V = (ts + 1) // lay.m
            for k in parts:
                v = h[k]
                if len(v) < V:                              # the entry this step pools
                    v = np.concatenate([v, np.zeros((1,) + v.shape[1:], v.dtype)])
                parts[k].append(v)
            r += V
        cat = {k: np.concatenate(v) for k, v in parts.items()}
        lv = SimpleNamespace(mode=lay.mode, m=lay.m, fmt="quant", B=self.S, W_cap=self.W, n_rows=r,
                             cache_row_start=starts, win=self.win, q=q, sink=lay.sink,
                             q_pos=t, seq_id=np.array(live, np.int32), gate_w=lay.gate_w,
                             gate_b=lay.gate_b, cache_nope=cat["nope"], cache_rope=cat["rope"],
                             cache_scale=cat["scale"])
        lv.pool = dict(block_row=np.array([s * self.W + (j * lay.m) % self.W for s, j in blocks], np.int64),
                       block_pos=np.array([j * lay.m for _, j in blocks], np.int64),
                       out_row=np.array([starts[s] + j for s, j in blocks], np.int64))
        if lay.mode == "csa":
            lv.idx_fmt, lv.idx_fp8, lv.q_I, lv.w, lv.win_idx = "fp8", cat["idx"], q_I, w, self.win_idx
        return lv

    def _layer_step(self, lay, live, t, q, q_I, w):
        from long_context_attention_softmax_amd import _abi as A
        from long_context_attention_softmax_amd.ops import (IdxCache, KVCache, hca_attn_decode,
                                                            hca_indexer_topk, hca_kv_compress)
        g, dev = self.g, self.dev
        # blocks completed by this step's tokens; a block starting a page opens one
        blocks = [(s, int((ts + 1) // lay.m) - 1) for s, ts in zip(live, t) if (ts + 1) % lay.m == 0]
        for s, j in blocks:
            if j % lay.pr == 0:
                lay.open_page(s, j)
                lay.opened += 1
        out_rows = np.array([lay.page_row(s, j) for s, j in blocks], np.int64)
        cache = KVCache(nope=lay.nope, rope=lay.rope, scale=lay.scale)
        keys = IdxCache(lay.keys, A.FP8_E4M3) if lay.mode == "csa" else None
        pages = (lay.table_d, lay.pr)
        if blocks:
            i64 = lambda x: torch.tensor(x, dtype=torch.int64, device=dev)       # noqa: E731
            hca_kv_compress(self.win_d, i64([s * self.W + (j * lay.m) % self.W for s, j in blocks]),
                            i64([j * lay.m for _, j in blocks]), i64(out_rows),
                            torch.from_numpy(lay.gate_w).to(dev), torch.from_numpy(lay.gate_b).to(dev), cache,
                            m=lay.m, D_r=g.D_r, rope_base=g.rope_base,
                            raw_idx=self.win_idx_d if lay.mode == "csa" else None, out_idx=keys)
        seq_id = torch.tensor(live, dtype=torch.int32, device=dev)
        q_pos = torch.from_numpy(t).to(dev)
        max_vis = int(((t + 1) // lay.m).max())
        qd = torch.from_numpy(q.view(np.int16)).to(dev).view(torch.bfloat16)
        lse = torch.empty((len(live), g.H), dtype=torch.float32, device=dev)
        idx = None
        if lay.mode == "csa":
            idx = hca_indexer_topk(IdxCache(torch.from_numpy(q_I).to(dev), A.FP8_E4M3),
                                   torch.from_numpy(w).to(dev), keys, None, seq_id, q_pos, k=g.topk, m=lay.m,
                                   max_visible=max_vis, pages=pages)
        o = hca_attn_decode(qd, cache, None, self.win_d, torch.from_numpy(lay.sink).to(dev), seq_id, q_pos,
                            mode=A.MODE_CSA if lay.mode == "csa" else A.MODE_HCA, m=lay.m, n_win=g.n_win,
                            D_r=g.D_r, max_visible=max_vis, k=g.topk if lay.mode == "csa" else 0, idx=idx,
                            tau=g.tau, rope_base=g.rope_base, lse=lse, pages=pages)
        torch.cuda.synchronize()
        # the oracle's step of the same logical state
        lv = self._oracle_view(lay, live, t, q, q_I, w, blocks)
        ref = ostep.run_layer(lv, g)
        kv = ref["pooled"]["kv"]
        if blocks:
            rows = torch.from_numpy(out_rows).to(dev)
            D_n = g.D_n
            assert np.array_equal(to_np(lay.scale[rows]), kv["scale"]), "pooled entry scales"
            assert_codes_equal(to_np(lay.nope[rows]), kv["nope"], kv["fragile"][:, :D_n], "pooled nope")
            assert_codes_equal(to_np(lay.rope[rows]), kv["rope"], kv["fragile"][:, D_n:], "pooled rope")
            if lay.mode == "csa":
                ix = ref["pooled"]["idx"]
                assert_codes_equal(to_np(lay.keys[rows]), ix["fp8"], ix["fragile"], "pooled index key")
        if lay.mode == "csa":
            assert np.array_equal(to_np(idx), ref["idx"]), "top-k sets differ"
        err = row_rel_err(bf16_values(to_np(o)), ref["o"])
        assert err <= TOL_QUANT, f"{lay.mode}: output rel err {err:.3e}"
        lse_err = float(np.abs(to_np(lse) - ref["lse"]).max())
        assert lse_err <= TOL_LSE, f"{lay.mode}: lse abs err {lse_err:.3e}"
        # the oracle's pooled entries become part of the logical state
        for i, (s, j) in enumerate(blocks):
            h = lay.host[s]
            assert len(h["nope"]) == j
            h["nope"] = np.concatenate([h["nope"], kv["nope"][i:i + 1]])
            h["scale"] = np.concatenate([h["scale"], kv["scale"][i:i + 1]])
            h["rope"] = np.concatenate([h["rope"], kv["rope"][i:i + 1]])
            if lay.mode == "csa":
                h["idx"] = np.concatenate([h["idx"], ref["pooled"]["idx"]["fp8"][i:i + 1]])
        return err, lse_err, len(blocks)


def test_continuous_batching_paged_pair(gpu):
    g = synth.FULL_GEOMETRY
    b = _Batch(g, slots=6, dev=gpu, seed=91)
    # prefix lengths just short of CSA page boundaries (32 entries = 128 tokens) and of
    # HCA blocks (128 tokens), so pooling opens pages within the first steps
    for slot, L0 in enumerate([128 * 41 - 1, 128 * 97 - 3, 128 * 13 - 6, 128 * 301 - 30, 128 * 8 - 2]):
        b.admit(slot, L0)
    schedule = {14: ("leave", 1), 15: ("join", 1, 128 * 51 - 2), 27: ("leave", 3), 28: ("leave", 4),
                29: ("join", 4, 128 * 20 - 1), 33: ("join", 5, 128 * 64 - 9), 40: ("join", 3, 4097)}
    worst = [0.0, 0.0]
    for s in range(48):
        ev = schedule.get(s)
        if ev and ev[0] == "leave":
            b.release(ev[1])
        elif ev:
            b.admit(ev[1], ev[2])
        (ec, lc, nc), (eh, lh, nh) = b.step()
        worst = [max(worst[0], ec, eh), max(worst[1], lc, lh)]
        _print(f"step {s}: live {sorted(b.L)}, pooled csa {nc} hca {nh}; rel err {ec:.2e}/{eh:.2e}, "
               f"lse err {lc:.2e}/{lh:.2e}")
    _print(f"pages opened by pooling: csa {b.csa.opened}, hca {b.hca.opened}; worst rel err {worst[0]:.2e}, "
           f"lse {worst[1]:.2e}")
    assert b.csa.opened >= 4 and b.hca.opened >= 3
