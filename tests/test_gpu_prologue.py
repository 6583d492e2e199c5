"""GPU parity of the query / key-value normalization prologue (hca_qkv_prologue)
against oracle/prologue.py: normalized codes bit-exact except where the oracle flags
a value within 1e-12 of a rounding boundary, ring rows written exactly at
(seq, pos mod W_cap) and nowhere else, the index stream copied unchanged; then a
whole decode step with the prologue in front matches the oracle step on the
oracle-normalized inputs (bars of the other parity tests)."""
import copy

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import run_and_compare, to_np
from oracle import prologue as opro

pytestmark = pytest.mark.gpu


def _print(msg):
    print(msg, flush=True)


def _bf16(x):
    return synth.bf16_bits(np.asarray(x, np.float32))


def _dev_bits(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


@pytest.mark.parametrize("fmt", ["bf16", "f32"])
def test_prologue_parity(gpu, fmt):
    from long_context_attention_softmax_amd.ops import hca_qkv_prologue
    rng = np.random.default_rng(70)
    Nq, H, D, Nt, B, W, d_I = (13, 64, 512, 9, 5, 128, 128) if fmt == "bf16" else (6, 4, 128, 7, 3, 16, 32)
    scale = rng.uniform(0.01, 30.0, size=(Nq, H, 1))               # rows far from unit scale
    q = rng.normal(size=(Nq, H, D)) * scale
    kv = rng.normal(size=(Nt, D)) * rng.uniform(0.05, 20.0, size=(Nt, 1))
    gq, gk = rng.uniform(0.5, 1.5, D).astype(np.float32), rng.uniform(0.5, 1.5, D).astype(np.float32)
    seq = np.array([0, 4, 2, 2, 1, 7, 3, -1, 4][:Nt] if fmt == "bf16" else [0, 2, 1, 5, 2, 0, 1], np.int32)
    pos = np.array([5, 900, 127, 128, 66, 3, -2, 40, 1000][:Nt] if fmt == "bf16" else [0, 17, 3, 1, 31, 9, -5],
                   np.int64)
    eps = 1e-6
    if fmt == "bf16":
        from oracle import quant
        qs, kvs = _bf16(q), _bf16(kv)                              # stored inputs
        qv, kvv = quant.bf16_decode(qs), quant.bf16_decode(kvs)
        ring0 = _bf16(rng.normal(size=(B, W, D)))
        idx = _bf16(rng.normal(size=(Nt, d_I)))
        ridx0 = _bf16(rng.normal(size=(B, W, d_I)))
        t = lambda a: _dev_bits(a, gpu)                            # noqa: E731
    else:
        qs, kvs = q.astype(np.float32), kv.astype(np.float32)
        qv, kvv = qs.astype(np.float64), kvs.astype(np.float64)
        ring0 = rng.normal(size=(B, W, D)).astype(np.float32)
        idx = rng.normal(size=(Nt, d_I)).astype(np.float32)
        ridx0 = rng.normal(size=(B, W, d_I)).astype(np.float32)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)   # noqa: E731
    want_q, fr_q = opro.encode(opro.rms_norm(qv, gq, eps), fmt)
    want_k, fr_k = opro.encode(opro.rms_norm(kvv, gk, eps), fmt)
    keep = (seq >= 0) & (seq < B)
    raw = lambda a: a.view(np.uint32) if fmt == "f32" else a      # noqa: E731
    ring_w = opro.append_ring(raw(ring0), seq[keep], pos[keep], want_k[keep])
    ridx_w = opro.append_ring(raw(ridx0), seq[keep], pos[keep], raw(idx)[keep])
    dq, dring, dridx = t(qs), t(ring0), t(ridx0)
    _print(f"prologue {fmt}: Nq={Nq} H={H} D={D} Nt={Nt} (one token out of range, negative positions)")
    hca_qkv_prologue(dq, torch.from_numpy(gq).to(gpu), t(kvs),
                     torch.from_numpy(gk).to(gpu), torch.from_numpy(seq).to(gpu), torch.from_numpy(pos).to(gpu),
                     dring, eps=eps, idx_in=t(idx), win_idx=dridx)
    torch.cuda.synchronize()
    got_q = raw(to_np(dq))
    ok = ~fr_q
    assert np.array_equal(got_q[ok], want_q[ok]), f"{int((got_q != want_q)[ok].sum())} q codes differ"
    got_r = raw(to_np(dring))
    frr = np.zeros(ring_w.shape, bool)
    for i in np.flatnonzero(keep):
        frr[seq[i], pos[i] % W] = fr_k[i]
    assert np.array_equal(got_r[~frr], ring_w[~frr]), "ring rows differ"
    assert np.array_equal(raw(to_np(dridx)), ridx_w), "index-stream ring differs"


def test_step_with_prologue(gpu):
    """Decode step of a ragged CSA+HCA pair whose queries and new tokens arrive
    un-normalized: prologue (q in place, token into the ring) then pool, select,
    attend; the oracle runs the step on its own normalized codes."""
    from long_context_attention_softmax_amd.layer import DeviceLayer
    from long_context_attention_softmax_amd.ops import hca_qkv_prologue
    from oracle import quant
    from dataclasses import replace
    w = synth.ragged_pair(seed=71, B=6, lo=1024, hi=65536, round_every4=True)
    # normalized queries have unit RMS, so the softmax scale 1/sqrt(D) that the raw
    # workload folds into q's draw goes into tau
    g = replace(w.g, tau=1.0 / np.sqrt(w.g.D))
    rng = np.random.default_rng(72)
    eps = 1e-6
    for lay in w.layers:
        B, Wc = lay.win.shape[0], lay.win.shape[1]
        raw_q = _bf16(quant.bf16_decode(lay.q) * rng.uniform(0.1, 10.0, size=(B, 1, 1)))
        raw_tok = _bf16(rng.normal(size=(B, g.D)) * rng.uniform(0.1, 10.0, size=(B, 1)))
        gq, gk = rng.uniform(0.5, 1.5, g.D).astype(np.float32), rng.uniform(0.5, 1.5, g.D).astype(np.float32)
        seq, pos = lay.seq_id.astype(np.int32), lay.q_pos.astype(np.int64)
        nq, fq = opro.encode(opro.rms_norm(quant.bf16_decode(raw_q), gq, eps), "bf16")
        nk, fk = opro.encode(opro.rms_norm(quant.bf16_decode(raw_tok), gk, eps), "bf16")
        assert not fq.any() and not fk.any()          # no rounding decision within 1e-12 of a boundary
        ref_lay = copy.copy(lay)                      # the oracle's inputs: its own normalized codes
        ref_lay.q = nq
        ref_lay.win = opro.append_ring(lay.win, seq, pos, nk)
        dev_lay = copy.copy(lay)                      # the device starts from the raw query
        dev_lay.q = raw_q
        dev = DeviceLayer.from_host(dev_lay, g)
        _print(f"step with prologue, layer={lay.mode}, lengths={w.lengths.tolist()}")
        hca_qkv_prologue(dev.q, torch.from_numpy(gq).to(gpu), _dev_bits(raw_tok, gpu), torch.from_numpy(gk).to(gpu),
                         torch.from_numpy(seq).to(gpu), torch.from_numpy(pos).to(gpu), dev.win, eps=eps)
        ref, _, err = run_and_compare(ref_lay, g, dev=dev)
        _print(f"  rel err {err:.2e}")


def test_prologue_one_part_only(gpu):
    """Only queries (no tokens), then only tokens (no queries): each part alone, the
    other's buffers untouched."""
    from long_context_attention_softmax_amd.ops import hca_qkv_prologue
    from oracle import quant
    rng = np.random.default_rng(73)
    D, H = 512, 16
    q = _bf16(rng.normal(size=(3, H, D)) * 4.0)
    gq = rng.uniform(0.5, 1.5, D).astype(np.float32)
    dq = _dev_bits(q, gpu)
    _print("prologue: queries only")
    hca_qkv_prologue(dq, torch.from_numpy(gq).to(gpu), None, None, None, None, None)
    want, fr = opro.encode(opro.rms_norm(quant.bf16_decode(q), gq, 1e-6), "bf16")
    got = to_np(dq)
    assert np.array_equal(got[~fr], want[~fr])
    tok = _bf16(rng.normal(size=(2, D)))
    ring = np.zeros((2, 4, D), np.uint16)
    dring = _dev_bits(ring, gpu)
    gk = rng.uniform(0.5, 1.5, D).astype(np.float32)
    _print("prologue: tokens only")
    hca_qkv_prologue(None, None, _dev_bits(tok, gpu), torch.from_numpy(gk).to(gpu),
                     torch.tensor([1, 0], dtype=torch.int32, device=gpu),
                     torch.tensor([6, 3], dtype=torch.int64, device=gpu), dring)
    wk, fk = opro.encode(opro.rms_norm(quant.bf16_decode(tok), gk, 1e-6), "bf16")
    ring_w = opro.append_ring(ring, np.array([1, 0]), np.array([6, 3]), wk)
    assert not fk.any() and np.array_equal(to_np(dring), ring_w)


@pytest.mark.parametrize("fmt,D", [("bf16", 1024), ("bf16", 2048), ("bf16", 4096), ("f32", 512), ("f32", 1024),
                                   ("f32", 2048)])
def test_prologue_wide_rows(gpu, fmt, D):
    """Rows of 2, 4 and 8 sixteen-byte vectors per lane (the wider kernel variants)."""
    from long_context_attention_softmax_amd.ops import hca_qkv_prologue
    from oracle import quant
    rng = np.random.default_rng(74 + D)
    Nq, H, Nt, B, W = 3, 5, 4, 2, 8
    q = rng.normal(size=(Nq, H, D)) * rng.uniform(0.1, 10.0, size=(Nq, H, 1))
    kv = rng.normal(size=(Nt, D)) * 3.0
    gq, gk = rng.uniform(0.5, 1.5, D).astype(np.float32), rng.uniform(0.5, 1.5, D).astype(np.float32)
    seq, pos = np.array([0, 1, 0, 1], np.int32), np.array([2, 9, 3, 5], np.int64)
    if fmt == "bf16":
        qs, kvs = _bf16(q), _bf16(kv)
        qv, kvv = quant.bf16_decode(qs), quant.bf16_decode(kvs)
        ring0 = np.zeros((B, W, D), np.uint16)
        t = lambda a: _dev_bits(a, gpu)                            # noqa: E731
        raw = lambda a: a                                          # noqa: E731
    else:
        qs, kvs = q.astype(np.float32), kv.astype(np.float32)
        qv, kvv = qs.astype(np.float64), kvs.astype(np.float64)
        ring0 = np.zeros((B, W, D), np.float32)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)   # noqa: E731
        raw = lambda a: a.view(np.uint32)                          # noqa: E731
    wq, fq = opro.encode(opro.rms_norm(qv, gq, 1e-6), fmt)
    wk, fk = opro.encode(opro.rms_norm(kvv, gk, 1e-6), fmt)
    dq, dring = t(qs), t(ring0)
    _print(f"prologue {fmt} D={D}")
    hca_qkv_prologue(dq, torch.from_numpy(gq).to(gpu), t(kvs), torch.from_numpy(gk).to(gpu),
                     torch.from_numpy(seq).to(gpu), torch.from_numpy(pos).to(gpu), dring)
    torch.cuda.synchronize()
    got = raw(to_np(dq))
    assert np.array_equal(got[~fq], wq[~fq])
    ring_w = opro.append_ring(raw(ring0), seq, pos, wk)
    assert not fk.any() and np.array_equal(raw(to_np(dring)), ring_w)
