"""GPU parity of the grouped output projection (hca_out_proj) against
oracle/project.py on seeded BF16 inputs.  Bars: per-row relative error
max|y - ref| / max|ref| <= 1e-4 for binary32 output (exact products summed in
binary32 over K_g = 4096 terms in a fixed order: about sqrt(K_g) * 2^-24 typical,
K_g * 2^-24 = 2.4e-4 worst case) and <= 2e-2 for BF16 output (one rounding,
2^-9)."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import row_rel_err, to_np, bf16_values
from oracle import project, quant

pytestmark = pytest.mark.gpu

H, D, G = 64, 512, 8


def _print(msg):
    print(msg, flush=True)


def _inputs(seed, Nq, d_g):
    rng = np.random.default_rng(seed)
    K_g = H // G * D
    o = synth.bf16_bits(rng.normal(size=(Nq, H, D)).astype(np.float32) * np.float32(0.05))
    w = synth.bf16_bits((rng.normal(size=(G, d_g, K_g)) / np.sqrt(K_g)).astype(np.float32))
    return o, w


def _dev(bits, gpu):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(gpu).view(torch.bfloat16)


# (rows, units per group): up to 64 rows the K-split kernel; more rows with units a
# multiple of 128 the 128-wide tiled kernel, more than 128 rows with units a multiple
# of 256 the 256-wide one (ragged last row tiles included)
@pytest.mark.parametrize("Nq,d_g", [(1, 64), (5, 64), (32, 64), (33, 64), (100, 64), (65, 128), (100, 128),
                                    (300, 128), (128, 256), (129, 256), (300, 256), (600, 512)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_out_proj_parity(gpu, Nq, d_g, out):
    from long_context_attention_softmax_amd.ops import hca_out_proj
    o, w = _inputs(80 + Nq, Nq, d_g)
    ref = project.grouped_out_proj(quant.bf16_decode(o), quant.bf16_decode(w))
    _print(f"out proj Nq={Nq} G={G} d_g={d_g} out={out}")
    y = hca_out_proj(_dev(o, gpu), _dev(w, gpu), G=G,
                     out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    got = to_np(y).astype(np.float64) if out == "f32" else bf16_values(to_np(y))
    err = row_rel_err(got.reshape(Nq, -1), ref.reshape(Nq, -1))
    _print(f"  rel err {err:.2e}")
    assert err <= (1e-4 if out == "f32" else 2e-2)


def test_out_proj_full_size_sampled(gpu):
    """The prefill-chunk size (4096 rows, G = 8 groups of 1024 outputs): every row
    is computed, 66 rows (rows on both sides of the 64- and 256-row tile edges included) are
    checked against the oracle; the decode size (32 rows) in full."""
    from long_context_attention_softmax_amd.ops import hca_out_proj
    d_g = 1024
    for Nq in (32, 4096):
        o, w = _inputs(90 + Nq, Nq, d_g)
        y = hca_out_proj(_dev(o, gpu), _dev(w, gpu), G=G)
        torch.cuda.synchronize()
        rows = np.arange(Nq) if Nq <= 64 else np.unique(np.concatenate(
            [[0, 63, 64, 255, 256, Nq - 1], np.random.default_rng(9).choice(Nq, 60, replace=False)]))
        ref = project.grouped_out_proj(quant.bf16_decode(o[rows]), quant.bf16_decode(w))
        got = to_np(y)[rows].astype(np.float64)
        err = row_rel_err(got.reshape(len(rows), -1), ref.reshape(len(rows), -1))
        _print(f"out proj Nq={Nq} d_g={d_g}: {len(rows)} rows checked, rel err {err:.2e}")
        assert err <= 1e-4


def test_out_proj_no_rows(gpu):
    """Zero rows: nothing launched, the (empty) result returned."""
    from long_context_attention_softmax_amd.ops import hca_out_proj
    o = torch.zeros((0, H, D), dtype=torch.bfloat16, device=gpu)
    w = torch.zeros((G, 32, H // G * D), dtype=torch.bfloat16, device=gpu)
    y = hca_out_proj(o, w, G=G)
    torch.cuda.synchronize()
    assert y.shape == (0, G, 32)


@pytest.mark.parametrize("Nq", [8, 40])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_out_proj_short_groups(gpu, Nq, out):
    """K_g = 256 (a multiple of 256 but not of 512): the four-wave variant for one row
    block, and the two-row-block kernel for more than 32 rows."""
    from long_context_attention_softmax_amd.ops import hca_out_proj
    rng = np.random.default_rng(95 + Nq)
    Hs, Ds, Gs, d_g = 4, 256, 4, 32
    o = synth.bf16_bits(rng.normal(size=(Nq, Hs, Ds)).astype(np.float32))
    w = synth.bf16_bits((rng.normal(size=(Gs, d_g, Hs // Gs * Ds)) / 16).astype(np.float32))
    ref = project.grouped_out_proj(quant.bf16_decode(o), quant.bf16_decode(w))
    _print(f"out proj K_g=256 Nq={Nq} out={out}")
    y = hca_out_proj(_dev(o, gpu), _dev(w, gpu), G=Gs,
                     out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    got = to_np(y).astype(np.float64) if out == "f32" else bf16_values(to_np(y))
    err = row_rel_err(got.reshape(Nq, -1), ref.reshape(Nq, -1))
    assert err <= (1e-4 if out == "f32" else 2e-2), err
