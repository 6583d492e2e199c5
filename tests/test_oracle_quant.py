"""Pins of the oracle's storage-format codecs (CPU only).

Pinned against: the OCP format tables (tests/golden), round-trip of every code,
round-half-even at every midpoint, saturation, and PyTorch's own FP8/BF16 casts.
"""
import os

import numpy as np
import pytest
import torch

from oracle import quant

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _points(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    return rows


def test_fp8_table_points():
    for code, val in _points("fp8_e4m3fn_points.txt"):
        got = quant.fp8_decode(np.array([int(code, 16)]))[0]
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-"), code


def test_fp8_roundtrip_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(quant.fp8_encode(quant.fp8_decode(codes)), codes)


def test_fp8_midpoints_round_to_even():
    pos = quant.fp8_decode(np.arange(127))
    mids = (pos[:-1] + pos[1:]) / 2
    got = quant.fp8_encode(mids)
    lo = np.arange(126)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want)
    # just off the midpoint goes to the nearer neighbour
    eps = (pos[1:] - pos[:-1]) * 1e-6
    assert np.array_equal(quant.fp8_encode(mids - eps), lo)
    assert np.array_equal(quant.fp8_encode(mids + eps), lo + 1)
    _, fr = quant.fp8_encode(mids, return_fragile=True)
    assert fr.all()


def test_fp8_saturates():
    assert list(quant.fp8_encode(np.array([449.0, 464.0, 500.0, 1e30, -1e30]))) == \
        [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_fp8_matches_torch_cast():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1, 30, 150)])
    x = np.clip(x, -460, 460).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(quant.fp8_encode(x.astype(np.float64)), want)


def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-30, 30, 100000))).astype(np.float32)
    # plant exact ties: low 16 bits = 0x8000
    t = (rng.integers(0, 2 ** 31, 2000, dtype=np.uint32) & 0xFFFF0000) | 0x8000
    x = np.concatenate([x, t.view(np.float32)])
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(quant.bf16_encode(x.astype(np.float64)), want)
    assert np.array_equal(quant.bf16_decode(want), torch.from_numpy(want.view(np.int16))
                          .view(torch.bfloat16).float().numpy().astype(np.float64))


def test_e2m1_and_e8m0_points():
    for kind, code, val in _points("mxfp4_points.txt"):
        c = np.array([int(code, 16)])
        got = (quant.e2m1_decode(c) if kind == "e2m1" else quant.e8m0_decode(c))[0]
        assert got == float(val) and np.signbit(got) == val.startswith("-"), (kind, code)


@pytest.mark.parametrize("v,want", [(0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0),
                                    (2.5, 2.0), (3.5, 4.0), (5.0, 4.0), (7.0, 6.0),
                                    (0.26, 0.5), (5.01, 6.0)])
def test_e2m1_rounding(v, want):
    # block with amax 4 -> shared exponent floor(log2 4) - 2 = 0, scale 1
    x = np.zeros(32)
    x[0] = 4.0
    x[1] = v
    x[2] = -v
    packed, scales = quant.mxfp4_encode(x)
    assert scales[0] == 127
    vals = quant.mxfp4_decode(packed, scales)
    assert vals[1] == want and vals[2] == -want


def test_mxfp4_scale_rule():
    x = np.zeros((4, 32))
    x[0, 5] = 1.0      # floor(log2 1) - 2 = -2
    x[1, 7] = -6.0     # 2 - 2 = 0
    x[2, 0] = 0.09     # floor(log2 .09) = -4 -> -6
    _, s = quant.mxfp4_encode(x)
    assert list(s[:, 0]) == [125, 127, 121, 0]          # all-zero block -> byte 0
    packed, s = quant.mxfp4_encode(x)
    v = quant.mxfp4_decode(packed, s)
    assert v[0, 5] == 1.0 and v[1, 7] == -6.0 and v[3].max() == 0


def test_mxfp4_roundtrip_codes():
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 16, (500, 64)).astype(np.uint8)
    codes[:, 0] = 7                      # amax code 6 keeps the shared exponent
    codes[:, 32] = 6 | 8                 # amax code -4 in the second block
    scales = rng.integers(100, 140, (500, 2)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    v = quant.mxfp4_decode(packed, scales)
    p2, s2 = quant.mxfp4_encode(v)
    assert np.array_equal(s2, scales)
    # -0 codes may come back as +0 (value equality is what counts)
    assert np.array_equal(quant.mxfp4_decode(p2, s2), v)


def test_entry_scale_rule():
    nope = np.zeros((5, 8))
    nope[0, 0] = 448.0
    nope[1, 3] = -449.0
    nope[2, 1] = 224.0
    nope[3, 2] = 1.0
    s, fr = quant.entry_scale(nope)
    assert list(s) == [1.0, 2.0, 0.5, 2.0 ** -8, 1.0]
    assert fr[0] and fr[2] and not fr[1]
