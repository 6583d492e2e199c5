"""Storage formats of the compressed cache (oracle side).

"DeepSeek V4: How They Crushed the Million-Token Memory Problem"
(sameershanbhag.com), "Two kinds of memory instead of one": most KV entries are
stored in FP8, the indexer in FP4 and the RoPE dimensions in BF16.  The pages do
not name the exact encodings; this oracle reads them as

  * FP8  = OCP 8-bit float E4M3FN (bias 7, no infinities, max 448, NaN = S.1111.111),
    round to nearest, ties to even, saturating at +-448;
  * BF16 = IEEE binary32 truncated to 8 significant bits, round to nearest even;
  * FP4  = OCP Microscaling MXFP4: E2M1 elements {0, .5, 1, 1.5, 2, 3, 4, 6} with one
    E8M0 power-of-two scale per 32 elements, scale exponent floor(log2 amax) - 2,
    elements rounded to nearest even and saturated at +-6; an all-zero block gets
    the smallest scale (byte 0).

Encoders take fp64 values and round once.  Rounding is written as "scale the
value by its binade's spacing, round to the nearest integer with ties to even
(numpy ``rint``), scale back" - a different formulation from the bit manipulation
used on the device.  Each encoder can also report *fragile* elements whose exact
value lies within a relative 1e-12 of a rounding boundary, where a different
(fp64-rounding-order) evaluation may legitimately land on the other neighbour.
"""
from __future__ import annotations

import numpy as np

FRAGILE_REL = 1e-12


# ------------------------------------------------------------------- FP8 E4M3FN
def fp8_decode(codes: np.ndarray) -> np.ndarray:
    """Exact value of each E4M3FN code (fp64); NaN for S.1111.111."""
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    mt = c & 7
    mag = np.where(e == 0, mt * 2.0 ** -9, (8 + mt) * np.exp2(e.astype(np.float64) - 10))
    mag = np.where((e == 15) & (mt == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


_FP8_POS = fp8_decode(np.arange(127))          # codes 0x00..0x7E, ascending values


def _rne_to_grid(a: np.ndarray, lo_binade: int, mant_bits: int):
    """Round non-negative ``a`` to a float grid with ``mant_bits`` fraction bits whose
    smallest normal binade is 2^lo_binade (subnormal spacing below it).
    Returns (rounded value, fragile mask)."""
    a = np.asarray(a, np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # log2 can be off by one ulp at exact powers of two; fix the binade exactly
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    e = np.maximum(e, lo_binade)
    ulp = np.exp2(e - mant_bits)
    q = a / ulp
    r = np.rint(q) * ulp
    frac = q - np.floor(q)
    fragile = np.abs(frac - 0.5) < FRAGILE_REL * np.maximum(q, 1.0)
    return r, fragile


def fp8_round(x: np.ndarray):
    """Nearest E4M3FN value (ties to even, saturating).  Returns (values, fragile)."""
    x = np.asarray(x, np.float64)
    r, fragile = _rne_to_grid(np.abs(x), -6, 3)
    r = np.minimum(r, 448.0)
    return np.copysign(r, x), fragile


def fp8_encode(x: np.ndarray, return_fragile: bool = False):
    """E4M3FN codes of ``x`` (RNE, saturating); the sign bit follows ``x``'s sign."""
    x = np.asarray(x, np.float64)
    v, fragile = fp8_round(x)
    mag_code = np.searchsorted(_FP8_POS, np.abs(v)).astype(np.uint8)
    assert np.all(_FP8_POS[mag_code] == np.abs(v))
    code = mag_code | (np.signbit(x).astype(np.uint8) << 7)
    return (code, fragile) if return_fragile else code


# ------------------------------------------------------------------------- BF16
def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """Value (fp64) of BF16 bit patterns."""
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_round(x: np.ndarray):
    """Nearest BF16 value of fp64 ``x`` (ties to even).  Returns (values, fragile)."""
    x = np.asarray(x, np.float64)
    r, fragile = _rne_to_grid(np.abs(x), -126, 7)
    return np.copysign(r, x), fragile


def bf16_encode(x: np.ndarray, return_fragile: bool = False):
    v, fragile = bf16_round(x)
    bits = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.all(bf16_decode(bits) == v)
    return (bits, fragile) if return_fragile else bits


def f32_round(x: np.ndarray):
    """Nearest binary32 value (ties to even).  Returns (values, fragile)."""
    x = np.asarray(x, np.float64)
    r, fragile = _rne_to_grid(np.abs(x), -126, 23)
    return np.copysign(r, x), fragile


# ------------------------------------------------------------------------ MXFP4
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_VALUES[c & 7]
    return np.where(c & 8, -mag, mag)


def e8m0_decode(b: np.ndarray) -> np.ndarray:
    return np.exp2(np.asarray(b).astype(np.float64) - 127.0)


def mxfp4_unpack(packed: np.ndarray) -> np.ndarray:
    """[..., d/2] bytes -> [..., d] codes; element 2i in the low nibble of byte i."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def mxfp4_decode(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Values [..., d] of packed codes [..., d/2] with E8M0 scales [..., d/32]."""
    v = e2m1_decode(mxfp4_unpack(packed))
    s = e8m0_decode(scales)
    return v * np.repeat(s, 32, axis=-1)


def mxfp4_encode(x: np.ndarray, return_fragile: bool = False):
    """OCP MX v1.0 MXFP4 encode of fp64 ``x`` [..., d] (d multiple of 32).

    Per 32-element block: shared exponent floor(log2 amax) - 2, clamped to the E8M0
    range; elements x / 2^exponent rounded to E2M1 (ties to even), saturating at 6.
    """
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    assert d % 32 == 0
    blk = x.reshape(x.shape[:-1] + (d // 32, 32))
    amax = np.max(np.abs(blk), axis=-1)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    e = np.where(np.exp2(e) > amax, e - 1, e)
    e = np.where(np.exp2(e + 1) <= amax, e + 1, e)
    # an exact power of two is a boundary of the scale decision
    scale_fragile = (amax > 0) & (np.abs(amax / np.exp2(e) - 1.0) < FRAGILE_REL)
    sexp = np.clip(e - 2, -127, 127)
    sexp = np.where(amax > 0, sexp, -127)
    scales = (sexp + 127).astype(np.uint8)
    v = blk / np.exp2(sexp)[..., None]
    a = np.abs(v)
    r, fragile = _rne_to_grid(a, 0, 1)
    r = np.minimum(r, 6.0)
    mag_code = np.searchsorted(E2M1_VALUES, r).astype(np.uint8)
    assert np.all(E2M1_VALUES[mag_code] == r)
    code = (mag_code | (np.signbit(v).astype(np.uint8) << 3)).reshape(x.shape)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    fragile = fragile.reshape(x.shape) | np.repeat(scale_fragile, 32, axis=-1)
    return (packed, scales, fragile) if return_fragile else (packed, scales)


# --------------------------------------------------------------- entry planes
def entry_scale(nope: np.ndarray):
    """Per-entry power-of-two scale of the FP8 nope plane: the smallest 2^e with
    amax <= 448 * 2^e (1 when the entry is all zero).  Returns (scale, fragile)."""
    a = np.max(np.abs(np.asarray(nope, np.float64)), axis=-1)
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(np.where(a > 0, a / 448.0, 1.0)))
    e = np.where(448.0 * np.exp2(e) < a, e + 1, e)
    e = np.where(448.0 * np.exp2(e - 1) >= a, e - 1, e)
    e = np.where(a > 0, e, 0)
    fragile = (a > 0) & (np.abs(a / (448.0 * np.exp2(e)) - 1.0) < FRAGILE_REL)
    return np.exp2(e), fragile
