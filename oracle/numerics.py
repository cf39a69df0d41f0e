"""Number formats of the latent cache, written from their definitions (oracle side).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module.

* bf16: the upper 16 bits of an IEEE-754 binary32; widening to fp64 is exact;
  narrowing float32 to bf16 rounds to nearest, ties to even.
* e4m3fn (OCP 8-bit floating point, E4M3 variant): 1 sign bit, 4 exponent bits
  with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
  m/8 * 2^-6; codes 0x7F and 0xFF are NaN; there is no infinity; the largest
  finite magnitude is 448.  The 656-byte row of vLLM PR #55543 (description,
  "656B packed row layout"; commit "per-128-block fp8 quantization reference")
  stores the latent in this format with one scale per 128 values; the
  absmax/448 scale rule fixes the OCP variant (max 448), not the fnuz variant.
* Quantisation of a 128-value block (reading of the PR's per-128-block
  quantisation, which gives no formula): a = max |x| in float32;
  s = fl32(a / 448) (IEEE division, round to nearest even);
  code_i = e4m3(fl32(x_i / s)) rounded to nearest, ties to even mantissa,
  magnitudes at or above 448 saturate to 448, sign kept (so -0.0 and negative
  values that round to zero give 0x80).  A block with a == 0 stores s = 0 and
  all codes 0x00.
* Non-finite latents (reading: the pages quantise finite values only).  A block
  holding a NaN or an infinity stores the quiet NaN scale (bits 0x7FC00000) and
  the NaN code 0x7F for all 128 values, so that every value of the block decodes
  to NaN, as the bf16 row would carry the non-finite value itself into the
  scores.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def f32_to_bf16_bits(x) -> np.ndarray:
    """bf16 bits of float32 values: round to nearest, ties to even; NaN stays NaN.

    Rounding by integer arithmetic on the binary32 pattern: adding 0x7FFF plus the
    lowest kept bit, then dropping the low 16 bits, rounds half-way cases to the even
    neighbour and carries into the exponent when the mantissa overflows (up to inf).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = np.where(nan, (u >> np.uint64(16)) | np.uint64(0x0040), r)
    return r.astype(np.uint16)


def _e4m3_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# Value of every code, index = code.
E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
# Non-negative finite values, codes 0x00..0x7E, strictly increasing with the code.
_E4M3_POS = E4M3_TABLE[:0x7F].copy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """fp64 value of e4m3fn codes (exact)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3fn code to each finite float32 value; ties to the even code; saturating.

    Distances are taken in fp64.  Where the choice is close (near a midpoint
    between two neighbouring codes) the float32 input and the two candidates
    span at most 25 significant bits, so both distances are exact and the
    comparison is the true one.
    """
    x = np.asarray(x, dtype=np.float32)
    if not np.isfinite(x).all():
        raise ValueError("e4m3_encode takes finite inputs")
    a = np.minimum(np.abs(x.astype(np.float64)), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")  # first code whose value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    return (mag | sign).astype(np.uint8)


def quantize_block128(x_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantise bf16 values in blocks of 128 along the last axis.

    x_bits: uint16 bf16 bits [..., 128 * k].  Returns (scales float32 [..., k],
    codes uint8 [..., 128 * k]) following the rule in the module docstring.
    """
    x = bf16_to_f32(x_bits)
    shp = x.shape
    k = shp[-1] // 128
    xb = x.reshape(shp[:-1] + (k, 128))
    bad = ~np.isfinite(xb).all(axis=-1)  # blocks holding a NaN or an infinity
    xb = np.where(bad[..., None], np.float32(0), xb)
    a = np.max(np.abs(xb), axis=-1)  # float32, exact
    s = (a / np.float32(E4M3_MAX)).astype(np.float32)  # IEEE float32 division
    safe = np.where(s == 0, np.float32(1), s)
    with np.errstate(over="ignore"):
        y = (xb / safe[..., None]).astype(np.float32)  # IEEE float32 division
    # Division overflow only happens when s is subnormal and x/s exceeds fp32;
    # the result saturates like every other magnitude above 448.
    y = np.where(np.isinf(y), np.copysign(np.float32(E4M3_MAX), y), y).astype(np.float32)
    codes = e4m3_encode(y)
    codes = np.where((s == 0)[..., None], np.uint8(0), codes).astype(np.uint8)
    codes = np.where(bad[..., None], np.uint8(0x7F), codes).astype(np.uint8)
    s = np.where(bad, np.uint32(0x7FC00000).view(np.float32), s).astype(np.float32)
    return s, codes.reshape(shp)
