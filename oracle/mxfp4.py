"""Decoding of block-scaled 4-bit index vectors (MXFP4) for the fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the benchmark's
CPU-baseline leg may import this module. It shares no code with the HIP path.

"Sparse Attention", Chapter 4 (FP4: token-level scoring, block-level selection): the index
vectors Qidx and Kidx are compared in 4-bit precision, one score per (query, key), and each
block keeps its largest score; the selection is then the usual top-K. The page scores
prepared 4-bit vectors with their scales (preparation and quantisation lie outside the timed
scorer). On gfx950 the 4-bit format is OCP MXFP4: every 32 consecutive elements of a proxy
row share one E8M0 scale, each element is an E2M1 code.

* E2M1 code (4 bits: sign, 2 exponent bits, 1 mantissa bit, exponent bias 1): exponent field
  e = 0 gives the subnormal value m * 2^-1, otherwise (1 + m / 2) * 2^(e - 1); the sign bit
  negates. The eight magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6. No infinities or NaNs.
* E8M0 scale (8 bits, unsigned exponent, bias 127): 2^(code - 127); code 255 is NaN.
* Packing (this library's layout): element 2i of a row in the low nibble of byte i, element
  2i + 1 in the high nibble; scale b of a row covers elements 32b .. 32b + 31.

The oracle's proxy value is code value times scale, exactly, in fp64; the index branch then
runs unchanged on those values (dot products, max-pooling, top-K).

Pins (CPU tests): the sixteen code values against the format's defining formula written as a
table of sign/exponent/mantissa fields; the E8M0 decode against torch's float8_e8m0fnu; the
decode of quantised Gaussian rows against a brute-force nearest-value search; a dot product of
dequantised rows against the same sum computed by integer arithmetic on codes and exponents.
"""
from __future__ import annotations

import numpy as np

MX_BLOCK = 32


def e2m1_value(code: np.ndarray) -> np.ndarray:
    """Value of 4-bit E2M1 codes (any integer array with values 0..15) as float64."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return sign * mag


def e8m0_value(code: np.ndarray) -> np.ndarray:
    """Value of E8M0 scale codes (0..255) as float64; 255 gives NaN."""
    c = np.asarray(code, dtype=np.int64)
    return np.where(c == 255, np.nan, np.exp2(c.astype(np.float64) - 127.0))


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[..., dp / 2] bytes -> [..., dp] codes (low nibble first)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def dequantize(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 rows -> float64 values: packed [..., dp / 2] uint8, scales [..., dp / 32] uint8."""
    codes = unpack_codes(packed)
    dp = codes.shape[-1]
    assert scales.shape[-1] * MX_BLOCK == dp, (scales.shape, dp)
    vals = e2m1_value(codes)
    sc = np.repeat(e8m0_value(scales), MX_BLOCK, axis=-1)
    return vals * sc
