"""Number formats, written from their definitions (test infrastructure only).

* bf16: the upper 16 bits of an IEEE-754 binary32 value. Decoding is exact;
  encoding from binary32 rounds to nearest, ties to even, on the 16 dropped
  bits.
* fp8 E4M3FN [OCP-FP8]: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
  bits. Exponent field 0 encodes subnormals m * 2^-9; exponent field 15 with
  mantissa 7 is NaN; there is no infinity; the largest finite value is 448.
* Dequantization [DCP-PR, section 3.2 figure and 3.3 "fp8 stays on the wire"]:
  the cached latent is converted to bf16 and multiplied by the per-tensor
  scale. Reading (documented): the fp8 value is widened exactly, multiplied by
  the f32 scale in binary32 with round-to-nearest-even, and the product is
  rounded to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import math

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def f32_to_bf16_rne(x) -> np.ndarray:
    """binary32 -> bf16 bit patterns, round to nearest, ties to even.

    NaN inputs give a quiet NaN with the input's sign; overflow past the
    largest bf16 gives infinity (the carry runs into the exponent field).
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if np.any(nan):
        rounded = np.where(nan, ((u >> np.uint64(16)) | np.uint64(0x0040)).astype(np.uint16),
                           rounded)
    return rounded.astype(np.uint16)


def fp8_e4m3_to_f64(bits) -> np.ndarray:
    """Exact value of OCP E4M3FN bit patterns (uint8) as float64 [OCP-FP8]."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = sign * m * 2.0 ** -9
    val = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, val)


def fp8_e4m3_dequant_bf16(bits, scale: float) -> np.ndarray:
    """fp8 bits -> bf16 bits of RNE_bf16(RNE_f32(value * scale))."""
    v32 = fp8_e4m3_to_f64(bits).astype(np.float32)  # exact: every E4M3 value is a binary32
    prod = v32 * np.float32(scale)                   # binary32 multiply, RNE
    return f32_to_bf16_rne(prod)


def decode(raw, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Stored values of a KV or query tensor as float64.

    ``dtype`` is 'f32' (float32 storage), 'bf16' (uint16 bit patterns) or
    'fp8_e4m3' (uint8 bit patterns, dequantized to bf16 with ``scale``
    before use, as the DCP-PR pipeline does).
    """
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(raw)
    if dtype == "fp8_e4m3":
        return bf16_to_f64(fp8_e4m3_dequant_bf16(raw, scale))
    raise ValueError(f"unknown dtype {dtype!r}")


LN2 = math.log(2.0)
