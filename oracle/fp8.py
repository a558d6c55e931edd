"""FP8 KV cache: quantised cache write and read-back, float64 reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Pinned by
tests/test_oracle_fp8.py.

What the pages fix: the cache-write step takes the cache's element type and
two per-tensor scales, k_scale and v_scale, and converts the new K/V rows
when the cache is FP8 ([vllm] §6.3 ``reshape_and_cache_flash(...,
kv_cache_dtype, k_scale, v_scale)``, §7.4 the flash variant of the write
kernel, §8 FP8 KV-cache quantisation among the Triton features).  What they
leave open is read as follows:

* the format is OCP FP8 E4M3 (``e4m3fn``): sign bit 7, exponent bits 6..3
  with bias 7, mantissa bits 2..0; exponent 0 encodes the subnormals
  m/8 * 2^-6; exponent 15 with mantissa 7 is NaN; there are no infinities,
  so the largest finite magnitude is 1.75 * 2^8 = 448;
* the stored code of an element x is x / scale, divided in fp32 (IEEE,
  correctly rounded), rounded to the nearest E4M3 value with ties to the
  even code (the one whose mantissa ends in 0), and saturated to +-448
  (infinities too); NaN stays NaN, as the code 0x7F with the element's
  sign bit (0xFF for a negative NaN);
* a stored code reads back as its E4M3 value times the scale (exact in
  float64).
"""
from __future__ import annotations

import math

import numpy as np

SAT = 448.0  # largest finite E4M3 magnitude


def _code_value(c: int) -> float:
    """Value of one E4M3 code from its sign, exponent and mantissa fields."""
    sign = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3 = np.array([_code_value(c) for c in range(256)], dtype=np.float64)
_POS = E4M3[:0x7F]  # codes 0x00 .. 0x7E: the non-negative finite values, increasing


def e4m3_from_f32(x) -> np.ndarray:
    """Round float32 values to E4M3 codes (nearest, ties to the even code,
    saturating to +-448; NaN -> 0x7F with the input's sign bit)."""
    v = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.minimum(np.abs(v), SAT)
    nan = np.isnan(v)
    a = np.where(nan, 0.0, a)
    i = np.clip(np.searchsorted(_POS, a, side="left"), 0, len(_POS) - 1)  # _POS[i-1] < a <= _POS[i]
    lo = np.maximum(i - 1, 0)
    exact = _POS[i] == a
    d_lo = a - _POS[lo]
    d_hi = _POS[i] - a
    take_lo = ~exact & ((d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0)))
    code = np.where(take_lo, lo, i).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    return (code | np.where(np.signbit(v), np.uint8(0x80), np.uint8(0))).astype(np.uint8)


def f32_of(raw, dtype: str) -> np.ndarray:
    """Stored bf16/f16/f32 elements as float32 (exact)."""
    raw = np.asarray(raw)
    if dtype == "f32":
        return raw.view(np.float32) if raw.dtype != np.float32 else raw
    if dtype == "bf16":
        return (raw.astype(np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    if dtype == "f16":
        return raw.astype(np.uint16).view(np.float16).astype(np.float32)
    raise ValueError(dtype)


def quantize(raw, dtype: str, scale: float) -> np.ndarray:
    """E4M3 codes of stored elements: round(x / scale) with the division in
    fp32 (the write kernel's precision).  A NaN element is stored as the NaN
    code 0x7F carrying the element's own sign bit (the sign of a quotient
    of NaN is not fixed by IEEE arithmetic, so it is taken from x)."""
    x = f32_of(raw, dtype)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        y = (x / np.float32(scale)).astype(np.float32)
    codes = e4m3_from_f32(y)
    nan_code = np.where(np.signbit(x), np.uint8(0xFF), np.uint8(0x7F)).astype(np.uint8)
    return np.where(np.isnan(x), nan_code, codes).astype(np.uint8)


def dequantize(codes, scale: float) -> np.ndarray:
    """Values a cache of E4M3 codes holds: code value times scale (float64)."""
    return E4M3[np.asarray(codes, dtype=np.uint8)] * float(np.float32(scale))
