"""OCP FP8 E4M3 ("e4m3fn") codec for the fp8 KV cache — oracle side.

[course] §11 "Engineering Decision Framework" and §12 "Hands-On Lab" step 3
name an fp8 KV cache (``--kv-cache-dtype fp8``) as the way to shrink per-
sequence KV; the pages fix no fp8 variant. The reading taken here is the OCP
8-bit floating point format E4M3 as published in the OCP OFP8 specification:

  bit layout  s eeee mmm, exponent bias 7
  normal      (-1)^s * 2^(e-7) * (1 + m/8)          for 1 <= e <= 15
  subnormal   (-1)^s * 2^-6 * (m/8) = m * 2^-9       for e = 0
  NaN         s 1111 111 (no infinities); largest finite value 448

Quantisation of a value x with per-tensor scale ``scale``:
  y = float32(x) * float32(1/scale)  (fp32 multiply)
  code = nearest finite E4M3 value to y, ties to the even code,
         |y| >= 448 (and +-inf) saturate to +-448, NaN stays NaN,
         the sign bit is kept (so -0 -> 0x80)
Dequantisation: decode(code) * scale, done in fp64 here.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def _decode_code(code: int) -> float:
    """Value of one E4M3 code, straight from the format definition."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * 2.0 ** (e - 7) * (1.0 + m / 8.0)


DECODE_TABLE = np.array([_decode_code(c) for c in range(256)], dtype=np.float64)
DECODE_TABLE.setflags(write=False)

# Finite non-negative codes 0x00..0x7e in ascending value order.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = DECODE_TABLE[:0x7F].copy()


def decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> fp64 values (table lookup)."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_rne_sat(y: np.ndarray) -> np.ndarray:
    """fp32 values -> uint8 E4M3 codes: nearest value, ties to even code,
    saturating at +-448, NaN -> 0x7f/0xff, sign kept."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    sign = np.where(np.signbit(y), 0x80, 0x00).astype(np.int64)
    flat = a.reshape(-1)
    hi = np.searchsorted(_POS_VALUES, flat, side="left")  # first value >= a
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = flat - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - flat
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(flat >= E4M3_MAX, 0x7E, code)  # saturate (covers +inf)
    code = code.reshape(a.shape) | sign
    code = np.where(np.isnan(y), 0x7F | sign, code)
    return code.astype(np.uint8)


def quantize(x, scale: float) -> np.ndarray:
    """Per-tensor quantisation: encode(float32(x) * float32(1/scale))."""
    inv = np.float32(1.0) / np.float32(scale)
    y = np.asarray(x, dtype=np.float32) * inv
    return encode_rne_sat(y.astype(np.float32))


def dequantize(codes, scale: float) -> np.ndarray:
    """decode(code) * scale in fp64, with the scale taken as its fp32 value."""
    return decode(codes) * np.float64(np.float32(scale))
