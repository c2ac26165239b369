"""CPU oracle for the fp8 KV cache: OCP E4M3 codes with one scale per KV head.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``; never imported by the
product path and sharing no code with the GPU kernels.

The pages name quantisation of the KV cache as the lever for long contexts
(runbyai section 5, on the trade-offs in practice).  They fix no format, so
this is a reading: an 8-bit float per element, OCP "E4M3" (1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits; no infinities; 0x7F / 0xFF
are NaN; largest finite value 448 = 1.75 * 2^8; subnormals m * 2^-9), with
one positive fp32 scale per KV head for K and one for V:

* cache write:  code = E4M3(fp32(x / scale[h])), x the bf16 or fp32 input
  row element, fp32(.) one correctly rounded fp32 division, E4M3(.)
  round-to-nearest-even with saturation to +-448;
* attention reads K = decode(code) * k_scale[h], V = decode(code) * v_scale[h].

Everything here follows that definition directly, in float64 (every fp32
and every E4M3 value is exact in float64).
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

from .paged_attention import widen, write_k_row, write_v_row

E4M3_MAX = 448.0
E4M3_NAN_CODES = (0x7F, 0xFF)


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code, from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * m * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_DECODE_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """float64 values of an array of E4M3 codes (uint8)."""
    return _DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode_scalar(y: float) -> int:
    """Nearest E4M3 code to a finite y (ties to even mantissa), saturating at +-448."""
    if math.isnan(y):
        raise ValueError("NaN has no E4M3 encoding here")
    sign = 0x80 if (y < 0 or (y == 0 and math.copysign(1.0, y) < 0)) else 0
    a = abs(y)
    if a >= E4M3_MAX:
        return sign | 0x7E
    # candidates: the two representable magnitudes around a
    mags = _DECODE_TABLE[:0x7F]                  # codes 0x00..0x7E, increasing
    i = int(np.searchsorted(mags, a, side="right")) - 1   # mags[i] <= a < mags[i+1]
    lo, hi = mags[i], mags[min(i + 1, 0x7E)]
    if a == lo:
        return sign | i
    if a - lo < hi - a:
        return sign | i
    if a - lo > hi - a:
        return sign | (i + 1)
    return sign | (i if i % 2 == 0 else i + 1)   # tie: even code = even mantissa


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Vectorised ``e4m3_encode_scalar`` over finite float arrays."""
    flat = np.asarray(y, dtype=np.float64).reshape(-1)
    out = np.fromiter((e4m3_encode_scalar(v) for v in flat), dtype=np.uint8, count=flat.size)
    return out.reshape(np.shape(y))


def quantize_row(x_bits: np.ndarray, src_dtype: str, scale: float) -> np.ndarray:
    """Codes of one row: E4M3(fp32(x / scale)) with a correctly rounded fp32 division."""
    x32 = widen(x_bits, src_dtype).astype(np.float32)
    y = (x32 / np.float32(scale)).astype(np.float32)
    return e4m3_encode(y)


def ref_reshape_and_cache_fp8(k_new: np.ndarray, v_new: np.ndarray, slot_mapping: np.ndarray, k_pool: np.ndarray,
                              v_pool: np.ndarray, k_scale: Sequence[float], v_scale: Sequence[float],
                              src_dtype: str):
    """Copies of the uint8 pools after quantising every new row into its slot.

    ``k_new``/``v_new`` ``[T, Hkv, D]`` hold fp32 values or bf16 bit
    patterns (``src_dtype``); pools use the documented layout with 16
    elements per 16-byte K chunk.
    """
    kp = k_pool.copy()
    vp = v_pool.copy()
    bs = kp.shape[3]
    T, Hkv, _ = k_new.shape
    for t in range(T):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        b, o = divmod(slot, bs)
        for h in range(Hkv):
            write_k_row(kp, b, h, o, quantize_row(k_new[t, h], src_dtype, float(k_scale[h])))
            write_v_row(vp, b, h, o, quantize_row(v_new[t, h], src_dtype, float(v_scale[h])))
    return kp, vp


def dequantize_pool(pool: np.ndarray, scale: Sequence[float]) -> np.ndarray:
    """float64 values of a uint8 pool: decode(code) * scale[head] (head = axis 1)."""
    vals = e4m3_decode(pool)
    s = np.asarray(scale, dtype=np.float64).reshape((1, -1) + (1,) * (pool.ndim - 2))
    return vals * s
