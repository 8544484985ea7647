"""Quantization of K/V rows into 8-bit codes for a quantized cache.  TEST
INFRASTRUCTURE ONLY (see the package header).

Page 1 (jisaku.com glossary, section 「他のKVキャッシュ最適化との組み合わせ」)
pairs paging with an INT8-quantized KV cache: one byte per element halves the
block's size, traded against accuracy.  The pages fix neither the scale's
granularity nor the rounding; the readings used here:

* one scale per pool (a K scale and a V scale): an element's value is
  code * scale, so a block holds codes only and is exactly half the size of a
  16-bit block;
* an element x (a bf16/fp16/fp32 source value, exact in fp32) is encoded as
      y = fp32(x * fp32(1 / scale))       (both steps rounded to nearest even)
  followed by
      "i8":  code = clamp(round_half_even(y), -127, 127)   (symmetric range)
      "fp8": code = the E4M3 value nearest to clamp(y, -448, 448), ties to
             the code with an even last bit, sign kept (so -0 and negative
             values rounding to zero give 0x80).
  FP8 E4M3 is not on the pages; it is the other 8-bit format with a native
  conversion on the target GPU, and the same scale reading applies.
"""
from __future__ import annotations

import numpy as np

from .numerics import E4M3_TABLE, to_f64

I8_MAX = 127
E4M3_MAX = 448.0
# non-negative finite E4M3 values, index = code (0x00 .. 0x7E)
_POS = E4M3_TABLE[:0x7F]


def inv_scale_f32(scale) -> np.float32:
    """fp32 reciprocal of a positive finite scale, rounded to nearest even."""
    s = np.float32(scale)
    if not (np.isfinite(s) and s > 0):
        raise ValueError("scale must be a positive finite fp32 value")
    return np.float32(1.0) / s


def scaled_f32(x_bits, src_dtype, scale) -> np.ndarray:
    """y = fp32(x * fp32(1/scale)) for every element (fp32 product, one rounding)."""
    x = to_f64(x_bits, src_dtype).astype(np.float32)      # exact: sources are <= fp32
    if not np.isfinite(x).all():
        raise ValueError("quantization needs finite inputs")
    return (x * inv_scale_f32(scale)).astype(np.float32)


def _e4m3_code(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of fp32 values, by brute force over the 127
    non-negative finite values (ties: the even code), with the sign of y."""
    a = np.minimum(np.abs(y.astype(np.float64)), E4M3_MAX).ravel()
    codes = np.empty(a.shape, dtype=np.uint8)
    for s in range(0, a.size, 1 << 15):
        d = np.abs(a[s:s + (1 << 15), None] - _POS[None, :])         # [n][127]
        best = d.min(axis=1, keepdims=True)
        tie = d == best                                               # 1 or 2 candidates
        even = tie & (np.arange(0x7F)[None, :] % 2 == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), tie.argmax(axis=1))
        codes[s:s + (1 << 15)] = pick
    codes = codes.reshape(y.shape)
    return np.where(np.signbit(y), codes | np.uint8(0x80), codes).astype(np.uint8)


def quantize_ref(x_bits, src_dtype: str, code_dtype: str, scale) -> np.ndarray:
    """Codes (uint8 bits) of source elements given by their stored bits."""
    y = scaled_f32(x_bits, src_dtype, scale)
    if code_dtype == "i8":
        c = np.clip(np.rint(y), -I8_MAX, I8_MAX).astype(np.int8)
        return c.view(np.uint8)
    if code_dtype == "fp8":
        return _e4m3_code(y)
    raise KeyError(code_dtype)


def dequantize_ref(codes, code_dtype: str, scale) -> np.ndarray:
    """fp64 values code * scale (scale taken as the fp32 the cache holds)."""
    return to_f64(codes, code_dtype) * float(np.float32(scale))
