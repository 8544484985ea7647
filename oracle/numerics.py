"""Stored bits of the KV dtypes and their exact widening to fp64.

bf16 is the top half of an IEEE binary32: widening shifts the 16 stored bits
into the high half of a 32-bit word.  fp16 (IEEE binary16) and fp32 widen
exactly through NumPy.  Every bf16/fp16/fp32 value is exactly representable in
fp64, so no rounding happens here.

Two 8-bit code formats hold quantized caches (one byte per element; the value
of an element is its code's value times the pool's scale, see quant.py):

* ``"i8"``: a two's-complement integer in [-128, 127];
* ``"fp8"``: OCP 8-bit floating point E4M3 ("e4m3fn"): sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
  m/8 * 2^-6; exponent 15 with mantissa 7 (0x7F, 0xFF) is NaN; there is no
  infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
"""
import numpy as np
import torch

_BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8,
         "i8": np.uint8}

CODE_DTYPES = ("fp8", "i8")     # 8-bit quantized cache formats


def bits_of(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Raw stored bits of a CPU-or-device tensor in ``dtype`` as a NumPy array."""
    t = t.detach().to("cpu").contiguous()
    if dtype == "f32":
        assert t.dtype == torch.float32
        return t.view(torch.int32).numpy().view(np.uint32).copy()
    if dtype in CODE_DTYPES:
        assert t.element_size() == 1, t.dtype
        return t.view(torch.uint8).numpy().copy()
    if dtype == "f16":
        assert t.dtype == torch.float16
    elif dtype == "bf16":
        assert t.dtype == torch.bfloat16
    else:
        raise KeyError(dtype)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code, from the field layout in the module header."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# value of every code, indexed by the code
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of stored bits (codes: the code's value, unscaled)."""
    if dtype == "f32":
        return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    if dtype == "i8":
        return np.asarray(bits, dtype=np.uint8).view(np.int8).astype(np.float64)
    if dtype == "fp8":
        return E4M3_TABLE[np.asarray(bits, dtype=np.uint8)]
    raise KeyError(dtype)


def bits_dtype(dtype: str):
    return _BITS[dtype]
