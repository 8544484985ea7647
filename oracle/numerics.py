"""Stored bits of the KV dtypes and their exact widening to fp64.

bf16 is the top half of an IEEE binary32: widening shifts the 16 stored bits
into the high half of a 32-bit word.  fp16 (IEEE binary16) and fp32 widen
exactly through NumPy.  Every bf16/fp16/fp32 value is exactly representable in
fp64, so no rounding happens here.
"""
import numpy as np
import torch

_BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}


def bits_of(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Raw stored bits of a CPU-or-device tensor in ``dtype`` as a NumPy array."""
    t = t.detach().to("cpu").contiguous()
    if dtype == "f32":
        assert t.dtype == torch.float32
        return t.view(torch.int32).numpy().view(np.uint32).copy()
    if dtype == "f16":
        assert t.dtype == torch.float16
    elif dtype == "bf16":
        assert t.dtype == torch.bfloat16
    else:
        raise KeyError(dtype)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of stored bits."""
    if dtype == "f32":
        return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    raise KeyError(dtype)


def bits_dtype(dtype: str):
    return _BITS[dtype]
