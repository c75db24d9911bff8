"""Exact decoding of stored element bytes to fp64 (test infrastructure only).

The oracle reads the same bytes the GPU reads and widens them exactly:
bf16 is the upper half of an IEEE fp32 word, so shifting its 16 bits left by
16 gives the fp32 value bit for bit; fp16 and fp32 convert to fp64 exactly.
"""
import numpy as np


def decode_bf16(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_f16(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float16).astype(np.float64)


def decode_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def decode(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return decode_bf16(x)
    if dtype == "f32":
        return decode_f32(x)
    if dtype == "f16":
        return decode_f16(x)
    raise ValueError(dtype)
