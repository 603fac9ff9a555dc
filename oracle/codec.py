"""Decoding of the stored element types into float64 / float32 for the oracle."""
import numpy as np


def bf16_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32, exactly (bf16 is float32's top half)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def decode(a, dtype):
    """Stored tensor -> float64.  dtype is 'f32' or 'bf16' (uint16 bit patterns)."""
    if dtype == "bf16":
        return bf16_to_f32(a).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def decode_f32(a, dtype):
    """Stored tensor -> float32 (exact for both element types)."""
    if dtype == "bf16":
        return bf16_to_f32(a)
    return np.asarray(a, dtype=np.float32)
