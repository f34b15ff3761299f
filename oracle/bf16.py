"""Exact decoding of bfloat16 and float16 bit patterns (oracle side; test infrastructure only).

A bfloat16 value is the upper 16 bits of an IEEE-754 binary32 value, so
shifting the 16-bit pattern into the top half of a 32-bit word and
reinterpreting it as float32 recovers the value exactly; widening float32 to
float64 is exact too.  A float16 pattern is IEEE-754 binary16, which numpy's
float16 type reads directly; widening it to float64 is exact.
"""

import numpy as np


def bf16_bits_to_float64(bits) -> np.ndarray:
    """uint16 (or int16) bfloat16 bit patterns -> float64 values, exactly."""
    b = np.asarray(bits)
    if b.dtype == np.int16:
        b = b.view(np.uint16)
    if b.dtype != np.uint16:
        raise TypeError(f"expected uint16/int16 bit patterns, got {b.dtype}")
    words = b.astype(np.uint32) << np.uint32(16)
    return words.view(np.float32).astype(np.float64)


def fp16_bits_to_float64(bits) -> np.ndarray:
    """uint16 (or int16) IEEE binary16 bit patterns -> float64 values, exactly."""
    b = np.asarray(bits)
    if b.dtype == np.int16:
        b = b.view(np.uint16)
    if b.dtype != np.uint16:
        raise TypeError(f"expected uint16/int16 bit patterns, got {b.dtype}")
    return np.ascontiguousarray(b).view(np.float16).astype(np.float64)


def bits_to_float64(bits, dtype="bf16") -> np.ndarray:
    """Decode 16-bit patterns of the given storage type ("bf16" or "fp16")."""
    if dtype == "bf16":
        return bf16_bits_to_float64(bits)
    if dtype == "fp16":
        return fp16_bits_to_float64(bits)
    raise ValueError(f"unknown 16-bit type {dtype!r}")
