"""Exact decoding of the storage formats the oracle is handed.

Test infrastructure only (see :mod:`oracle`).

Every stored value is widened exactly to float64: a bfloat16 is the upper
half of an IEEE binary32, so shifting its 16 bits left by 16 and reading the
word as binary32 reproduces its value; binary16 widens exactly through
numpy's ``float16``.  Packed int4 codes hold two 4-bit unsigned codes per
byte, the even channel in the low nibble (the layout of the quantized
compressed cache this library reads).
"""
import numpy as np


def bf16_to_f64(bits):
    """uint16 bfloat16 bit patterns -> float64 values (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f16_to_f64(bits):
    """uint16 binary16 bit patterns -> float64 values (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return bits.view(np.float16).astype(np.float64)


def unpack_int4(packed):
    """uint8 ``[..., D/2]`` -> int64 codes ``[..., D]``; low nibble = even channel."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = (packed & 0x0F).astype(np.int64)
    hi = (packed >> 4).astype(np.int64)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out
