"""Exact decoding of the storage formats the oracle is handed.

Test infrastructure only (see :mod:`oracle`).

Every stored value is widened exactly to float64: a bfloat16 is the upper
half of an IEEE binary32, so shifting its 16 bits left by 16 and reading the
word as binary32 reproduces its value; binary16 widens exactly through
numpy's ``float16``.  Packed int4 codes (the layout of the quantized
compressed cache this library reads) hold eight 4-bit unsigned codes per
little-endian 32-bit word: code i of the word sits in nibble (i // 2) + 4 (i % 2),
i.e. the even codes fill the low 16 bits and the odd codes the high 16 bits.
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
    """uint8 ``[..., N/2]`` -> int64 codes ``[..., N]`` (N a multiple of 8).

    Four bytes form one little-endian word w; code i of its group of eight is
    ``(w >> 4 k) & 15`` with nibble index ``k = i // 2 + 4 (i % 2)``.
    """
    packed = np.asarray(packed, dtype=np.uint8)
    nb = packed.shape[-1]
    if nb % 4:
        raise ValueError("int4 codes are packed in whole 32-bit words")
    b = packed.reshape(packed.shape[:-1] + (nb // 4, 4)).astype(np.int64)
    w = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)
    out = np.empty(packed.shape[:-1] + (nb // 4, 8), dtype=np.int64)
    for i in range(8):
        k = i // 2 + 4 * (i % 2)
        out[..., i] = (w >> (4 * k)) & 15
    return out.reshape(packed.shape[:-1] + (nb * 2,))
