"""Int4 group quantization of the compressed cache (the quantizing drafter).

Test infrastructure only (see :mod:`oracle`).

"Riepilogo Tecnico: VeriCache", section "Supporto Architetturale": the
drafter's compressed cache may come from a quantizer as well as from token
eviction, behind one interface.  The pages fix no quantization scheme, so
this module fixes one asymmetric min/max scheme (a reading, not a page fact):

* K: one group = one channel over 32 consecutive tokens
  (``k_scale/k_zero [cap/32][D]`` per KV head);
* V: one group = one token over 32 consecutive channels
  (``v_scale/v_zero [cap][D/32]`` per KV head);
* per group ``s = (max - min) / 15`` and ``z = min``, each rounded to binary16
  (round to nearest even);
* code ``c = clip(rint((x - z16) / s16), 0, 15)`` (ties to even), ``c = 0``
  when ``s16 == 0``;
* reconstruction ``x_hat = c * s16 + z16``;
* storage eight codes per little-endian 32-bit word, code i in nibble
  i // 2 + 4 (i % 2) (the compressed-cache layout the library reads).

Parity: pinned by the half-step error bound, exactness on constant groups and
on values that already lie on the grid, and by reduction of quantized
attention to dense attention over the reconstructed values.
"""
import numpy as np

GROUP = 32


def _scale_zero(mn, mx):
    s16 = ((mx - mn) / 15.0).astype(np.float16)
    z16 = mn.astype(np.float16)
    return s16, z16


def _codes(x, s, z):
    safe = np.where(s > 0, s, 1.0)
    c = np.clip(np.rint((x - z) / safe), 0, 15)
    return np.where(s > 0, c, 0).astype(np.int64)


def quantize_k(k):
    """``k [T][D]`` (T a multiple of 32) -> ``codes [T][D]``, ``scale [T/32][D]``
    and ``zero [T/32][D]`` (binary16)."""
    k = np.asarray(k, dtype=np.float64)
    T, D = k.shape
    g = k.reshape(T // GROUP, GROUP, D)
    s16, z16 = _scale_zero(g.min(axis=1), g.max(axis=1))
    s = s16.astype(np.float64)[:, None, :]
    z = z16.astype(np.float64)[:, None, :]
    return _codes(g, s, z).reshape(T, D), s16, z16


def quantize_v(v):
    """``v [T][D]`` (D a multiple of 32) -> ``codes [T][D]``, ``scale [T][D/32]``
    and ``zero [T][D/32]`` (binary16)."""
    v = np.asarray(v, dtype=np.float64)
    T, D = v.shape
    g = v.reshape(T, D // GROUP, GROUP)
    s16, z16 = _scale_zero(g.min(axis=2), g.max(axis=2))
    s = s16.astype(np.float64)[:, :, None]
    z = z16.astype(np.float64)[:, :, None]
    return _codes(g, s, z).reshape(T, D), s16, z16


def dequantize_k(codes, scale, zero):
    """Reconstruct K: ``codes [T][D]``, ``scale/zero [T/32][D]`` (float64 values)."""
    codes = np.asarray(codes, dtype=np.float64)
    s = np.repeat(np.asarray(scale, dtype=np.float64), GROUP, axis=0)[:codes.shape[0]]
    z = np.repeat(np.asarray(zero, dtype=np.float64), GROUP, axis=0)[:codes.shape[0]]
    return codes * s + z


def dequantize_v(codes, scale, zero):
    """Reconstruct V: ``codes [T][D]``, ``scale/zero [T][D/32]`` (float64 values)."""
    codes = np.asarray(codes, dtype=np.float64)
    s = np.repeat(np.asarray(scale, dtype=np.float64), GROUP, axis=1)
    z = np.repeat(np.asarray(zero, dtype=np.float64), GROUP, axis=1)
    return codes * s + z


def pack_int4(codes):
    """``codes [..., N]`` in 0..15 (N a multiple of 8) -> ``uint8 [..., N/2]``:
    code i of each group of eight in nibble i // 2 + 4 (i % 2) of a
    little-endian 32-bit word."""
    codes = np.asarray(codes, dtype=np.int64)
    if codes.min(initial=0) < 0 or codes.max(initial=0) > 15:
        raise ValueError("int4 codes must lie in 0..15")
    n = codes.shape[-1]
    if n % 8:
        raise ValueError("int4 codes are packed eight per 32-bit word")
    g = codes.reshape(codes.shape[:-1] + (n // 8, 8))
    w = np.zeros(g.shape[:-1], dtype=np.int64)
    for i in range(8):
        w |= g[..., i] << (4 * (i // 2 + 4 * (i % 2)))
    out = np.stack([(w >> (8 * j)) & 255 for j in range(4)], axis=-1).astype(np.uint8)
    return out.reshape(codes.shape[:-1] + (n // 2,))
