"""Pins of the oracle's int4 group quantizer: the half-step error bound,
exactness on constant groups and on values already on the grid, and the
packing layout (eight codes per 32-bit word, even codes in the low half)."""
import numpy as np
import pytest

from oracle import quant as Q
from oracle.formats import unpack_int4, f16_to_f64

RNG = np.random.default_rng(99)


def _bound(x, groups_min, groups_max, s16, z16):
    s = s16.astype(np.float64)
    z = z16.astype(np.float64)
    # half a step, plus what binary16 rounding of the step and the zero adds
    return s / 2 + np.abs(groups_min - z) + 15 * np.abs((groups_max - groups_min) / 15 - s) + 1e-12


def test_k_error_bound_and_code_range():
    k = RNG.standard_normal((128, 64)) * 1.7
    c, s16, z16 = Q.quantize_k(k)
    assert c.min() >= 0 and c.max() <= 15
    kh = Q.dequantize_k(c, s16, z16)
    g = k.reshape(4, 32, 64)
    bound = _bound(k, g.min(1), g.max(1), s16, z16)
    err = np.abs(k - kh).reshape(4, 32, 64)
    assert np.all(err <= bound[:, None, :])
    # the error is not vacuously small: the quantizer is lossy
    assert np.abs(k - kh).max() > 1e-2


def test_v_error_bound():
    v = RNG.standard_normal((40, 128))
    c, s16, z16 = Q.quantize_v(v)
    vh = Q.dequantize_v(c, s16, z16)
    g = v.reshape(40, 4, 32)
    bound = _bound(v, g.min(2), g.max(2), s16, z16)
    assert np.all(np.abs(v - vh).reshape(40, 4, 32) <= bound[:, :, None])


def test_constant_group_exact():
    v = np.full((3, 64), 0.375)          # binary16-representable
    c, s16, z16 = Q.quantize_v(v)
    assert np.all(c == 0) and np.all(s16 == 0)
    np.testing.assert_array_equal(Q.dequantize_v(c, s16, z16), v)


def test_on_grid_values_roundtrip_exactly():
    # values c*s + z with both extreme codes present in every group: the
    # quantizer recovers the same scale, zero and codes
    T, D = 64, 64
    s = np.float16(0.25) * (1 + RNG.integers(0, 4, (T // 32, D))).astype(np.float16)
    z = (-RNG.integers(0, 8, (T // 32, D)) * 0.5).astype(np.float16)
    codes = RNG.integers(0, 16, (T, D))
    codes[0::32] = 0
    codes[1::32] = 15
    k = codes * np.repeat(s.astype(np.float64), 32, 0) + np.repeat(z.astype(np.float64), 32, 0)
    c2, s2, z2 = Q.quantize_k(k)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, s)
    np.testing.assert_array_equal(z2, z)
    np.testing.assert_array_equal(Q.dequantize_k(c2, s2, z2), k)


def test_rint_ties_to_even():
    # a value exactly half way between two grid points rounds to the even code
    v = np.zeros((1, 32))
    v[0, 1] = 15.0           # s = 1, z = 0
    v[0, 2] = 2.5            # -> code 2
    v[0, 3] = 3.5            # -> code 4
    c, s16, z16 = Q.quantize_v(v)
    assert f16_to_f64(s16.view(np.uint16))[0, 0] == 1.0
    assert c[0, 2] == 2 and c[0, 3] == 4


def test_pack_unpack_layout():
    codes = RNG.integers(0, 16, (5, 64))
    packed = Q.pack_int4(codes)
    assert packed.shape == (5, 32) and packed.dtype == np.uint8
    # worked by hand: codes 1..8 -> word 0x86427531, bytes 31 75 42 86
    assert Q.pack_int4(np.arange(1, 9)).tolist() == [0x31, 0x75, 0x42, 0x86]
    assert unpack_int4(np.array([0x31, 0x75, 0x42, 0x86], np.uint8)).tolist() == list(range(1, 9))
    np.testing.assert_array_equal(unpack_int4(packed), codes)
    with pytest.raises(ValueError):
        Q.pack_int4(np.array([[16, 0, 0, 0, 0, 0, 0, 0]]))
