"""Pins for the oracle's MX-FP8 quantiser (CPU only): the E4M3 table against its closed form
and torch's float8_e4m3fn conversion, round trips, ties to even at every midpoint,
saturation, the block scale exponent, the vectorised encoder against the brute-force one,
and the quantisation error bound."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp8 as F8


def test_table_closed_form():
    assert F8.e4m3_value(0x7E) == 448
    assert F8.e4m3_value(0x01) == Fraction(1, 512)          # smallest subnormal 2^-9
    assert F8.e4m3_value(0x08) == Fraction(1, 64)           # smallest normal 2^-6
    assert F8.e4m3_value(0x38) == 1
    assert F8.e4m3_value(0xB8) == -1
    vals = [F8.e4m3_value(c) for c in range(0x7F)]
    assert vals == sorted(vals) and len(set(vals)) == 127
    with pytest.raises(ValueError):
        F8.e4m3_value(0x7F)


def test_table_against_torch():
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)
    t = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert t.tolist() == [float(F8.e4m3_value(c)) for c in range(0x7F)]


def test_round_trip_and_midpoints():
    for c in range(0x7F):
        v = float(F8.e4m3_value(c))
        assert F8.e4m3_encode(v) == c and F8.e4m3_encode(-v) == (c | 0x80)
    for c in range(0x7E):
        mid = (F8.e4m3_value(c) + F8.e4m3_value(c + 1)) / 2
        want = c if c % 2 == 0 else c + 1
        assert F8.e4m3_encode(float(mid)) == want
        # just off the midpoint goes to the nearer code
        assert F8.e4m3_encode(float(mid) * (1 - 1e-12)) == c
        assert F8.e4m3_encode(float(mid) * (1 + 1e-12)) == c + 1


def test_saturation_and_sign():
    assert F8.e4m3_encode(449.0) == 0x7E and F8.e4m3_encode(1e30) == 0x7E
    assert F8.e4m3_encode(-1e30) == 0xFE
    assert F8.e4m3_encode(-0.0) == 0x80 and F8.e4m3_encode(0.0) == 0x00
    assert F8.e4m3_encode(-2.0 ** -12) == 0x80             # rounds to -0


def test_in_range_values_match_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.normal(size=4000) * s for s in (1e-3, 0.1, 1, 30, 200)])
    v = v[np.abs(v) < 440].astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(F8.e4m3_encode_array(v), ref)


def test_vectorised_encoder_equals_brute_force():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.normal(size=300) * 100, rng.normal(size=300) * 1e-3,
                        [0.0, -0.0, 448.0, 464.0, 500.0, -1e6, 2.0 ** -10, 3 * 2.0 ** -11]])
    v = v.astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(F8.e4m3_encode_array(v),
                                  np.array([F8.e4m3_encode(float(x)) for x in v], np.uint8))


def test_scale_exponent():
    assert F8.mx_scale_exponent([0.0] * 32) == -127
    assert F8.mx_scale_exponent([1.0] + [0.0] * 31) == -8        # 2^0 - 8
    assert F8.mx_scale_exponent([-256.0, 3.0]) == 0
    assert F8.mx_scale_exponent([511.9]) == 0 and F8.mx_scale_exponent([512.0]) == 1
    assert F8.mx_scale_exponent([2.0 ** 200]) == 127               # clamped
    X = np.array([[2.0 ** k] + [0.0] * 31 for k in range(-20, 20)])
    codes, sc = F8.mx_quantize_rows(X)
    assert (sc[:, 0].astype(int) - 127 == np.arange(-20, 20) - 8).all()
    assert (codes[:, 0] == 0x78).all()                              # 2^k / 2^(k-8) = 256


def test_quantisation_error_bound():
    # |deq(q(v)) - v| <= half an E4M3 ulp at v's binade (2^(floor(log2|v|) - 4) times the
    # block scale), except in the saturated range and below the subnormal step
    rng = np.random.default_rng(2)
    X = (rng.normal(size=(64, 256)) * np.exp(rng.normal(size=(64, 1)))).astype(np.float32)
    X = X.astype(np.float64)
    codes, sc = F8.mx_quantize_rows(X)
    D = F8.mx_dequantize(codes, sc)
    scale = np.repeat(np.exp2(sc.astype(float) - 127), 32, axis=1)
    y = np.abs(X) / scale
    binade = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
    bound = np.exp2(binade - 4) * scale
    ok = y <= 448
    assert (np.abs(D - X)[ok] <= bound[ok] * (1 + 1e-12)).all()
    assert (np.abs(D[~ok]) == 448 * scale[~ok]).all()
    # the block maximum lands in [256, 512): the top binades of E4M3 are used
    assert ((np.abs(X).reshape(64, 8, 32).max(2) / np.exp2(sc - 127.0)) >= 256).all()
