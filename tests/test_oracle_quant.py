"""Pins of the fp8 (OCP E4M3) and int8 oracles (CPU only): the format's
closed-form values, torch's float8_e4m3fn cast and qint8 quantisation, brute
force, and the saturation readings."""

import numpy as np
import pytest
import torch

from oracle import quant_oracle as Q


def test_table_closed_forms():
    t = Q.E4M3_TABLE
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest finite: 1.75 * 2^8
    assert t[0x08] == 2.0 ** -6                            # smallest normal
    assert t[0x01] == 2.0 ** -9                            # smallest subnormal: 1/8 * 2^-6
    assert t[0x38] == 1.0                                  # exponent 7 = bias
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])         # the only NaNs; no infinity
    assert np.isfinite(t).sum() == 254
    assert (np.diff(t[:0x7F]) > 0).all()                   # codes 0..0x7E increase
    np.testing.assert_array_equal(t[0x80:0xFF], -t[:0x7F])


def test_codes_match_torch_float8_e4m3fn():
    rng = np.random.default_rng(3)
    vals = Q.E4M3_TABLE[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2                      # exact ties between neighbours
    x = np.concatenate([rng.standard_normal(20000) * 30, rng.standard_normal(5000) * 1e-3, vals, mids, -vals, -mids,
                        [464.0, -464.0]]).astype(np.float32)
    x = x[np.abs(x.astype(np.float64)) <= 464.0]           # torch turns larger magnitudes into NaN
    got = Q.quantize_e4m3(x, 1.0)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, ref)


def test_brute_force_nearest_with_ties_to_even():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(300).astype(np.float32) * 20
    got = Q.quantize_e4m3(x, 1.0)
    for xi, ci in zip(x, got):
        best = min(range(0x7F), key=lambda c: (abs(Q.E4M3_TABLE[c] - abs(float(xi))), c & 1))
        assert ci == (best | (0x80 if xi < 0 else 0))


def test_saturation_sign_and_nan():
    q = Q.quantize_e4m3(np.array([500.0, -1000.0, 1e30, -1e30, 449.0], np.float32), 1.0)
    np.testing.assert_array_equal(q, [0x7E, 0xFE, 0x7E, 0xFE, 0x7E])
    q = Q.quantize_e4m3(np.array([-0.0, -1e-9, 0.0, 1e-9, np.nan], np.float32), 1.0)
    np.testing.assert_array_equal(q, [0x80, 0x80, 0x00, 0x00, 0x7F])


def test_scale_product_is_rounded_in_float32():
    # x * s_inv is formed in float32 before the code is chosen: here the exact
    # product 3.6250000812 lies above the 3.5 / 3.75 midpoint (code 71), but its
    # float32 rounding is the midpoint itself, which goes to the even code 70
    x, s_inv = np.float32(0.38119414), np.float32(9.50959)
    assert float(x) * float(s_inv) > 3.625 and np.float32(x * s_inv) == np.float32(3.625)
    assert Q.quantize_e4m3(np.array([x]), s_inv)[0] == 70


def test_round_trip_error_bound():
    # normal range: |x - dequant(quant(x))| <= 2^-4 |x| (half a unit in the last place)
    rng = np.random.default_rng(9)
    x = (rng.uniform(2.0 ** -6, 448.0, 5000) * rng.choice([-1, 1], 5000)).astype(np.float32)
    d = Q.dequantize_e4m3(Q.quantize_e4m3(x, 1.0), 1.0)
    assert (np.abs(d - x) <= 2.0 ** -4 * np.abs(x)).all()


def test_linear_fp8_brute_force():
    rng = np.random.default_rng(11)
    qa = rng.integers(0, 0x7F, (3, 5)).astype(np.uint8) | (rng.integers(0, 2, (3, 5)) * 0x80).astype(np.uint8)
    qw = rng.integers(0, 0x7F, (2, 5)).astype(np.uint8)
    b = rng.standard_normal(2)
    y = Q.linear_fp8(qa, 0.5, qw, 0.25, b)
    for m in range(3):
        for n in range(2):
            s = sum(Q.e4m3_value(int(qa[m, k])) * 0.5 * Q.e4m3_value(int(qw[n, k])) * 0.25 for k in range(5))
            assert y[m, n] == pytest.approx(s + b[n], rel=1e-13, abs=1e-13)


# ---------------------------------------------------------------- int8


def test_int8_codes_match_torch_qint8_in_range():
    # power-of-two scales make x * s_inv and torch's x / scale the same exact
    # value, so both sides round the same number (ties included)
    rng = np.random.default_rng(13)
    for k in (0, 3, -4):
        s_inv = 2.0 ** k
        ties = (np.arange(-127, 127) + 0.5) / s_inv
        x = np.concatenate([rng.uniform(-126.9, 126.9, 20000) / s_inv, ties]).astype(np.float32)
        got = Q.quantize_int8(x, s_inv)
        ref = torch.quantize_per_tensor(torch.from_numpy(x), 1.0 / s_inv, 0, torch.qint8).int_repr().numpy()
        np.testing.assert_array_equal(got, ref)


def test_int8_brute_force_nearest_with_ties_to_even():
    rng = np.random.default_rng(17)
    x = np.concatenate([rng.uniform(-130, 130, 400), np.arange(-130, 130) + 0.5]).astype(np.float32)
    got = Q.quantize_int8(x, 1.0)
    for xi, ci in zip(x, got):
        v = float(xi)
        best = min(range(-127, 128), key=lambda c: (abs(c - v), c & 1))
        assert ci == best


def test_int8_saturation_and_nan():
    x = np.array([200.0, -200.0, 1e30, -np.inf, np.inf, np.nan, 127.5, -127.5, 126.5, -0.5, 0.5, -1e-30], np.float32)
    np.testing.assert_array_equal(Q.quantize_int8(x, 1.0), [127, -127, 127, -127, 127, 0, 127, -127, 126, 0, 0, 0])


def test_int8_scale_product_is_rounded_in_float32():
    # the exact product 100.50000055 would round up to 101; its float32
    # rounding is the tie 100.5 itself, which goes to the even 100
    x, s_inv = np.float32(18.348232), np.float32(5.477367)
    assert float(x) * float(s_inv) > 100.5 and np.float32(x * s_inv) == np.float32(100.5)
    assert Q.quantize_int8(np.array([x]), s_inv)[0] == 100


def test_int8_round_trip_error_bound():
    # within range: |x - dequant(quant(x))| <= scale / 2
    rng = np.random.default_rng(19)
    scale = 0.037
    x = rng.uniform(-127 * scale, 127 * scale, 5000).astype(np.float32)
    d = Q.dequantize_int8(Q.quantize_int8(x, np.float32(1 / scale)), scale)
    assert (np.abs(d - x) <= scale / 2 * (1 + 1e-6)).all()


def test_linear_int8_brute_force_and_extremes():
    rng = np.random.default_rng(23)
    qa = rng.integers(-127, 128, (3, 7)).astype(np.int8)
    qw = rng.integers(-127, 128, (2, 7)).astype(np.int8)
    b = rng.standard_normal(2)
    y = Q.linear_int8(qa, 0.5, qw, 0.25, b)
    for m in range(3):
        for n in range(2):
            acc = sum(int(qa[m, k]) * int(qw[n, k]) for k in range(7))
            assert y[m, n] == acc * 0.125 + b[n]
    # every product at the extreme: the sum is K * 127^2, held exactly
    K = 4096
    ext = np.full((1, K), -127, np.int8)
    assert Q.int8_products(ext, -ext)[0, 0] == -K * 127 * 127
    assert Q.int8_products(ext, ext)[0, 0] == K * 16129
