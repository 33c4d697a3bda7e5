"""Pins for the oracle's E4M3 codec (oracle.fp8) against torch's
float8_e4m3fn (a library implementation of the OCP format) and against values
worked out by hand from the format definition."""

import numpy as np
import torch

from oracle import fp8


def test_all_256_codes_decode_like_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)) and nan.sum() == 2  # 0x7F, 0xFF only
    assert np.array_equal(got[~nan], ref[~nan])


def test_hand_values():
    # from the definition: bias 7, largest finite 1.75 * 2^8, smallest subnormal 2^-9
    assert fp8.decode_code(0x7E) == 448.0
    assert fp8.decode_code(0x01) == 2.0 ** -9
    assert fp8.decode_code(0x08) == 2.0 ** -6
    assert fp8.decode_code(0x38) == 1.0
    assert fp8.decode_code(0xB9) == -1.125
    assert fp8.decode_code(0x80) == 0.0 and np.signbit(fp8.decode_code(0x80))


def test_finite_codes_round_trip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8.quantise(fp8.decode(codes)), codes)


def test_ties_go_to_even_and_saturation():
    # 1.0625 lies half way between 1.0 (0x38, even) and 1.125 (0x39)
    assert fp8.quantise([1.0625])[0] == 0x38
    # 1.1875 lies half way between 1.125 (0x39) and 1.25 (0x3A, even)
    assert fp8.quantise([1.1875])[0] == 0x3A
    # half of the smallest subnormal rounds to zero (even), 1.5 of it to 2^-8
    assert fp8.quantise([2.0 ** -10])[0] == 0x00
    assert fp8.quantise([1.5 * 2.0 ** -9])[0] == 0x02
    assert list(fp8.quantise([448.0, 460.0, 1e6, -1e6])) == [0x7E, 0x7E, 0x7E, 0xFE]
    assert fp8.quantise([-1e-30])[0] == 0x80


def test_quantise_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000) * 50,
        rng.standard_normal(50000) * 0.01,
        rng.uniform(-448, 448, 50000),
        # every midpoint between neighbouring finite magnitudes, both signs
        (lambda v: np.concatenate([v, -v]))((fp8._POS[1:] + fp8._POS[:-1]) / 2),
    ]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.quantise(x), ref)


def test_scaled_quantisation_uses_one_fp32_division():
    x = np.float32([0.3, -2.5, 7.0])
    s = np.float32(1.0 / 64.0)
    codes = fp8.quantise_scaled(x, s)
    assert np.array_equal(codes, fp8.quantise(np.float32(x) / s))
    back = fp8.dequantise(codes, s)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2 ** -4 + 1e-12)
