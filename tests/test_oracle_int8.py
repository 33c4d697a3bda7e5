"""Pins for the oracle's INT8 codec (oracle.int8): values worked out by hand
from the definition (round half to even, clamp at +-127), the exact round
trip of every code, a bound on the error of a scaled value, and agreement with
torch's own rounding and clamping (library routines)."""

import numpy as np
import torch

from oracle import int8


def test_hand_values():
    # ties go to the even integer; magnitudes past 127 clamp; -0 is 0
    got = int8.quantise([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.4, 127.5, 1e9, -1e9, -0.0, 0.49999997])
    assert list(got) == [0, 2, 2, 0, -2, -2, 126, 127, 127, 127, -127, 0, 0]
    assert got.dtype == np.int8


def test_every_code_round_trips():
    codes = np.arange(-127, 128, dtype=np.int8)
    assert np.array_equal(int8.quantise(codes.astype(np.float64)), codes)
    for s in (np.float32(1.0), np.float32(1 / 32), np.float32(0.0123)):
        back = int8.dequantise(codes, s)
        assert np.array_equal(int8.quantise_scaled(back.astype(np.float32), s), codes)


def test_scaled_error_is_at_most_half_a_step():
    rng = np.random.default_rng(3)
    s = np.float32(1 / 28)
    x = rng.standard_normal(100000).astype(np.float32)
    x = x[np.abs(x) < 127 * float(s)]
    back = int8.dequantise(int8.quantise_scaled(x, s), s)
    assert np.max(np.abs(back - x)) <= 0.5 * float(s) * (1 + 1e-6)


def test_matches_torch_round_and_clamp():
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(100000) * 60, np.arange(-300, 300) + 0.5]).astype(np.float32)
    ref = torch.clamp(torch.round(torch.from_numpy(x)), -127, 127).to(torch.int8).numpy()
    assert np.array_equal(int8.quantise(x), ref)


def test_scaled_quantisation_uses_one_fp32_division():
    x = np.float32([0.3, -2.5, 7.0, 0.017857143])
    s = np.float32(1.0 / 28.0)
    assert np.array_equal(int8.quantise_scaled(x, s), int8.quantise(np.float32(x) / s))
