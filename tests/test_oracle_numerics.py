"""Pins for the oracle's decoders and roundings.

Everything here is checked against something other than the oracle: torch's
own CPU dtypes (an independent implementation of bf16 / fp8-e4m3fn), exact
rational arithmetic (fractions.Fraction), or hand-derived bit patterns.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.numerics import (
    bf16_to_f64, fp8e4m3fn_to_f64, f64_to_bf16_bits, f64_to_f32,
    fraction_to_bf16_bits, fraction_to_f32, sum_is_exact_in_f64,
)


def test_bf16_decoder_exhaustive_vs_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_fp8_decoder_exhaustive_vs_torch():
    bits = np.arange(256, dtype=np.uint8)
    ours = fp8e4m3fn_to_f64(bits)
    ref = torch.from_numpy(bits.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2                      # S.1111.111 only
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.nanmax(ours) == 448.0 and np.nanmin(np.abs(ours[ours != 0])) == 2.0 ** -9


def test_bf16_rounding_hand_cases():
    one_plus_half_ulp = 1.0 + 2.0 ** -8          # halfway 1 | 1+2^-7 -> even (1)
    cases = [
        (1.0, 0x3F80),
        (one_plus_half_ulp, 0x3F80),
        (1.0 + 3 * 2.0 ** -8, 0x3F82),            # halfway odd|even -> even (up)
        (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),   # just above halfway -> up
        (-1.5, 0xBFC0),
        (2.0 ** -133, 0x0001),                    # smallest subnormal
        (2.0 ** -134, 0x0000),                    # half of it: tie to even (0)
        (3 * 2.0 ** -134, 0x0002),                # 1.5 quanta -> 2
        ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),   # largest finite
        ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),   # halfway to 2^128 -> inf
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (float("inf"), 0x7F80),
    ]
    for x, want in cases:
        assert int(f64_to_bf16_bits(np.array([x]))[0]) == want, x
        if np.isfinite(x) and x != 0:
            assert fraction_to_bf16_bits(Fraction(x)) == want, x
    assert int(f64_to_bf16_bits(np.array([np.nan]))[0]) == 0x7FC0


def _halfway_values(rng, n, mant_bits, min_exp, max_exp):
    """Exact midpoints between adjacent representable values, and neighbours."""
    e = rng.integers(min_exp, max_exp, n)
    m = rng.integers(1 << (mant_bits - 1), 1 << mant_bits, n).astype(np.float64)
    mid = np.ldexp(m + 0.5, e - (mant_bits - 1))
    return np.concatenate([mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)])


def test_bf16_rounding_vs_exact_rationals():
    rng = np.random.default_rng(0)
    xs = np.concatenate([
        rng.standard_normal(3000) * np.exp2(rng.integers(-140, 130, 3000)),
        _halfway_values(rng, 400, 8, -125, 127),
        _halfway_values(rng, 200, 8, -140, -126),        # subnormal range
        rng.standard_normal(200),
    ])
    ours = f64_to_bf16_bits(xs)
    ref = np.array([fraction_to_bf16_bits(Fraction(float(x))) for x in xs], dtype=np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rounding_vs_torch_on_fp32_inputs():
    # torch's fp32 -> bf16 cast is an independent RNE implementation; on
    # fp32-representable inputs the single fp64 -> bf16 rounding must agree.
    rng = np.random.default_rng(1)
    x32 = (rng.standard_normal(100000) * np.exp2(rng.integers(-130, 120, 100000))).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = f64_to_bf16_bits(x32.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_f32_rounding_vs_exact_rationals():
    rng = np.random.default_rng(2)
    xs = np.concatenate([
        rng.standard_normal(2000) * np.exp2(rng.integers(-160, 130, 2000)),
        _halfway_values(rng, 300, 24, -125, 127),
        _halfway_values(rng, 200, 24, -160, -126),
    ])
    ours = f64_to_f32(xs)
    ref = np.array([fraction_to_f32(Fraction(float(x))) for x in xs], dtype=np.float32)
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_exact_sum_check():
    rng = np.random.default_rng(3)
    rows = bf16_to_f64(rng.integers(0, 1 << 16, (200, 16)).astype(np.uint16))
    rows = np.where(np.isfinite(rows), rows, 0.0)
    rows = np.clip(rows, -1e30, 1e30)
    flags = sum_is_exact_in_f64(rows)
    for row, ok in zip(rows, flags):
        exact = sum((Fraction(float(v)) for v in row), Fraction(0))
        if ok:
            assert Fraction(float(row.sum())) == exact
    # a row the check must refuse: huge and tiny terms together
    bad = np.array([[2.0 ** 100, 2.0 ** -100, -(2.0 ** 100), 1.0]])
    assert not sum_is_exact_in_f64(bad)[0]
    good = bf16_to_f64(np.full((1, 16), 0x3F80, dtype=np.uint16))
    assert sum_is_exact_in_f64(good)[0]
