"""Bit-level decoders and single-rounding conversions for the oracle.

TEST INFRASTRUCTURE ONLY (see the package header).

* bf16: the upper 16 bits of an IEEE binary32; decoding is exact.
* fp8 e4m3fn (OCP 8-bit float, the format gfx950 and torch.float8_e4m3fn
  use): 1 sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field
  0 is subnormal (m * 2**-9); S.1111.111 is NaN; there is no infinity and the
  largest finite magnitude is 448. Decoding is exact.
* Rounding float64 -> bf16 and float64 -> fp32 is ONE correct
  round-to-nearest-even step (no fp64 -> fp32 -> bf16 double rounding).

Pins (tests/test_oracle_numerics.py): exhaustive comparison of both decoders
with torch's CPU dtypes over every bit pattern; both roundings against exact
rational rounding (fractions.Fraction) on random values and on every kind of
halfway case; the exact-sum check against Fraction sums.
"""

from __future__ import annotations

from fractions import Fraction
import math

import numpy as np

BF16_QUANTUM_MIN_EXP = -133   # smallest bf16 subnormal is 2**-133
F32_QUANTUM_MIN_EXP = -149    # smallest fp32 subnormal is 2**-149


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def fp8e4m3fn_to_f64(bits) -> np.ndarray:
    """OCP fp8 e4m3fn bit patterns (uint8) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    exp = (b >> 3) & 0xF
    man = (b & 0x7).astype(np.float64)
    normal = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    sub = man * 2.0 ** -9
    val = np.where(exp == 0, sub, normal)
    val = np.where((exp == 0xF) & ((b & 0x7) == 0x7), np.nan, val)
    return sign * val


def _round_to_quantum(a: np.ndarray, mant_bits: int, min_qexp: int) -> np.ndarray:
    """RNE of non-negative finite float64 `a` to a binary format with
    `mant_bits` significant bits whose smallest quantum is 2**min_qexp.
    Returns float64 values that are exactly representable in that format
    (or 2**128 on overflow, which the callers turn into infinity)."""
    m, e = np.frexp(a)                       # a = m * 2**e, 0.5 <= m < 1
    qexp = np.maximum(e - mant_bits, min_qexp)
    scaled = np.ldexp(a, -qexp)              # exact: power-of-two scaling
    n = np.rint(scaled)                      # numpy rint: ties to even
    return np.ldexp(n, qexp)


def f64_to_bf16_bits(x) -> np.ndarray:
    """float64 -> bf16 bits, one round-to-nearest-even step."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    fin = np.isfinite(x)
    a = np.abs(np.where(fin, x, 0.0))
    r = _round_to_quantum(a, 8, BF16_QUANTUM_MIN_EXP)
    # r is exactly a bf16 value (or >= 2**128 -> +inf): the fp32 cast is exact.
    with np.errstate(over="ignore"):
        r32 = np.where(r >= 2.0 ** 128, np.float32(np.inf), r.astype(np.float32))
    bits = (r32.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.signbit(x), bits | np.uint16(0x8000), bits)
    out[...] = bits
    out[np.isposinf(x)] = 0x7F80
    out[np.isneginf(x)] = 0xFF80
    out[np.isnan(x)] = 0x7FC0
    return out


def f64_to_f32(x) -> np.ndarray:
    """float64 -> float32, one IEEE round-to-nearest-even step (numpy's cast)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float32)


def _frac_rne(a: Fraction, mant_bits: int, min_qexp: int) -> Fraction:
    """Exact RNE of a non-negative rational to `mant_bits` significant bits."""
    if a == 0:
        return Fraction(0)
    # e with 2**e <= a < 2**(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    qexp = max(e - (mant_bits - 1), min_qexp)
    n = round(a / Fraction(2) ** qexp)       # Fraction.__round__: ties to even
    return n * Fraction(2) ** qexp


def fraction_to_bf16_bits(v: Fraction) -> int:
    """Exact rational -> bf16 bits, round-to-nearest-even (reference rounding)."""
    r = _frac_rne(abs(v), 8, BF16_QUANTUM_MIN_EXP)
    if r >= Fraction(2) ** 128:
        bits = 0x7F80
    else:
        bits = int(np.float32(float(r)).view(np.uint32)) >> 16
    return bits | (0x8000 if v < 0 else 0)


def fraction_to_f32(v: Fraction) -> np.float32:
    """Exact rational -> float32, round-to-nearest-even (reference rounding)."""
    r = _frac_rne(abs(v), 24, F32_QUANTUM_MIN_EXP)
    if r >= Fraction(2) ** 128:
        f = np.float32(np.inf)
    else:
        f = np.float32(float(r))
    return np.float32(-f) if v < 0 else f


def sum_is_exact_in_f64(terms: np.ndarray, axis: int = -1) -> np.ndarray:
    """True where the float64 sum of `terms` along `axis` is exact whatever the
    summation order: every partial sum is a multiple of the smallest unit in
    last place present and is below count * max|term| < 2**(top + 1 + log2 n),
    so it fits in 53 bits when (top + ceil(log2 n) + 1) - min_lsb <= 53."""
    t = np.moveaxis(np.asarray(terms, dtype=np.float64), axis, -1)
    n = t.shape[-1]
    nz = t != 0
    m, e = np.frexp(np.abs(t))
    mant = (m * 2.0 ** 53).astype(np.int64)            # exact 53-bit integer
    lowbit = (mant & -mant).astype(np.float64)         # power of two (or 0)
    tz = np.where(nz, np.log2(np.where(nz, lowbit, 1.0)), 0).astype(np.int64)
    lsb_exp = np.where(nz, e - 53 + tz, np.iinfo(np.int64).max)
    top_exp = np.where(nz, e - 1, np.iinfo(np.int64).min)
    lo = lsb_exp.min(axis=-1)
    hi = top_exp.max(axis=-1)
    width = hi + int(math.ceil(math.log2(max(n, 1)))) + 1 - lo
    return np.where(nz.any(axis=-1), width <= 53, True)


def exact_fraction(x: float) -> Fraction:
    return Fraction(float(x))
