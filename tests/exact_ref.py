"""Exact rational helpers used to pin the oracle (tests only).

These are written independently of the oracle's C code: bf16 values are
decoded with ``struct`` into exact Fractions, and rounding to bf16 is done on
rationals (pick the nearer of the two neighbouring grid points, ties to the
even significand) instead of the oracle's frexp / nearbyint route.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

import torch


def bits_to_fraction(bits: int) -> Fraction:
    f = struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]
    if math.isnan(f) or math.isinf(f):
        raise ValueError("non-finite bf16")
    return Fraction(f)


def fraction_to_bf16_bits(q: Fraction) -> int:
    """Correct rounding of a rational to bf16 (nearest, ties to even)."""
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 7)
    m = a / ulp
    lo = math.floor(m)
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    val = lo * ulp
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    f32 = struct.unpack("<I", struct.pack("<f", float(val)))[0]
    assert Fraction(struct.unpack("<f", struct.pack("<I", f32))[0]) == val
    return sign | (f32 >> 16)


def tensor_bits(t: torch.Tensor):
    """bf16 tensor -> nested Python lists of 16-bit patterns."""
    return (t.contiguous().view(torch.int16).to(torch.int32) & 0xFFFF).tolist()


def bf16_ulp_half(ref: torch.Tensor) -> torch.Tensor:
    """Half a bf16 grid spacing at |ref| (float64), for a correct-rounding
    check |o - ref| <= half-spacing of ref's binade."""
    a = ref.abs().clamp_min(2.0 ** -126)
    e = torch.floor(torch.log2(a))
    # guard log2 rounding at exact powers of two
    e = torch.where(torch.pow(2.0, e) > a, e - 1, e)
    e = torch.where(torch.pow(2.0, e + 1) <= a, e + 1, e)
    return torch.pow(2.0, e - 8)
