"""Pins for the oracle's scalar building blocks: bf16 widening, one-step
rounding of a double to bf16 (nearest, ties to even) and SiLU."""
import math
import random
import struct
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle
from tests.exact_ref import bits_to_fraction, fraction_to_bf16_bits


def test_every_finite_bf16_round_trips():
    # widening then rounding must return the same pattern for every finite bf16
    for b in range(0x10000):
        exp = (b >> 7) & 0xFF
        if exp == 0xFF:
            continue
        v = oracle.f64_from_bf16(b)
        assert Fraction(v) == bits_to_fraction(b)
        assert oracle.bf16_from_f64(v) == b, hex(b)


def test_ties_go_to_even_and_neighbours_to_nearest():
    rng = random.Random(7)
    for _ in range(4000):
        b = rng.randrange(0x0001, 0x7F7F)      # positive finite, not the max
        lo, hi = bits_to_fraction(b), bits_to_fraction(b + 1)
        mid = (lo + hi) / 2
        even = b if b % 2 == 0 else b + 1
        assert oracle.bf16_from_f64(float(mid)) == even
        assert oracle.bf16_from_f64(-float(mid)) == even | 0x8000
        eps = (hi - lo) / 1024
        assert oracle.bf16_from_f64(float(mid - eps)) == b
        assert oracle.bf16_from_f64(float(mid + eps)) == b + 1


def test_rounding_matches_exact_rational_rounding_on_random_doubles():
    rng = random.Random(11)
    for _ in range(20000):
        v = rng.uniform(-1, 1) * 2.0 ** rng.randint(-140, 126)
        assert oracle.bf16_from_f64(v) == fraction_to_bf16_bits(Fraction(v)), v


def test_rounding_matches_float32_bit_trick_for_float32_inputs():
    # For values exact in binary32, the textbook integer trick
    # (u + 0x7FFF + lsb) >> 16 is correct rounding; compare with it.
    rng = np.random.default_rng(3)
    f = (rng.standard_normal(50000) * np.exp2(rng.integers(-60, 60, 50000))).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    want = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32)
    got = np.array([oracle.bf16_from_f64(float(v)) for v in f], dtype=np.uint32)
    assert np.array_equal(got, want)


def test_rounding_special_values():
    assert oracle.bf16_from_f64(0.0) == 0x0000
    assert oracle.bf16_from_f64(-0.0) == 0x8000
    assert oracle.bf16_from_f64(float("inf")) == 0x7F80
    assert oracle.bf16_from_f64(float("-inf")) == 0xFF80
    assert oracle.bf16_from_f64(float("nan")) == 0x7FC0
    big = float(bits_to_fraction(0x7F7F))                    # largest finite
    assert oracle.bf16_from_f64(big) == 0x7F7F
    assert oracle.bf16_from_f64(3.5e38) == 0x7F80            # rounds past it
    # subnormal grid 2^-133: smallest subnormal, ties to even around it
    assert oracle.bf16_from_f64(2.0 ** -133) == 0x0001
    assert oracle.bf16_from_f64(2.0 ** -134) == 0x0000       # tie -> 0 (even)
    assert oracle.bf16_from_f64(3 * 2.0 ** -134) == 0x0002   # tie -> 2 (even)
    assert oracle.bf16_from_f64(2.0 ** -126) == 0x0080       # smallest normal


@pytest.mark.parametrize("a", [-30.0, -5.5, -1.0, -0.02, -1e-6, 0.0, 1e-6, 0.013, 0.7, 3.0, 40.0])
def test_silu_closed_forms(a):
    s = oracle.silu(a)
    # library routine: a * logistic(a)
    assert s == pytest.approx(a * scipy.special.expit(a), rel=1e-14, abs=1e-300)
    # odd-part identity: silu(a) - silu(-a) = a
    assert s - oracle.silu(-a) == pytest.approx(a, rel=1e-13, abs=1e-300)


def test_silu_limits():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(800.0) == 800.0
    assert oracle.silu(-800.0) == 0.0
    # derivative at 0 is 1/2: silu(h) ~ h/2 + h^2/4
    h = 1e-5
    assert oracle.silu(h) == pytest.approx(h / 2 + h * h / 4, rel=1e-9)
