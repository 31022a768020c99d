"""Pins of the gradient-arrival oracle (accumulate + fused norm statistics).

Independent reference: exact rational arithmetic (fractions) rounds the exact
sum to 24 significant bits and then to the storage precision (8 bits for bf16,
11 for fp16), to nearest with ties to even, over random pairs spanning many
binades.  Tie cases are worked by hand.  Copy mode must return the arriving
buffer bit for bit; adding zero must return the held buffer; the fused
statistics must equal the norm pass on the new gradients.  Planted mistakes
(truncation, half-up ties, adding in fp64, ignoring the held value) must each
fail a pin.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
from oracle import accumulate_fp64 as AC

RNG = np.random.default_rng(20251202)


def rne(x: Fraction, bits: int) -> Fraction:
    """Round a rational to `bits` significant bits, nearest, ties to even
    (no overflow or subnormal handling: the test values stay in range)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    scale = Fraction(2) ** (bits - 1 - e)
    m = a * scale
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * Fraction(n) / scale


def bf16_value(bits) -> Fraction:
    return Fraction(float((np.uint32(bits) << np.uint32(16)).view(np.float32)))


def random_bf16(n, lo=-20, hi=20):
    """bf16 bit patterns with exponents in [lo, hi] and random signs/mantissas."""
    e = RNG.integers(lo, hi + 1, size=n) + 127
    m = RNG.integers(0, 128, size=n)
    s = RNG.integers(0, 2, size=n)
    return ((s << 15) | (e << 7) | m).astype(np.uint16)


def pin_bf16_exact_rounding_random_pairs():
    held = random_bf16(3000)
    inc = random_bf16(3000)
    # near-cancelling pairs and pairs a few binades apart
    inc[:300] = held[:300] ^ np.uint16(0x8000)
    inc[300:600] = (held[300:600].astype(np.int32) + RNG.integers(-3, 4, size=300)).astype(np.uint16) ^ np.uint16(0x8000)
    got = AC.accumulate_gradient(held, inc, True)
    for h, i, gbits in zip(held, inc, got):
        want = rne(rne(bf16_value(h) + bf16_value(i), 24), 8)
        assert bf16_value(gbits) == want, (hex(h), hex(i), hex(gbits), want)


def pin_f16_exact_rounding_random_pairs():
    e = RNG.integers(-10, 11, size=3000).astype(np.float64)
    held = (RNG.uniform(1, 2, size=3000) * 2.0 ** e * RNG.choice([-1, 1], size=3000)).astype(np.float16)
    inc = (RNG.uniform(1, 2, size=3000) * 2.0 ** e[::-1] * RNG.choice([-1, 1], size=3000)).astype(np.float16)
    got = AC.accumulate_gradient(held, inc, True)
    assert got.dtype == np.float16
    for h, i, g in zip(held, inc, got):
        want = rne(rne(Fraction(float(h)) + Fraction(float(i)), 24), 11)
        assert Fraction(float(g)) == want, (h, i, g, want)


def pin_fp32_exact_rounding_random_pairs():
    held = (RNG.standard_normal(2000) * 10.0 ** RNG.integers(-6, 6, size=2000)).astype(np.float32)
    inc = (RNG.standard_normal(2000) * 10.0 ** RNG.integers(-6, 6, size=2000)).astype(np.float32)
    got = AC.accumulate_gradient(held, inc, True)
    assert got.dtype == np.float32
    for h, i, g in zip(held, inc, got):
        assert Fraction(float(g)) == rne(Fraction(float(h)) + Fraction(float(i)), 24)


def pin_bf16_ties_by_hand():
    one, tiny = np.uint16(0x3F80), np.uint16(0x3B80)          # 1.0 and 2^-8
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even 1.0
    assert AC.accumulate_gradient(np.array([one]), np.array([tiny]), True)[0] == 0x3F80
    # (1 + 2^-7) + 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert AC.accumulate_gradient(np.array([np.uint16(0x3F81)]), np.array([tiny]), True)[0] == 0x3F82
    # 1 + 2^-30 rounds to 1.0 already in fp32
    assert AC.accumulate_gradient(np.array([one]), np.array([np.uint16(0x3080)]), True)[0] == 0x3F80
    # 3 + 1 = 4 exactly
    assert AC.accumulate_gradient(np.array([np.uint16(0x4040)]), np.array([one]), True)[0] == 0x4080


def pin_f16_tie_by_hand():
    # 1 + 2^-11 is halfway between 1 and 1 + 2^-10: ties to the even 1.0
    got = AC.accumulate_gradient(np.array([1.0], np.float16), np.array([2.0 ** -11], np.float16), True)
    assert got[0] == np.float16(1.0)
    got = AC.accumulate_gradient(np.array([1.0 + 2.0 ** -10], np.float16), np.array([2.0 ** -11], np.float16), True)
    assert got[0] == np.float16(1.0 + 2.0 ** -9)


def pin_copy_mode_and_identities():
    held, inc = random_bf16(500), random_bf16(500)
    assert np.array_equal(AC.accumulate_gradient(held, inc, False), inc)
    zeros = np.zeros(500, np.uint16)
    assert np.array_equal(AC.accumulate_gradient(held, zeros, True), held)
    assert np.array_equal(AC.accumulate_gradient(zeros, inc, True), inc)
    f = RNG.standard_normal(100).astype(np.float32)
    assert np.array_equal(AC.accumulate_gradient(f, np.zeros_like(f), True), f)


def pin_fused_statistics_are_the_norm_of_the_new_gradients():
    held = [random_bf16(n, -8, 2) for n in (7, 130, 64)]
    inc = [random_bf16(n, -8, 2) for n in (7, 130, 64)]
    new = [AC.accumulate_gradient(h, i, True) for h, i in zip(held, inc)]
    owned = [True, False, True]
    s = oracle.normalized_sumsq(new, owned, 4.0)
    brute = sum(float(bf16_value(b)) ** 2 for k, g in enumerate(new) if owned[k] for b in g) / 16.0
    assert math.isclose(s, brute, rel_tol=1e-13)


PINS = [pin_bf16_exact_rounding_random_pairs, pin_f16_exact_rounding_random_pairs,
        pin_fp32_exact_rounding_random_pairs, pin_bf16_ties_by_hand, pin_f16_tie_by_hand,
        pin_copy_mode_and_identities, pin_fused_statistics_are_the_norm_of_the_new_gradients]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_accumulate_pin(pin):
    pin()


def _truncate(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _half_up(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x8000) >> 16).astype(np.uint16)


def _widen_in_fp64(g):
    return AC._REAL_WIDEN(g).astype(np.float64)


def _ignore_held(held, incoming, accumulate):
    return incoming.copy()


AC._REAL_WIDEN = AC._widen32
MUTANTS = {
    "bf16_truncates": ("round_to_bf16_bits", _truncate),
    "bf16_half_up": ("round_to_bf16_bits", _half_up),
    "sum_in_fp64": ("_widen32", _widen_in_fp64),
    "held_ignored": ("accumulate_gradient", _ignore_held),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_accumulate_mutants_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(AC, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
