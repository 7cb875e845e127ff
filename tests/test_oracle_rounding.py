"""Pins of the oracle's two roundings against exact rational arithmetic.

Page "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding",
definition paragraph: l_i = floor(s|v_i|/||v||), p_i = s|v_i|/||v|| - l_i, and
Q_s(v)_i = ||v|| sgn(v_i) k_i / s. The pages fix no precision; the reading is
that both quotients are the binary32 values nearest to the exact real ones
(ties to even):
  * the ratio r_i = RN32(s |v_i| / ||v||), then l = floor(r), p = r - l, and the
    coordinate rounds up iff u < p with u = u24 2^-24;
  * the magnitude m = RN32(||v|| k / s).
Everything expected here comes from `rn32`, which rounds a Python Fraction by
integer arithmetic, never from the oracle. The cases include exact fp32
midpoints ("ties"), which a quotient evaluated through an inexact fp64
reciprocal or scale factor can round the wrong way.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.ties import U24, dequant_ties, f32, ratio_ties, rn32


def test_rn32_agrees_with_numpy_on_doubles():
    # numpy's float64 -> float32 cast rounds to nearest even; on exact doubles
    # (not ties of the double itself) rn32 must give the same value
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000),
                         [1.5 * 2.0**-149, 2.0**-150, 3 * 2.0**-150, 1 + 2.0**-24, 1 + 3 * 2.0**-24]])
    for x in xs:
        assert rn32(Fraction(float(x))) == f32(x), x


def exact_ratio_decision(a: float, norm: float, s: int, u24: int) -> int:
    """k for |v| = a by the definition: r = RN32(s a / norm), round up iff u < p."""
    r = Fraction(rn32(Fraction(s) * Fraction(a) / Fraction(norm)))
    l = math.floor(r)
    p = r - l
    return l + (1 if Fraction(u24, U24) < p else 0)


def oracle_levels(a_vals, norm, s, u24s):
    v = np.asarray(a_vals, np.float32)
    bst = oracle.uniform_buckets(v.size, v.size)
    lev, _ = oracle.quantize(v, bst, s, seed=0, norms=np.array([norm], np.float32),
                             u24=np.asarray(u24s, np.uint32))
    return np.abs(lev)


def probe_u24s(a: float, norm: float, s: int):
    """Uniforms one step either side of the exact p of the correctly rounded
    ratio, and the extremes: they tell apart ratios one fp32 ulp apart."""
    r = Fraction(rn32(Fraction(s) * Fraction(a) / Fraction(norm)))
    p = r - math.floor(r)
    P = math.ceil(p * U24)
    return sorted({0, max(P - 1, 0), min(P, U24 - 1), U24 - 1})


@pytest.mark.parametrize("s", [3, 100, 1000])
def test_ratio_on_constructed_ties(s):
    cases = ratio_ties(s, 60, seed=s)
    old_form_wrong = 0
    for a, norm in cases:
        u24s = probe_u24s(a, norm, s)
        got = oracle_levels([a] * len(u24s), norm, s, u24s)
        want = [exact_ratio_decision(a, norm, s, u) for u in u24s]
        assert list(got) == want, (a, norm, s, u24s)
        exact = rn32(Fraction(s) * Fraction(a) / Fraction(norm))
        if f32(np.float64(a) * (np.float64(s) / np.float64(norm))) != exact:
            old_form_wrong += 1
    if s != 3:
        # ties whose quotient an inexact fp64 scale factor rounds the wrong
        # way exist among the cases (for s = 3 the factor 3 / 2^e is exact)
        assert old_form_wrong > 0


@pytest.mark.parametrize("s", [1, 3, 5, 7, 12, 100, 1000, 12345, (1 << 24) - 1])
def test_ratio_decision_at_one_ulp_of_u(s):
    rng = np.random.default_rng(s)
    n = 48
    for trial in range(6):
        norm = f32(10.0 ** rng.uniform(-30, 30))
        a_vals = [f32(norm * x) for x in rng.uniform(0, 1, n)]
        a_vals[0] = norm                    # r = s exactly
        a_vals[1] = f32(norm * 2.0**-20)
        for a in a_vals:
            u24s = probe_u24s(a, norm, s)
            got = oracle_levels([a] * len(u24s), norm, s, u24s)
            want = [exact_ratio_decision(a, norm, s, u) for u in u24s]
            assert list(got) == want, (a, norm, s, u24s)


def test_ratio_tiny_results():
    # quotients in the fp32 subnormal range, and exactly half the smallest
    # subnormal (2^-150, which rounds to 0): a draw of u = 0 rounds up iff p > 0
    s = 1
    cases = [(2.0**-149, 2.0), (2.0**-149, 4.0), (3 * 2.0**-149, 2.0), (2.0**-148, 3.0),
             (5 * 2.0**-149, 10.0), (2.0**-149, 1.5)]
    for a, norm in cases:
        for u in (0, 1):
            got = oracle_levels([a], norm, s, [u])
            assert int(got[0]) == exact_ratio_decision(a, norm, s, u), (a, norm, u)
    # 2^-150 exactly: p = 0, never up
    assert int(oracle_levels([2.0**-149], 2.0, 1, [0])[0]) == 0
    assert int(oracle_levels([3 * 2.0**-149], 2.0, 1, [0])[0]) == 1


def oracle_magnitudes(norm: float, s: int, ks):
    lev = np.asarray(ks, np.int32)
    bst = oracle.uniform_buckets(lev.size, lev.size)
    return oracle.dequantize(lev, np.array([norm], np.float32), bst, s)


def test_dequantize_known_tie():
    # 71116920 * 85 / 100 = 60449382 exactly, halfway between the fp32 values
    # 60449380 and 60449384; ties to even gives 60449384
    assert rn32(Fraction(71116920 * 85, 100)) == 60449384.0
    assert float(oracle_magnitudes(71116920.0, 100, [85])[0]) == 60449384.0
    assert float(oracle_magnitudes(71116920.0, 100, [-85])[0]) == -60449384.0


@pytest.mark.parametrize("s", [100, 1000, 12])
def test_dequantize_on_constructed_ties(s):
    cases = dequant_ties(s, 200, seed=s)
    old_form_wrong = 0
    for norm, k in cases:
        q = Fraction(norm) * k / s
        m = q / Fraction(2) ** (math.floor(math.log2(q)) - 24)
        assert m.denominator == 1 and m.numerator % 2 == 1
        want = rn32(q)
        got = float(oracle_magnitudes(norm, s, [k])[0])
        assert got == want, (norm, k, s)
        if f32(k * (np.float64(norm) / s)) != want:
            old_form_wrong += 1
    if s in (100, 1000):
        # ties that k times an inexact fp64 norm / s rounds the wrong way
        assert old_form_wrong > 0


@pytest.mark.parametrize("s", [3, 5, 7, 100, 1000, 12345, (1 << 24) - 1])
def test_dequantize_random_against_exact(s):
    rng = np.random.default_rng(1000 + s)
    norms = (10.0 ** rng.uniform(-40, 38, 400)).astype(np.float32)
    for norm in norms:
        ks = rng.integers(1, s + 1, 8)
        got = oracle_magnitudes(float(norm), s, ks)
        for k, g in zip(ks, got):
            assert float(g) == rn32(Fraction(float(norm)) * int(k) / s), (float(norm), int(k), s)
