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
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle

U24 = 1 << 24


def rn32(q: Fraction) -> float:
    """The binary32 value nearest to q (ties to even), by integer arithmetic."""
    if q == 0:
        return 0.0
    neg = q < 0
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    quantum = max(e, -126) - 23        # exponent of the spacing at q (subnormals: 2^-149)
    scaled = q / Fraction(2) ** quantum
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = float(Fraction(n) * Fraction(2) ** quantum)
    assert float(np.float32(val)) == val  # representable
    return -val if neg else val


def f32(x) -> float:
    return float(np.float32(x))


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


def ratio_ties(s: int, count: int, seed: int):
    """(a, norm) with s a / norm exactly an fp32 midpoint (a 25-bit odd
    significand). With s = sigma 2^es, a = alpha 2^ea and norm = nu 2^en (odd
    sigma, alpha, nu), that needs sigma alpha = mu nu with mu odd in
    (2^24, 2^25), hence nu < sigma: take alpha = nu beta, mu = sigma beta."""
    sigma = s >> ((s & -s).bit_length() - 1)
    rnd = random.Random(seed)
    out = []
    nus = [nu for nu in range(1, sigma, 2)]
    assert nus, "a power-of-two s has no ratio ties in the normal range"
    while len(out) < count:
        nu = rnd.choice(nus)
        lo = (1 << 24) // sigma + 1
        hi = min((1 << 25) // sigma, ((1 << 24) - 1) // nu)
        if lo > hi:
            continue
        beta = rnd.randrange(lo, hi + 1) | 1
        if beta > hi or nu * beta >= 1 << 24:
            continue
        alpha = nu * beta
        j = rnd.randrange(-3, max(1, s.bit_length() - 1))   # r in [2^j, 2^(j+1))
        es = (s & -s).bit_length() - 1
        ea = j - 24 - es
        norm_exp = rnd.randrange(-3, 4)
        a = math.ldexp(alpha, ea + norm_exp)
        norm = math.ldexp(nu, norm_exp)
        if not (0 < a <= norm) or f32(a) != a or f32(norm) != norm:
            continue
        q = Fraction(s) * Fraction(a) / Fraction(norm)
        m = q / Fraction(2) ** (math.floor(math.log2(q)) - 24)
        assert m.denominator == 1 and m.numerator % 2 == 1  # an exact midpoint
        if q > s:
            continue
        out.append((a, norm))
    return out


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


def dequant_ties(s: int, count: int, seed: int):
    """(norm, k) with norm k / s exactly an fp32 midpoint: nu kappa = mu sigma
    (odd parts) with mu odd in (2^24, 2^25), hence kappa > sigma."""
    es = (s & -s).bit_length() - 1
    sigma = s >> es
    rnd = random.Random(seed)
    kappas = [kp for kp in range(sigma + 2, s + 1, 2)]
    assert kappas, "no dequantization ties for this s"
    out = []
    while len(out) < count:
        kappa = rnd.choice(kappas)
        g = math.gcd(kappa, sigma)
        # nu = sigma / g * t, mu = kappa / g * t with t odd
        lo = ((1 << 24) * g) // kappa + 1
        hi = min(((1 << 25) * g) // kappa, ((1 << 24) - 1) * g // sigma)
        if lo > hi:
            continue
        t = rnd.randrange(lo, hi + 1) | 1
        nu, mu = sigma // g * t, kappa // g * t
        if not ((1 << 24) < mu < (1 << 25)) or nu >= 1 << 24 or t % 2 == 0:
            continue
        kmax = s // kappa
        k = kappa << rnd.randrange(0, kmax.bit_length())
        if k > s:
            continue
        norm = math.ldexp(nu, rnd.randrange(-20, 20))
        out.append((norm, k))
    return out


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
