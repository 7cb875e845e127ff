"""Exact-arithmetic helpers for tests of the two roundings of the method
(page "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding",
definition paragraph: the ratio s|v_i|/||v|| and the value ||v|| k_i / s, each
read as the binary32 value nearest to the exact quotient, ties to even).

rn32 rounds a Python Fraction by integer arithmetic. ratio_ties and
dequant_ties construct operands whose exact quotient is an fp32 midpoint (a
25-bit odd significand), where a quotient evaluated through an inexact fp64
factor can round the wrong way. Nothing here calls the oracle or the library.
"""
import math
import random
from fractions import Fraction

import numpy as np

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


def dequant_ties(s: int, count: int, seed: int, inexact_quotient: bool = False):
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
        if inexact_quotient and nu % sigma == 0:
            continue
        kmax = s // kappa
        k = kappa << rnd.randrange(0, kmax.bit_length())
        if k > s:
            continue
        norm = math.ldexp(nu, rnd.randrange(-20, 20))
        out.append((norm, k))
    return out




def targeted_ratio_tie(s: int, N: float, U: int, j: int):
    """|v| = a such that r = s a / N is an exact fp32 midpoint in [2^j, 2^(j+1))
    whose two fp32 neighbours give different levels for the uniform draw
    u = U 2^-24: the fractional parts of the neighbours, times 2^24, are
    t 2^j -+ 2^(j-1), so U must lie in [t 2^j - 2^(j-1), t 2^j + 2^(j-1)) (for
    j = 0: U = t).
    The midpoint is mu 2^(j-24) with mu odd in (2^24, 2^25), mu = t mod 2^(24-j)
    and sigma | mu (sigma: the odd part of s); a = (N's odd part) mu / sigma, scaled.
    Returns None when no such a exists."""
    es = (s & -s).bit_length() - 1
    sigma = s >> es
    Nf = Fraction(N)
    nu, pN = Nf.numerator, 0
    while nu % 2 == 0:
        nu //= 2
        pN += 1
    assert Nf.denominator == 1
    t = (U + (1 << (j - 1))) >> j if j else U
    if t % 2 == 0:
        return None
    m24 = 24 - j
    mod = 1 << m24
    beta0 = (t * pow(sigma, -1, mod)) % mod
    for m in range(0, 64):
        beta = beta0 + m * mod
        mu = sigma * beta
        if mu <= 1 << 24:
            continue
        if mu >= 1 << 25:
            return None
        alpha = nu * beta
        if alpha >= 1 << 24:
            return None
        a = math.ldexp(alpha, j - 24 - es + pN)
        if f32(a) != a or a > N:
            return None
        q = Fraction(s) * Fraction(a) / Nf
        assert q == Fraction(mu) * Fraction(2) ** (j - 24)
        return a
    return None


def tie_bucket_values(s: int, d: int, words, rnd: random.Random, maxnorm: bool = False):
    """One bucket of d fp32 values whose norm N = 2 (s with odd part 3) or 6
    (otherwise) has an odd part below the odd part of s, with some coordinates
    at exact ratio midpoints whose level the uniform draw of that coordinate
    (words: the bucket's Philox words) decides differently for the two fp32
    neighbours; zeros elsewhere. L2: a balancing coordinate b makes the fp64
    sum of squares round to N, every square and partial sum being exact in
    fp64 so that the norm is the same in any summation order. maxnorm: N
    itself is a coordinate. Returns (values, N, tie positions)."""
    sigma = s >> ((s & -s).bit_length() - 1)
    assert sigma > 1, "s must not be a power of two"
    N = 2.0 if sigma == 3 else 6.0
    # midpoints in [2^j, 2^(j+1)): every residue class has one when sigma <= 2^j
    j = min((sigma - 1).bit_length(), s.bit_length() - 1)
    while True:
        order = list(range(d))
        rnd.shuffle(order)
        vals, pos = [], []
        S = Fraction(0)
        budget = Fraction(N) ** 2 * Fraction(3, 4)
        for i in order:
            if len(pos) >= 8 or len(pos) >= d - 1:
                break
            a = targeted_ratio_tie(s, N, int(words[i]) >> 8, j)
            if a is None or (not maxnorm and S + Fraction(a) ** 2 > budget):
                continue
            S += Fraction(a) ** 2
            vals.append(a if rnd.random() < 0.5 else -a)
            pos.append(i)
        if not pos:
            continue
        rest = [i for i in range(d) if i not in pos]
        if maxnorm:
            vals.append(N if rnd.random() < 0.5 else -N)
        else:
            b0 = np.float32(math.sqrt(N * N - float(S)))
            ok = None
            for t in range(0, 9):
                for sgn in (1, -1):
                    b = b0
                    for _ in range(t):
                        b = np.nextafter(b, np.float32(np.inf if sgn > 0 else 0.0), dtype=np.float32)
                    X = S + Fraction(float(b)) ** 2
                    if float(X) == X and f32(math.sqrt(float(X))) == N:
                        ok = float(b)
                        break
                if ok is not None:
                    break
            if ok is None:
                continue
            vals.append(ok)
        out = np.zeros(d, np.float32)
        out[pos + [rest[0]]] = np.asarray(vals, np.float32)
        return out, N, pos


def tie_vector(s: int, d: int, nb: int, seed: int, philox_seed: int, random_words, maxnorm: bool = False,
               every: int = 2):
    """nb buckets of d coordinates: every `every`-th one built by
    tie_bucket_values for the Philox seed philox_seed (random_words(seed,
    first, count) gives the draws), the others N(0, 1) values. Returns the
    vector and the (index, N) of each tie coordinate."""
    rnd = random.Random(seed)
    rng = np.random.default_rng(seed)
    parts, ties = [], []
    for b in range(nb):
        if b % every == 0:
            words = random_words(philox_seed, b * d, d)
            vals, N, pos = tie_bucket_values(s, d, words, rnd, maxnorm)
            parts.append(vals)
            ties += [(b * d + p, N) for p in pos]
        else:
            parts.append(rng.standard_normal(d).astype(np.float32))
    return np.concatenate(parts), ties
