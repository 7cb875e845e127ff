"""Pins of the oracle's stochastic quantizer Q_s.

Page "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding":
  * definition paragraph: l_i = floor(s|v_i|/||v||), p_i = s|v_i|/||v|| - l_i,
    xi_i = (l_i + 1)/s with probability p_i, else l_i/s; Q_s(v)_i = ||v|| sgn(v_i) xi_i.
  * claim "unbiased stochastic quantization, variance and sparsity bounds"
    (Lemma 3.1, Lemma A.5): E[Q_s(v)] = v,
    E||Q_s(v) - v||^2 = (||v||^2/s^2) sum p_i(1 - p_i) <= min(n/s^2, sqrt(n)/s) ||v||^2,
    E||Q_s(v)||_0 <= s^2 + s sqrt(n).
The expectations are computed exactly by enumerating all 2^n rounding outcomes
(forcing each outcome through the oracle with chosen uniforms) and weighting them
with the exact round-up probabilities, computed here in rational arithmetic.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle

U24_MAX = (1 << 24) - 1


def exact_norm(v):
    return math.sqrt(math.fsum(float(x) * float(x) for x in v))


def up_probability(p):
    """P(u < p) for u uniform on {0, 2^-24, ..., 1 - 2^-24}, p a Fraction."""
    return Fraction(math.ceil(p * (1 << 24)), 1 << 24)


def exact_split(v, norm, s):
    """l_i and p_i of the page's definition, in exact rational arithmetic, for the
    fp32 norm that the stream carries."""
    ls, ps = [], []
    for x in v:
        r = Fraction(s) * abs(Fraction(float(x))) / Fraction(float(norm))
        l = math.floor(r)
        ls.append(l)
        ps.append(r - l)
    return ls, ps


def enumerate_outcomes(v, s):
    """All 2^n outcomes: returns list of (probability, Q vector, levels)."""
    n = len(v)
    bst = oracle.uniform_buckets(n, n)
    _, norms = oracle.quantize(v, bst, s, seed=0)
    ls, ps = exact_split(v, norms[0], s)
    pu = [up_probability(p) for p in ps]
    outs = []
    for mask in range(1 << n):
        up = [(mask >> i) & 1 for i in range(n)]
        u24 = np.array([0 if b else U24_MAX for b in up], dtype=np.uint32)
        lev, nrm = oracle.quantize(v, bst, s, seed=0, u24=u24)
        q = oracle.dequantize(lev, nrm, bst, s)
        prob = Fraction(1)
        for i in range(n):
            prob *= pu[i] if up[i] else (1 - pu[i])
        outs.append((prob, q, lev, up))
    return outs, norms[0], ls, ps, pu


@pytest.mark.parametrize("n,s,seed", [(8, 1, 0), (10, 2, 1), (12, 4, 2), (12, 3, 3), (9, 8, 4)])
def test_enumeration_unbiased_and_variance(n, s, seed):
    v = np.random.default_rng(seed).standard_normal(n).astype(np.float32)
    outs, norm, ls, ps, pu = enumerate_outcomes(v, s)
    assert abs(float(norm) - exact_norm(v)) <= np.spacing(np.float32(norm))
    # every outcome is l_i or l_i + 1 as forced (an up-draw only when p_i > 0)
    for prob, q, lev, up in outs:
        k = np.abs(lev)
        for i in range(n):
            want = ls[i] + (1 if (up[i] and ps[i] > 0) else 0)
            assert k[i] == want
            if k[i]:
                assert np.signbit(lev[i]) == np.signbit(v[i]) or lev[i] == 0
    tot = sum(p for p, *_ in outs)
    assert tot == 1
    # E[Q] = v: exact up to the 2^-24 granularity of the uniform and fp32 rounding
    mean = np.zeros(n)
    for prob, q, *_ in outs:
        mean += float(prob) * q.astype(np.float64)
    tol = float(norm) / s * 2.0**-23 + 4 * np.spacing(np.abs(v).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(mean - v.astype(np.float64)) <= tol)
    # variance identity (Lemma 3.1) with the exact p_i, and the bound
    var = 0.0
    for prob, q, *_ in outs:
        var += float(prob) * float(np.sum((q.astype(np.float64) - v.astype(np.float64)) ** 2))
    norm2 = exact_norm(v) ** 2
    ident = norm2 / s**2 * sum(float(p * (1 - p)) for p in ps)
    assert var == pytest.approx(ident, rel=1e-5, abs=1e-9 * norm2)
    assert var <= min(n / s**2, math.sqrt(n) / s) * norm2 * (1 + 1e-6)
    # support size (Lemma A.5): E||Q||_0 <= s^2 + s sqrt(n)
    nnz = sum(float(prob) * np.count_nonzero(lev) for prob, q, lev, up in outs)
    assert nnz <= s * s + s * math.sqrt(n)
    want_nnz = sum((1.0 if l >= 1 else float(p_up)) for l, p_up in zip(ls, pu))
    assert nnz == pytest.approx(want_nnz, rel=1e-12)


def test_rounding_rule_against_independent_philox_words():
    # With an external norm equal to s (a power of two) the ratio is exactly
    # |v_i|, so p_i = frac(|v_i|) and the round-up decision is [w >> 8 < p 2^24]
    # with w the Philox word of coordinate i (pinned separately to PyTorch's engine).
    rng = np.random.default_rng(3)
    s, seed, n = 4, 99, 4096
    v = (rng.uniform(-4, 4, size=n)).astype(np.float32)
    bst = oracle.uniform_buckets(n, n)
    lev, _ = oracle.quantize(v, bst, s, seed, norms=np.array([4.0], np.float32))
    w = oracle.random_words(seed, 0, n)
    for i in range(n):
        a = Fraction(float(abs(v[i])))
        l = math.floor(a)
        p = a - l
        k = l + (1 if Fraction(int(w[i]) >> 8) < p * (1 << 24) else 0)
        assert abs(int(lev[i])) == k, i
        if k:
            assert (lev[i] < 0) == bool(np.signbit(v[i]))


def test_d1_is_exact():
    # a bucket of one coordinate has ||v|| = |v_i|, so r = s, p = 0 and the
    # dequantized value is v_i itself for every s
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(500), [1e-40, -3e-45, 3.0e38, -1.0, 0.0]]).astype(np.float32)
    bst = oracle.uniform_buckets(len(v), 1)
    for s in [1, 3, 7, 8, 64, 1000, 1 << 24]:
        lev, nrm = oracle.quantize(v, bst, s, seed=s)
        q = oracle.dequantize(lev, nrm, bst, s)
        assert np.array_equal(q.view(np.uint32)[v != 0], v.view(np.uint32)[v != 0])
        assert np.all(q[v == 0] == 0)


def test_zero_buckets_and_signed_zero():
    v = np.array([0.0, -0.0, 0.0, 0.0, 1.0, -0.0], np.float32)
    bst = oracle.uniform_buckets(6, 3)
    lev, nrm = oracle.quantize(v, bst, 4, seed=1)
    assert list(nrm) == [0.0, 1.0]
    assert list(lev) == [0, 0, 0, 0, 4, 0]


def test_monte_carlo_unbiased_over_seeds():
    # the whole path with Philox uniforms: the mean over seeds approaches v
    rng = np.random.default_rng(8)
    n, s, seeds = 64, 2, 4000
    v = rng.standard_normal(n).astype(np.float32)
    bst = oracle.uniform_buckets(n, 16)
    acc = np.zeros(n)
    acc2 = np.zeros(n)
    for seed in range(seeds):
        lev, nrm = oracle.quantize(v, bst, s, seed)
        q = oracle.dequantize(lev, nrm, bst, s).astype(np.float64)
        acc += q
        acc2 += q * q
    mean = acc / seeds
    # the standard error of the mean from the page's model: Q_i takes the two
    # values l_i and l_i + 1 (times ||v||/s) with probabilities 1 - p_i and p_i
    _, nrm = oracle.quantize(v, bst, s, 0)
    norm_of = np.repeat(nrm.astype(np.float64), 16)
    r = s * np.abs(v.astype(np.float64)) / norm_of
    p = r - np.floor(r)
    sd = norm_of / s * np.sqrt(p * (1 - p) / seeds)
    floor = 4 * np.spacing(np.abs(v)).astype(np.float64) + norm_of / s * 2.0**-23
    z = np.abs(mean - v) / np.maximum(sd, floor)
    assert np.all(z < 5.0), (z.max(), int(np.argmax(z)))


def test_invalid_arguments_rejected():
    v = np.ones(4, np.float32)
    bst = oracle.uniform_buckets(4, 4)
    with pytest.raises(ValueError):
        oracle.quantize(v, bst, 0, 1)
    with pytest.raises(ValueError):
        oracle.quantize(np.array([1, np.inf, 0, 0], np.float32), bst, 4, 1)


def test_ragged_buckets_restart_per_segment():
    b = oracle.ragged_buckets([5, 0, 3, 8], 4)
    assert list(b) == [0, 4, 5, 8, 12, 16]
    assert list(oracle.uniform_buckets(10, 4)) == [0, 4, 8, 10]
    assert list(oracle.uniform_buckets(3, 8)) == [0, 3]
