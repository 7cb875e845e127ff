"""Pins of the oracle's max-norm scaling, the reading of the heuristic variant
that page "NUQSGD: Provably Communication-efficient Data-parallel SGD via
Nonuniform Quantization" (abstract) names QSGDinf: the quantizer of the page
"QSGD (Quantized Stochastic Gradient Descent) with Elias Coding" (definition
paragraph) with max_i |v_i| in place of ||v||_2. Unbiasedness holds for any scale
at least max|v_i|, so the exact enumeration of all 2^n rounding outcomes must
give E[Q] = v, and the variance must be (scale/s)^2 sum p_i (1 - p_i)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.test_oracle_quantize import U24_MAX, exact_split, up_probability


def test_max_norms_are_numpy_max_abs():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(10007) * 10.0 ** rng.integers(-30, 30, 10007)).astype(np.float32)
    v[::13] = -0.0
    for d in (1, 7, 512, 4096):
        bst = oracle.uniform_buckets(v.size, d)
        got = oracle.bucket_max_norms(v, bst)
        want = np.array([np.max(np.abs(v[bst[b]:bst[b + 1]])) for b in range(len(bst) - 1)], np.float32)
        assert np.array_equal(got, want)


@pytest.mark.parametrize("n,s,seed", [(8, 1, 0), (10, 2, 1), (12, 4, 2), (11, 3, 3)])
def test_enumeration_unbiased_and_variance(n, s, seed):
    v = np.random.default_rng(seed).standard_normal(n).astype(np.float32)
    bst = oracle.uniform_buckets(n, n)
    norm = oracle.bucket_max_norms(v, bst)
    ls, ps = exact_split(v, norm[0], s)
    pu = [up_probability(p) for p in ps]
    mean = [Fraction(0)] * n
    second = Fraction(0)
    for mask in range(1 << n):
        up = [(mask >> i) & 1 for i in range(n)]
        u24 = np.array([0 if b else U24_MAX for b in up], dtype=np.uint32)
        lev, nrm = oracle.quantize(v, bst, s, seed=0, norms=norm, u24=u24)
        q = oracle.dequantize(lev, nrm, bst, s)
        prob = Fraction(1)
        for i in range(n):
            prob *= pu[i] if up[i] else (1 - pu[i])
        for i in range(n):
            mean[i] += prob * Fraction(float(q[i]))
        second += prob * sum((Fraction(float(q[i])) - Fraction(float(v[i]))) ** 2 for i in range(n))
    # E[Q] = v up to the fp32 rounding of the dequantized values and the 2^-24
    # granularity of the uniforms: within a few ulps of the scale
    scale = Fraction(float(norm[0]))
    for i in range(n):
        assert abs(mean[i] - Fraction(float(v[i]))) <= scale * Fraction(1, 1 << 20)
    var = (scale / s) ** 2 * sum(p * (1 - p) for p in ps)
    assert abs(second - var) <= scale * scale * Fraction(1, 1 << 18)


def test_largest_coordinates_get_level_s():
    rng = np.random.default_rng(4)
    for s in (1, 3, 64, 1000):
        v = rng.standard_normal(4096).astype(np.float32)
        bst = oracle.uniform_buckets(v.size, 512)
        mx = oracle.bucket_max_norms(v, bst)
        for seed in range(3):
            lev, nrm = oracle.quantize(v, bst, s, seed, norms=mx)
            assert np.all(np.abs(lev) <= s)
            for b in range(len(bst) - 1):
                seg = slice(int(bst[b]), int(bst[b + 1]))
                top = np.abs(v[seg]) == mx[b]
                assert np.all(np.abs(lev[seg][top]) == s)


def test_single_nonzero_bucket_matches_l2():
    # one non-zero coordinate per bucket: max|v| = ||v||_2, both variants agree
    v = np.zeros(2048, np.float32)
    v[::256] = np.linspace(-3, 5, 8).astype(np.float32)
    bst = oracle.uniform_buckets(v.size, 256)
    a = oracle.quantize(v, bst, 16, 5, norms=oracle.bucket_max_norms(v, bst))
    b = oracle.quantize(v, bst, 16, 5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
