"""Statistics of the GPU path over Philox seeds (page "QSGD (Quantized Stochastic
Gradient Descent) with Elias Coding": definition paragraph, xi_i = (l_i + 1)/s
with probability p_i, else l_i/s; claim of unbiased quantization, Lemma 3.1).

With the bucket norms fixed by the input, each seed draws every coordinate's
rounding independently, so over many seeds:
  * the frequency of rounding up at coordinate i is binomial with
    P(up) = ceil(p_i 2^24) / 2^24 (u = (w >> 8) 2^-24, round up iff u < p_i);
  * the mean decoded value approaches sgn(v_i) ||v|| (l_i + P(up)) / s, which is
    v_i up to the 2^-24 granularity of u;
  * the mean stream length approaches the exact expectation of the record
    lengths (the dynamic programme in test_oracle_stream).
Thresholds are z-scores that a correct path fails with probability far below
1e-6; the seeds are fixed, so the outcome is reproducible."""
import math

import numpy as np
import pytest
import torch

import oracle
import quantized_sgd_amd as q
from quantized_sgd_amd import workloads as wl
from tests.test_oracle_stream import expected_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


def test_rounding_mean_and_bits_over_seeds():
    n, d, s, seeds = 2048, 512, 2, 2000
    v = wl.small_gaussian(n, 61)
    vd = torch.from_numpy(v).cuda()
    bst = oracle.uniform_buckets(n, d)
    ups = np.zeros(n)
    vsum = np.zeros(n)
    bits = np.zeros(seeds)
    norms = None
    for seed in range(seeds):
        lev, nrm = q.quantize(vd, s, d, seed)
        out, nb, offs = q.encode(vd, s, d, seed)
        vh = q.decode(out, offs, n, s, d)
        lev = lev.cpu().numpy()
        if norms is None:
            norms = nrm.cpu().numpy()
            # the reading of the scaling: r = RN32(s |v| / norm), l = floor(r), p = r - l
            # (s |v| is exact in fp64 and the fp64 quotient rounds to the right fp32)
            nrm_of = np.repeat(norms.astype(np.float64), d)[:n]
            r = ((np.float64(s) * np.abs(v).astype(np.float64)) / nrm_of).astype(np.float32)
            l = np.floor(r).astype(np.int64)
            p = (r - np.float32(l)).astype(np.float64)
            pup = np.ceil(p * 2.0**24) / 2.0**24
        ups += (np.abs(lev) > l)
        vsum += vh.cpu().numpy().astype(np.float64)
        bits[seed] = int(nb.item())
    # every level is l or l + 1
    assert np.all((np.abs(lev) == l) | (np.abs(lev) == l + 1))
    # round-up frequency against P(up), coordinate by coordinate
    mid = (pup > 0.02) & (pup < 0.98)
    assert mid.sum() > 500
    z = (ups[mid] / seeds - pup[mid]) / np.sqrt(pup[mid] * (1 - pup[mid]) / seeds)
    assert np.max(np.abs(z)) < 6.0, float(np.max(np.abs(z)))
    # and in aggregate: the sum of squared z-scores is chi-square with mid.sum() degrees
    k = int(mid.sum())
    assert abs(float(np.sum(z * z)) - k) < 8 * math.sqrt(2 * k)
    assert coordinate_never_rounds_up_when_p_is_zero(ups, pup)
    # mean decoded value: the two-point model's mean and standard error
    step = np.repeat(norms.astype(np.float64) / s, d)[:n]
    want = np.sign(v) * step * (l + pup)
    se = step * np.sqrt(pup * (1 - pup) / seeds)
    assert np.all(np.abs(vsum / seeds - want) <= 6 * se + 1e-6 * step)
    # ... which is v up to the granularity of u
    assert np.all(np.abs(want - v.astype(np.float64)) <= step * 2.0**-23 + 4 * np.spacing(np.abs(v)))
    # mean stream length against its exact expectation
    eb = expected_bits(v, bst, s, norms)
    sb = bits.std() / math.sqrt(seeds)
    assert abs(bits.mean() - eb) < 6 * sb + 1e-9, (bits.mean(), eb, sb)


def coordinate_never_rounds_up_when_p_is_zero(ups, pup):
    return bool(np.all(ups[pup == 0] == 0))
