"""GPU parity on exact fp32 midpoints ("ties") of the method's two quotients.

Page "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding",
definition paragraph: the ratio s|v_i|/||v|| and the value ||v|| k_i / s. Both are
read as the binary32 value nearest to the exact quotient, ties to even. The
inputs below are built so that these quotients are exact midpoints where it
matters:
  * encode: coordinates whose ratio is a midpoint and whose Philox draw decides
    the level differently for the two fp32 neighbours, in buckets whose norm
    (L2 or max-norm) is 2 or 6, at s = 3, 100 and 1000, through both encoders
    and the ragged path;
  * decode: streams written by the oracle whose (norm, k) pairs give
    magnitudes at midpoints, at s = 100 (levels staged in LDS) and s = 1000
    (each lane writes its outputs), also accumulated.
Each case also checks on the host that rounding through an fp64 scale factor
would get some of these cases wrong, so the cases can tell the two apart.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import quantized_sgd_amd as q
from tests.parity import check_parity, to_dev
from tests.ties import dequant_ties, f32, rn32, tie_vector

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


def scale_factor_decisions_wrong(v, ties, s, seed):
    """Ties whose level the rounding RN32(|v| RN64(s / N)) decides wrongly."""
    w = oracle.random_words(seed, 0, v.size)
    wrong = 0
    for i, N in ties:
        a = abs(float(v[i]))

        def dec(r):
            l = int(r)
            return l + (1 if Fraction(int(w[i]) >> 8, 1 << 24) < r - l else 0)
        r = Fraction(rn32(Fraction(s) * Fraction(a) / Fraction(N)))
        rold = Fraction(f32(np.float64(a) * (np.float64(s) / np.float64(N))))
        wrong += dec(rold) != dec(r)
    return wrong


@pytest.mark.parametrize("s,d,maxnorm,seed", [
    (3, 64, False, 1),      # aligned encoder (d a power of two, s <= 64)
    (3, 64, True, 2),
    (3, 100, False, 3),     # general encoder
    (100, 64, False, 4),
    (100, 64, True, 5),
    (1000, 128, False, 6),
    (1000, 96, True, 7),
])
def test_encode_ratio_ties(s, d, maxnorm, seed):
    nb = 300
    v, ties = tie_vector(s, d, nb, seed, seed, oracle.random_words, maxnorm=maxnorm)
    print(f"ratio ties s={s} d={d} maxnorm={maxnorm} ties={len(ties)}", flush=True)
    g, _ = check_parity(v, s, d, seed, norm=q.MAXNORM if maxnorm else q.L2)
    # the tie buckets kept their norm N on the GPU, so the ties were exercised
    assert all(float(g["norms"][i // d]) == N for i, N in ties)
    if s != 3:
        assert scale_factor_decisions_wrong(v, ties, s, seed) > 0


def test_encode_ratio_ties_ragged():
    s, d, seed = 100, 64, 9
    v, ties = tie_vector(s, d, 200, seed, seed, oracle.random_words)
    seg = [64 * 37, 64 * 100, 64 * 63]        # segment starts on bucket boundaries
    print(f"ragged ratio ties ties={len(ties)}", flush=True)
    g, _ = check_parity(v, s, d, seed, seg_len=seg)
    assert all(float(g["norms"][i // d]) == N for i, N in ties)


def tie_stream(s, d, nb, seed):
    """Levels and norms whose magnitudes norm k / s are midpoints in every
    other bucket (other coordinates random levels), plus the oracle's stream."""
    rng = np.random.default_rng(seed)
    cases = dequant_ties(s, nb, seed, inexact_quotient=True)
    n = nb * d
    levels = np.zeros(n, np.int32)
    norms = (10.0 ** rng.uniform(-3, 3, nb)).astype(np.float32)
    for b in range(nb):
        pos = rng.choice(d, size=d // 3, replace=False)
        levels[b * d + pos] = rng.integers(1, s + 1, pos.size) * rng.choice([-1, 1], pos.size)
        if b % 2 == 0:
            norm, k = cases[b]
            norms[b] = norm
            tp = rng.choice(d, size=16, replace=False)
            levels[b * d + tp] = k * rng.choice([-1, 1], 16)
    if nb > 1:
        norms[1] = np.float32(71116920.0)
        levels[d:2 * d] = 0
        levels[d + 5] = 85
        levels[d + 9] = -85
    bst = oracle.uniform_buckets(n, d)
    words, offs, nbits = oracle.encode(levels, norms, bst, s)
    want = oracle.dequantize(levels, norms, bst, s)
    old = np.zeros(n, np.float32)
    nz = levels != 0
    old[nz] = (np.abs(levels[nz]) * (np.repeat(norms, d)[nz].astype(np.float64) / s)).astype(np.float32)
    old[nz] *= np.sign(levels[nz])
    return levels, norms, bst, words, offs, want, int(np.sum(old.view(np.uint32) != want.view(np.uint32)))


@pytest.mark.parametrize("s,d", [(100, 512), (100, 4096), (1000, 256), (1000, 8192)])
def test_decode_value_ties(s, d):
    nb = 40 if d <= 512 else 48
    levels, norms, bst, words, offs, want, old_wrong = tie_stream(s, d, nb, s + d)
    print(f"value ties s={s} d={d} old_wrong={old_wrong}", flush=True)
    assert old_wrong > 0
    n = levels.size
    vh = q.decode(to_dev(words.view(np.int64)), to_dev(offs.view(np.int64)), n, s, d)
    torch.cuda.synchronize()
    assert np.array_equal(vh.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_decode_accumulate_value_ties():
    s, d, nb = 100, 512, 24
    streams, wants = [], []
    for j in range(3):
        levels, norms, bst, words, offs, want, _ = tie_stream(s, d, nb, 77 + j)
        streams.append((to_dev(words.view(np.int64)), to_dev(offs.view(np.int64))))
        wants.append((words, offs))
    n = nb * d
    acc0 = np.random.default_rng(5).standard_normal(n).astype(np.float32)
    acc = to_dev(acc0.copy())
    q.decode_accumulate([w for w, _ in streams], [o for _, o in streams], n, s, d, acc)
    torch.cuda.synchronize()
    rc, exp = oracle.decode_accumulate([(w, o) for w, o in wants], bst, s, acc0.copy())
    assert rc == oracle.OK
    assert np.array_equal(acc.cpu().numpy().view(np.uint32), exp.view(np.uint32))
