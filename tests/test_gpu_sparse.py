"""GPU parity of plain decodes of sparse streams: units of 64 consecutive buckets
whose stream fits the decoder's stage and whose payloads are at most 1024 bits
each are decoded a lane per bucket, in windows of 16 coordinates per bucket that
the wave stores whole (quads shared by neighbouring buckets element by element);
other units take the team decode. Page "QSGD (Quantized Stochastic Gradient
Descent) with Elias Coding", encoding paragraph: a bucket's record stream is
parsed from its norm on, and coordinates without a record decode to zero.

The inputs are mostly tiny values with a few large ones per bucket (few nonzero
levels at s = 1, 2), a heavy-tailed Student-t draw like the 2^28-coordinate
workload, and mixes of dense and sparse stretches, so that both kinds of unit
occur; the host recomputes which units qualify from the oracle's offsets and
checks that the case exercises what it is meant to.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_sgd_amd as q
from tests.parity import check_parity

pytestmark = pytest.mark.gpu

UNIT = 64
MAX_BITS = 1024
STAGE_WORDS = 320


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


def solo_units(offs):
    """Units of 64 buckets the decoder takes a lane per bucket, and the others
    (none at all where the stream averages more than 320 bits per bucket)."""
    offs = np.asarray(offs, dtype=np.uint64)
    nb = offs.size - 1
    total_words = (int(offs[-1]) + 63) // 64
    if int(offs[-1]) > nb * (STAGE_WORDS * 64 // UNIT):
        return 0, (nb + UNIT - 1) // UNIT
    yes = no = 0
    for u0 in range(0, nb, UNIT):
        u1 = min(u0 + UNIT, nb)
        a0, e1 = int(offs[u0]), int(offs[u1])
        w0, w1 = a0 // 64, min((e1 + 63) // 64, total_words)
        lens = np.diff(offs[u0:u1 + 1].astype(np.int64))
        ok = e1 >= a0 and (w1 <= w0 or w1 - w0 <= STAGE_WORDS) and bool(np.all((lens >= 0) & (lens <= MAX_BITS)))
        yes += ok
        no += not ok
    return yes, no


def sparse_vector(n, seed, big_per=300):
    """Tiny N(0,1e-6) values with a value of size ~1 about every big_per coordinates."""
    rng = np.random.default_rng(seed)
    v = (1e-6 * rng.standard_normal(n)).astype(np.float32)
    idx = rng.choice(n, size=max(1, n // big_per), replace=False)
    v[idx] = rng.standard_normal(idx.size).astype(np.float32)
    return v


def one_big_per_bucket(n, d, seed):
    """Tiny N(0,1e-6) values and one value of size ~1 in every bucket of d: at
    s = 4 about one nonzero level per bucket."""
    rng = np.random.default_rng(seed)
    v = (1e-6 * rng.standard_normal(n)).astype(np.float32)
    starts = np.arange(0, n, d)
    pos = starts + rng.integers(0, d, size=starts.size)
    pos = np.minimum(pos, n - 1)
    v[pos] = (1.0 + rng.random(pos.size)).astype(np.float32)
    return v


def tuned_d_gate(d):
    # decode groups of 4096 // d buckets (at most 64); the sparse units need 8 or
    # more buckets per group and 64 divisible by that count
    tpw = max(1, min(64, 4096 // d))
    return tpw >= 8 and UNIT % tpw == 0


@pytest.mark.parametrize("n,d,s,code,seed", [
    (UNIT * 512 * 3 + 1234, 512, 1, oracle.OMEGA, 1),
    (UNIT * 512 * 2 + 7, 512, 2, oracle.GAMMA, 2),
    (UNIT * 64 * 9 + 63, 64, 1, oracle.OMEGA, 3),
    (UNIT * 37 * 11 + 5, 37, 1, oracle.OMEGA, 4),
    (UNIT * 256 * 4, 256, 3, oracle.OMEGA, 5),
])
def test_sparse_units_decode_exactly(n, d, s, code, seed):
    assert tuned_d_gate(d)
    v = sparse_vector(n, seed)
    g, _ = check_parity(v, s, d, seed, code=code)
    yes, no = solo_units(g["offsets"])
    print(f"n={n} d={d} s={s} code={code}: {yes} sparse units, {no} others", flush=True)
    assert yes > 0


def test_heavy_tailed_like_the_large_workload():
    # the 2^28-coordinate workload's recipe (Student-t nu = 3, scaled 1e-3; d = 512, s = 1) at 2^20
    rng = np.random.Generator(np.random.PCG64(4))
    v = (1e-3 * rng.standard_t(3, size=1 << 20)).astype(np.float32)
    g, _ = check_parity(v, 1, 512, 1)
    yes, no = solo_units(g["offsets"])
    print(f"heavy tail: {yes} sparse units, {no} others", flush=True)
    assert yes > 0


def test_mixed_dense_and_sparse_units():
    # a dense Gaussian unit (too long for the stage) after every three sparse
    # ones, ragged stretch lengths: the stream averages few enough bits per
    # bucket that the decoder looks for sparse units
    d, s = 512, 4
    parts = []
    rng = np.random.default_rng(8)
    for i in range(8):
        if i % 4 == 0:
            parts.append(rng.standard_normal(UNIT * d + 100 * i).astype(np.float32))
        else:
            parts.append(one_big_per_bucket(UNIT * d, d, 10 + i))
    v = np.concatenate(parts)
    g, _ = check_parity(v, s, d, 9)
    yes, no = solo_units(g["offsets"])
    print(f"mixed: {yes} sparse units, {no} others", flush=True)
    assert yes > 0 and no > 0


def test_sparse_ragged_batch():
    rng = np.random.default_rng(11)
    seg = [int(x) for x in rng.integers(1, 60000, size=12)] + [0, 513, 64 * 512]
    n = int(sum(seg))
    v = sparse_vector(n, 12, 500)
    g, _ = check_parity(v, 2, 512, 13, seg_len=seg)
    yes, no = solo_units(g["offsets"])
    print(f"ragged: {yes} sparse units, {no} others", flush=True)
    assert yes > 0


def test_decode_into_unaligned_unit_ends():
    # n not a multiple of 4 and d odd: units start and end inside 16-byte quads
    n, d, s = UNIT * 37 * 3 + 3, 37, 1
    v = sparse_vector(n, 14, 50)
    g, _ = check_parity(v, s, d, 15)
    yes, _ = solo_units(g["offsets"])
    assert yes > 0
