"""Pins of the oracle's Elias gamma variant (the page "QSGD (Quantized
Stochastic Gradient Descent) with Elias Coding", definition paragraph, names
"Elias recursive gamma/omega" coding for gaps and levels; the gamma code is
defined in Elias 1975). The hand-derived gamma streams live with the omega ones
in tests/golden/special_streams.json (checked by test_oracle_stream.py)."""
import math
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def golden():
    out = {}
    for line in open(os.path.join(HERE, "golden", "elias_gamma_codewords.txt")):
        if line.startswith("#") or not line.strip():
            continue
        n, zeros, body = line.split()
        out[int(n)] = ("" if zeros == "-" else zeros) + body
    return out


def test_textbook_codewords():
    for n, cw in golden().items():
        assert oracle.gamma_codeword(n) == cw, n


def test_length_is_twice_floor_log2_plus_one():
    for n in list(range(1, 5000)) + [2 ** 24 - 1, 2 ** 24, 2 ** 40 + 3]:
        L = 2 * int(math.floor(math.log2(n))) + 1
        assert oracle.gamma_length(n) == L
        if n < 5000:
            assert len(oracle.gamma_codeword(n)) == L


def test_prefix_free_and_complete():
    words = [oracle.gamma_codeword(n) for n in range(1, 2 ** 10)]
    ws = set(words)
    for w in words:
        for cut in range(1, len(w)):
            assert w[:cut] not in ws
    # the codewords of 1 .. 2^m - 1 have Kraft sum 1 - 2^-m exactly: the code is complete
    for m in range(1, 11):
        kraft = sum(2.0 ** -len(w) for w in words[: 2 ** m - 1])
        assert kraft == 1.0 - 2.0 ** -m


@pytest.mark.parametrize("n,d,s,seed", [(4096, 4096, 4, 1), (1000, 7, 3, 2), (5000, 512, 16, 3),
                                        (3000, 1, 5, 4), (4097, 64, 1 << 20, 7)])
def test_round_trip(n, d, s, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(n).astype(np.float32)
    bst = oracle.uniform_buckets(n, d)
    lev, nrm, words, offs, nbits = oracle.compress(v, bst, s, seed, code=oracle.GAMMA)
    rc, vh = oracle.decode(words, offs, bst, s, oracle.GAMMA)
    assert rc == oracle.OK
    assert np.array_equal(vh, oracle.dequantize(lev, nrm, bst, s))
    # the same levels coded with omega: bit counts differ exactly by the codeword lengths
    _, _, nbits_o = oracle.encode(lev, nrm, bst, s, oracle.OMEGA)
    delta = 0
    for b in range(len(bst) - 1):
        lo, hi = int(bst[b]), int(bst[b + 1])
        prev = -1
        for j in np.flatnonzero(lev[lo:hi]):
            k = abs(int(lev[lo + j]))
            delta += oracle.gamma_length(int(j - prev)) - oracle.omega_length(int(j - prev))
            delta += oracle.gamma_length(k) - oracle.omega_length(k)
            prev = j
    assert nbits - nbits_o == delta


def test_omega_stream_does_not_decode_as_gamma():
    v = np.random.default_rng(9).standard_normal(512).astype(np.float32)
    bst = oracle.uniform_buckets(512, 512)
    lev, nrm, words, offs, _ = oracle.compress(v, bst, 16, 1)
    rc, vh = oracle.decode(words, offs, bst, 16, oracle.GAMMA)
    assert rc != oracle.OK or not np.array_equal(vh, oracle.dequantize(lev, nrm, bst, 16))
