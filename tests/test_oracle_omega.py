"""Pins of the oracle's Elias omega code against the textbook code.

The page "QSGD ... with Elias Coding" (definition paragraph and the Elias-coding
claim) names Elias recursive coding of gaps and levels. The oracle's codeword
builder and its decoder are checked against textbook codewords, the Kraft sum,
and prefix-freeness.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "elias_omega_codewords.txt")


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((int(parts[0]), "".join(parts[1:])))
    return rows


def test_textbook_codewords():
    rows = _golden()
    assert len(rows) >= 20
    for N, code in rows:
        assert oracle.omega_codeword(N) == code, N
        assert oracle.omega_length(N) == len(code), N


def test_length_matches_codeword_everywhere():
    rng = np.random.default_rng(7)
    Ns = list(range(1, 5000)) + [int(x) for x in rng.integers(1, 2**63, size=2000, dtype=np.uint64)]
    for N in Ns:
        assert len(oracle.omega_codeword(N)) == oracle.omega_length(N)


def test_prefix_free_and_kraft():
    # every codeword ends in 0 and no codeword is a prefix of another (N < 2^12);
    # the Kraft sum over all N is at most 1 (here: the partial sum stays below 1)
    codes = [oracle.omega_codeword(N) for N in range(1, 4097)]
    assert all(c.endswith("0") for c in codes)
    s = sorted(codes)
    for a, b in zip(s, s[1:]):
        assert not b.startswith(a), (a, b)
    kraft = sum(2.0 ** -len(c) for c in codes)
    assert kraft < 1.0


def test_length_growth_is_log_plus_loglog():
    # the Elias-coding claim: log2(k) + O(log log k) bits; concretely
    # L(N) <= log2(N) + 2 log2(log2(N) + 1) + 3 for all N >= 2 here
    for N in [2, 3, 10, 100, 10**4, 10**6, 2**31, 2**40, 2**63 - 1]:
        L = oracle.omega_length(N)
        lg = np.log2(N)
        assert L <= lg + 2 * np.log2(lg + 1) + 3, (N, L)
        assert L >= lg + 1
