"""Pin of the oracle's random stream against an independent Philox4x32-10.

Which uniform a coordinate draws is not on the pages (they only say "with
probability p_i"); the reading is: word (i & 3) of Philox4x32-10 (Salmon et al.,
SC'11) with key = seed and counter = i >> 2. PyTorch's host engine
(ATen/core/PhiloxRNGEngine.h, compiled here with g++) implements the same block
function independently; its offset field is the counter's words 0-1.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    torch_inc = None
    try:
        import torch
        torch_inc = os.path.join(os.path.dirname(torch.__file__), "include")
    except Exception:  # pragma: no cover
        pytest.skip("torch headers not available")
    exe = str(tmp_path_factory.mktemp("philox") / "probe")
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", torch_inc,
                    os.path.join(HERE, "pins", "torch_philox_probe.cpp"), "-o", exe],
                   check=True)

    def run(pairs):
        inp = "".join(f"{s} {i}\n" for s, i in pairs)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True)
        return [int(x) for x in out.stdout.split()]
    return run


def test_words_match_torch_engine(probe):
    rng = np.random.default_rng(11)
    pairs = []
    for seed in [0, 1, 2**32 - 1, 2**32, 0xDEADBEEFCAFEF00D, int(rng.integers(0, 2**63))]:
        idx = [0, 1, 2, 3, 4, 5, 7, 8, 1023, 2**32 - 1, 2**32, 2**34 + 3, 2**40 + 1]
        idx += [int(x) for x in rng.integers(0, 2**45, size=40)]
        pairs += [(seed, i) for i in idx]
    want = probe(pairs)
    got = [oracle.random_word(s, i) for s, i in pairs]
    assert got == want


def test_bulk_words_match_single(probe):
    words = oracle.random_words(5, 1000, 64)
    want = probe([(5, 1000 + t) for t in range(64)])
    assert list(words) == want


def test_block_function_words_are_the_stream():
    # block (i >> 2) of the raw block function holds words i & 3
    seed, blk = 0x0123456789ABCDEF, 77
    out = oracle.philox4x32_10([blk, 0, 0, 0], [seed & 0xFFFFFFFF, seed >> 32])
    assert [oracle.random_word(seed, 4 * blk + t) for t in range(4)] == list(out)
