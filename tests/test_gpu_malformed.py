"""Decoding malformed streams on the GPU (through the C ABI).

The library promises that a malformed stream gives unspecified output but that
no kernel reads or writes outside the caller's buffers. Checked here:
  * a stream whose records in one bucket are overwritten with random bits (and,
    in another bucket, whose norm is) still decodes every other bucket exactly
    as the oracle decodes the intact stream. This holds where a bucket's records
    only ever reach that bucket's own outputs: one bucket per wave group
    (d = 4096, the level bytes staged in LDS), and the per-lane writer path
    (s > 127), whose writer is clamped to the bucket;
  * random words with random bucket lengths (empty buckets, buckets shorter than
    the 32-bit norm, and payloads that stage in LDS, across the stage and the
    level buffer, or stay in global memory) decode twice to the same bits, and
    guard elements on both sides of the output are left alone.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_sgd_amd as q
from quantized_sgd_amd import workloads as wl
from tests.parity import to_dev

pytestmark = pytest.mark.gpu

GUARD = 1024
SENTINEL = np.float32(-1234.5)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


def _bits(words):
    """Stream bits as a uint8 array (bit t is bit 63 - t % 64 of word t // 64)."""
    return np.unpackbits(np.asarray(words, dtype=np.uint64).byteswap().view(np.uint8))


def _words(bits):
    return np.packbits(bits).view(np.uint64).byteswap()


def _decode_guarded(words, offs, n, s, d, code):
    """Decodes into the middle of a buffer with GUARD sentinel floats on each side;
    returns (v_hat, guards intact)."""
    wd = to_dev(np.ascontiguousarray(words if len(words) else np.zeros(1, np.uint64)).view(np.int64))
    od = to_dev(np.ascontiguousarray(offs).view(np.int64))
    buf = torch.full((n + 2 * GUARD,), float(SENTINEL), dtype=torch.float32, device="cuda")
    q.decode(wd, od, n, s, d, v_hat=buf[GUARD:GUARD + n], code=code)
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    guards = np.concatenate([h[:GUARD], h[GUARD + n:]])
    return h[GUARD:GUARD + n], bool(np.all(guards.view(np.uint32) == SENTINEL.view(np.uint32)))


@pytest.mark.parametrize("n,d,s,code", [
    (6 * 4096 - 100, 4096, 64, oracle.OMEGA), (6 * 4096 - 100, 4096, 64, oracle.GAMMA),
    (7 * 2048 - 5, 2048, 1000, oracle.OMEGA),
])
def test_corrupt_bucket_leaves_the_others_exact(n, d, s, code):
    v = wl.small_gaussian(n, 71)
    bst = oracle.uniform_buckets(n, d)
    _, _, words, offs, _ = oracle.compress(v, bst, s, 5, code=code)
    rc, want = oracle.decode(words, offs, bst, s, code=code)
    assert rc == oracle.OK
    rng = np.random.default_rng(72)
    bits = _bits(words)
    bad_payload, bad_norm = 2, 4
    a, e = int(offs[bad_payload]) + 32, int(offs[bad_payload + 1])
    assert e - a > 1000
    bits[a:e] = rng.integers(0, 2, size=e - a, dtype=np.uint8)
    a = int(offs[bad_norm])
    bits[a:a + 32] = rng.integers(0, 2, size=32, dtype=np.uint8)
    bad_words = _words(bits)
    assert bad_words.size == words.size
    got, guards_ok = _decode_guarded(bad_words, offs, n, s, d, code)
    assert guards_ok
    keep = np.ones(n, dtype=bool)
    for b in (bad_payload, bad_norm):
        keep[bst[b]:bst[b + 1]] = False
    diff = np.flatnonzero(keep & (got.view(np.uint32) != want.view(np.uint32)))
    assert diff.size == 0, f"{diff.size} mismatches outside the corrupted buckets, first at {diff[:5]}"


@pytest.mark.parametrize("n,d,s,code", [
    (12 * 4096, 4096, 64, oracle.OMEGA), (12 * 4096, 4096, 64, oracle.GAMMA), (40000, 512, 8, oracle.OMEGA),
    (9999, 37, 3, oracle.OMEGA), (9 * 2048, 2048, 1000, oracle.OMEGA), (3 * 8192, 8192, 8, oracle.OMEGA),
])
def test_random_streams_decode_deterministically_in_bounds(n, d, s, code):
    rng = np.random.default_rng(n + d + s + code)
    bst = oracle.uniform_buckets(n, d)
    nb = bst.size - 1
    lens = bst[1:] - bst[:-1]
    # per bucket: empty, shorter than the norm, or 0.5 to 20 payload bits per coordinate
    kind = rng.integers(0, 6, size=nb)
    blen = np.where(kind == 0, 0, np.where(kind == 1, rng.integers(1, 32, size=nb),
                                           32 + (lens * rng.uniform(0.5, 20.0, size=nb)).astype(np.int64)))
    offs = np.zeros(nb + 1, dtype=np.uint64)
    offs[1:] = np.cumsum(blen).astype(np.uint64)
    nw = (int(offs[-1]) + 63) // 64
    words = rng.integers(0, 2**63, size=max(nw, 1), dtype=np.uint64) * np.uint64(2) + \
        rng.integers(0, 2, size=max(nw, 1), dtype=np.uint64)
    words = words[:nw]
    first, ok1 = _decode_guarded(words, offs, n, s, d, code)
    second, ok2 = _decode_guarded(words, offs, n, s, d, code)
    assert ok1 and ok2
    assert np.array_equal(first.view(np.uint32), second.view(np.uint32))
