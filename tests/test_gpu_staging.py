"""GPU parity of the decoder's three ways of reading a group's stream: staged in
the wave's stream buffer (at most 320 words), staged over the stream and level
buffers together (321 to 836 words; each lane then writes its outputs
directly), or read from global memory (longer). The stream sizes per group are
taken from the oracle's bucket offsets, so every case asserts that it covers
the classes it is meant to; the boundary case hits 320, 321, 836 and 837 words
exactly. Page "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding",
definition paragraph (the coding is lossless, so the decode must equal the
dequantized levels bit for bit)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_sgd_amd as q
from tests.parity import check_parity

pytestmark = pytest.mark.gpu

STAGE, BIG = 320, 836  # stream words of a group staged in LDS, alone and with the level buffer


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


def group_words(offs, tpw=1):
    """Stream words a decoder group of tpw buckets spans (as the decoder stages them)."""
    nb = len(offs) - 1
    return np.array([((int(offs[min(nb, b0 + tpw)]) + 63) >> 6) - (int(offs[b0]) >> 6)
                     for b0 in range(0, nb, tpw)])


def oracle_offsets(v, s, d, norm):
    bst = oracle.uniform_buckets(v.size, d)
    nr = oracle.bucket_max_norms(v, bst) if norm == q.MAXNORM else None
    _, _, _, offs, _ = oracle.compress(v, bst, s, 3, norms=nr)
    return offs


def mixed_buckets(nbk, d, seed):
    """Buckets of four kinds in turn: Gaussian, constant magnitude, 90% zeros,
    Gaussian with three spikes."""
    rng = np.random.default_rng(seed)
    parts = []
    for i in range(nbk):
        z = rng.standard_normal(d)
        kind = i % 4
        if kind == 0:
            x = z
        elif kind == 1:
            x = np.sign(z) * 0.5
        elif kind == 2:
            x = z * (rng.random(d) < 0.1)
        else:
            x = z.copy()
            x[rng.integers(0, d, 3)] *= rng.uniform(2, 12)
        parts.append(x)
    return np.concatenate(parts).astype(np.float32)


@pytest.mark.parametrize("d,s,norm,classes", [
    (4096, 64, q.MAXNORM, {"lds", "big", "global"}),
    (4096, 127, q.MAXNORM, {"lds", "big", "global"}),
])
def test_staging_classes(d, s, norm, classes):
    v = mixed_buckets(24, d, 7)
    gw = group_words(oracle_offsets(v, s, d, norm))
    seen = {"lds" if w <= STAGE else "big" if w <= BIG else "global" for w in gw}
    assert classes <= seen, (sorted(gw.tolist()), seen)
    check_parity(v, s, d, 41, norm=norm)


@pytest.mark.parametrize("s", [64, 127])
def test_staging_classes_large_buckets(s):
    """Buckets of 8192 coordinates (decoded by per-lane writers; the encoder's
    tiles hold at most 4096 coordinates, so the stream is the oracle's)."""
    d = 8192
    v = mixed_buckets(8, d, 7)
    bst = oracle.uniform_buckets(v.size, d)
    lev, nrm, words, offs, _ = oracle.compress(v, bst, s, 43)
    seen = {"lds" if w <= STAGE else "big" if w <= BIG else "global" for w in group_words(offs)}
    assert {"lds", "big"} <= seen, seen
    wd = torch.from_numpy(np.concatenate([words, np.zeros(1, np.uint64)]).view(np.int64)).cuda()
    od = torch.from_numpy(offs.view(np.int64)).cuda()
    vh = q.decode(wd, od, v.size, s, d).cpu().numpy()
    want = oracle.dequantize(lev, nrm, bst, s)
    assert np.array_equal(vh.view(np.uint32), want.view(np.uint32))


def test_staging_boundaries():
    """Buckets of d = 4096 under the max-norm with s = 64 whose first m
    coordinates are +-1 and the rest 0: each of those codes as a 15-bit record
    (gap 1, sign, level 64), so m sets the group's word count. m is searched per
    bucket (given the buckets before it) to hit 320, 321, 836 and 837 words."""
    d, s = 4096, 64
    rng = np.random.default_rng(51)
    targets = [320, 321, 836, 837, 500, 836]
    v = np.zeros(0, dtype=np.float32)
    for t in targets:
        hit = None
        for m in range(max(1, (t - 2) * 64 // 15 - 8), min(d, t * 64 // 15 + 8)):
            x = np.zeros(d, dtype=np.float32)
            x[:m] = np.where(rng.random(m) < 0.5, -1.0, 1.0)
            cand = np.concatenate([v, x])
            if group_words(oracle_offsets(cand, s, d, q.MAXNORM))[-1] == t:
                hit = cand
                break
        assert hit is not None, t
        v = hit
    assert group_words(oracle_offsets(v, s, d, q.MAXNORM)).tolist() == targets
    check_parity(v, s, d, 52, norm=q.MAXNORM)
    # the same stream twice under decode-accumulate, against the oracle's
    vd = torch.from_numpy(v).cuda()
    out, bits, offs = q.encode(vd, s, d, 52, norm=q.MAXNORM)
    acc0 = np.random.default_rng(53).standard_normal(v.size).astype(np.float32)
    acc = torch.from_numpy(acc0.copy()).cuda()
    q.decode_accumulate([out, out], [offs, offs], v.size, s, d, acc)
    torch.cuda.synchronize()
    nbits = int(bits.item())
    words = out[: (nbits + 63) // 64].cpu().numpy().view(np.uint64)
    offs_h = offs.cpu().numpy().view(np.uint64)
    bst = oracle.uniform_buckets(v.size, d)
    rc, want = oracle.decode_accumulate([(words, offs_h), (words, offs_h)], bst, s, acc0)
    assert rc == oracle.OK
    assert np.array_equal(acc.cpu().numpy().view(np.uint32), want.view(np.uint32))
