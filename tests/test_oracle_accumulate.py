"""Pins of the oracle's decode-accumulate (the receiving side of a gradient
exchange: page "QSGD: Communication-Efficient SGD via Gradient Quantization and
Encoding", abstract), against facts that do not come from the oracle itself.

Reading under test: acc_i <- (((acc_i + v_hat_0,i) + v_hat_1,i) + ...) with one
fp32 addition per stream, streams in order.

The pins use buckets of one coordinate with s = 1, where the method is exact:
the norm of a one-coordinate bucket is |v_i| (the fp64 square of an fp32 value
is exact and so is its square root), r = RN32(1 * |v_i| / |v_i|) = 1, so
l = 1, p = 0 and k = 1 whatever the random draw, and decoding returns
RN32(|v_i| * 1 / 1) = |v_i| with the sign: v_hat = v exactly, except
that zeros come back as +0.0. The accumulate must then be numpy's float32
left fold of the inputs.
"""
import numpy as np
import pytest

import oracle


def _streams(vectors, s, d, seed0=11, code=oracle.OMEGA):
    bst = oracle.uniform_buckets(vectors[0].size, d)
    out = []
    for j, v in enumerate(vectors):
        _, _, words, offs, _ = oracle.compress(v, bst, s, seed0 + j, code=code)
        out.append((words, offs))
    return bst, out


def _fold(acc, vectors):
    a = np.array(acc, dtype=np.float32, copy=True)
    with np.errstate(over="ignore"):
        for v in vectors:
            a = (a + np.where(v == 0, np.float32(0.0), v).astype(np.float32)).astype(np.float32)
    return a


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def test_identity_buckets_fold_in_stream_order():
    # 1e8 + 1 == 1e8 in fp32: the order of the additions shows in the result
    vs = [np.float32([1e8, 1, 2, -0.0, 3, 0, 5, -7, 1e-30, 9, -3e38]),
          np.float32([1, 1e-8, -2, 0, -3, 0, 5, 7, 1e-30, 9, -3e38]),
          np.float32([-1e8, 1, 0, 0, 1, 0, 5, 0, 0, -18, 1])]
    acc = np.float32([-0.0, 0, 0, -0.0, 0, -0.0, 0, 0, 0, 0, 0])
    bst, streams = _streams(vs, 1, 1)
    rc, out = oracle.decode_accumulate(streams, bst, 1, acc)
    assert rc == oracle.OK
    exp = _fold(acc, vs)
    assert np.array_equal(_bits(out), _bits(exp))
    assert out[0] == 0.0 and out[3] == 0.0 and not np.signbit(out[3])  # -0 + +0 = +0
    assert np.isneginf(out[10])  # -3e38 + -3e38 overflows in fp32


@pytest.mark.parametrize("code", [oracle.OMEGA, oracle.GAMMA])
def test_identity_buckets_random_fold(code):
    rng = np.random.default_rng(5)
    n, k = 2000, 6
    vs = []
    for _ in range(k):
        v = (rng.standard_normal(n) * 10.0 ** rng.integers(-20, 20, n)).astype(np.float32)
        v[rng.random(n) < 0.2] = 0.0
        vs.append(v)
    acc = (rng.standard_normal(n) * 1e3).astype(np.float32)
    acc[::7] = -0.0
    bst, streams = _streams(vs, 1, 1, code=code)
    rc, out = oracle.decode_accumulate(streams, bst, 1, acc, code=code)
    assert rc == oracle.OK
    assert np.array_equal(_bits(out), _bits(_fold(acc, vs)))


def test_one_stream_from_zero_is_decode_and_none_is_identity():
    rng = np.random.default_rng(6)
    v = rng.standard_normal(5000).astype(np.float32)
    bst = oracle.uniform_buckets(v.size, 512)
    _, _, words, offs, _ = oracle.compress(v, bst, 16, 3)
    rc, out = oracle.decode_accumulate([(words, offs)], bst, 16, np.zeros(v.size, np.float32))
    rc2, ref = oracle.decode(words, offs, bst, 16)
    assert rc == rc2 == oracle.OK
    assert np.array_equal(_bits(out), _bits(ref))
    # a gamma stream from zero decodes to the same values as the omega one
    _, _, gw, go, _ = oracle.compress(v, bst, 16, 3, code=oracle.GAMMA)
    rc, gout = oracle.decode_accumulate([(gw, go)], bst, 16, np.zeros(v.size, np.float32), code=oracle.GAMMA)
    assert rc == oracle.OK and np.array_equal(_bits(gout), _bits(ref))
    acc = rng.standard_normal(v.size).astype(np.float32)
    rc, out = oracle.decode_accumulate([], bst, 16, acc)
    assert rc == oracle.OK and np.array_equal(_bits(out), _bits(acc))


def test_malformed_stream_is_reported():
    v = np.float32([1.0, -2.0, 3.0, 0.5])
    bst = oracle.uniform_buckets(v.size, 4)
    _, _, words, offs, _ = oracle.compress(v, bst, 4, 1)
    bad = offs.copy()
    bad[-1] = bad[-1] + 64 * 8  # claims bits past the stream
    rc, _ = oracle.decode_accumulate([(words, offs), (words, bad)], bst, 4, np.zeros(4, np.float32))
    assert rc == oracle.ERR_MALFORMED
