"""GPU parity of decode-accumulate (through the C ABI) against the oracle.

The streams are written by the oracle (so no oracle input comes from the HIP
path), copied to the device, and summed into an accumulator that starts from
seeded values with some -0.0 entries; the result must be bit-identical to the
oracle's in-order fp32 fold. Cases cover the LDS-staged path (s <= 127,
d <= 4096): with up to 8 streams over buckets of 256 or more coordinates (a
multiple of 4) the streams of a group are decoded side by side and folded into
the accumulator at once (values tabulated per bucket, or formed directly where
groups hold several buckets and s is a power of two; groups that do not fit the
stage summed stream by stream), otherwise stream by stream; the per-lane writer
path (s > 127 or d > 4096), ragged buckets, one to 32 streams, zero streams,
and the config-3 workload at full size with the launch configuration the
benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_sgd_amd as q
from quantized_sgd_amd import workloads as wl
from tests.parity import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


def _oracle_streams(vs, bst, s, seed0):
    out = []
    for j, v in enumerate(vs):
        _, _, words, offs, _ = oracle.compress(v, bst, s, seed0 + j)
        out.append((words, offs))
    return out


def _start_acc(n, seed):
    rng = np.random.default_rng(seed)
    acc = rng.standard_normal(n).astype(np.float32)
    acc[::5] = -0.0
    return acc


def _run(streams, bst, n, s, d, acc0, seg_len=None):
    wd = [to_dev(np.ascontiguousarray(w if len(w) else np.zeros(1, np.uint64)).view(np.int64)) for w, _ in streams]
    od = [to_dev(np.ascontiguousarray(o).view(np.int64)) for _, o in streams]
    acc = to_dev(acc0.copy())
    if seg_len is None:
        q.decode_accumulate(wd, od, n, s, d, acc)
    else:
        q.decode_accumulate_ragged(wd, od, q.RaggedLayout(seg_len, d), s, acc)
    torch.cuda.synchronize()
    return acc.cpu().numpy()


def _check(vs, s, d, seed, seg_len=None):
    n = vs[0].size
    bst = oracle.uniform_buckets(n, d) if seg_len is None else oracle.ragged_buckets(seg_len, d)
    streams = _oracle_streams(vs, bst, s, seed)
    acc0 = _start_acc(n, seed)
    got = _run(streams, bst, n, s, d, acc0, seg_len)
    rc, exp = oracle.decode_accumulate(streams, bst, s, acc0)
    assert rc == oracle.OK
    bad = np.flatnonzero(got.view(np.uint32) != exp.view(np.uint32))
    assert bad.size == 0, f"{bad.size} mismatches, first at {bad[:5]}: {got[bad[:5]]} vs {exp[bad[:5]]}"


@pytest.mark.parametrize("n,d,s,k,seed", [
    (20000, 512, 16, 3, 1), (9999, 37, 3, 5, 2), (3 * 4096 + 5, 4096, 64, 4, 3),
    (5000, 64, 4, 32, 4), (4097, 4096, 1, 2, 5), (1, 1, 1, 3, 6),
    (50000, 512, 16, 1, 11), (20000, 256, 8, 5, 12), (30002, 1024, 32, 8, 13), (9000, 300, 4, 2, 14),
    (12000, 512, 12, 3, 16), (8002, 1024, 100, 2, 17),
])
def test_accumulate_lds_path(n, d, s, k, seed):
    vs = [wl.small_gaussian(n, seed * 100 + j) for j in range(k)]
    _check(vs, s, d, seed)


@pytest.mark.parametrize("n,d,s,k,seed", [(70000, 2048, 1 << 24, 2, 7), (30000, 8192, 8, 3, 8),
                                          (12345, 3, 1000, 2, 9)])
def test_accumulate_lane_writer_path(n, d, s, k, seed):
    vs = [wl.small_gaussian(n, seed * 100 + j) for j in range(k)]
    _check(vs, s, d, seed)


def test_accumulate_groups_past_the_stage():
    # d = 4096, s = 64, three streams; stream 1 scales buckets 1 and 3 by their
    # largest magnitude (about 9.5 bits per coordinate: those groups do not fit
    # the decoder's stage and are summed stream by stream), the other buckets and
    # streams by the L2 norm
    n, d, s, seed = 5 * 4096 + 100, 4096, 64, 15
    vs = [wl.small_gaussian(n, 1500 + j) for j in range(3)]
    bst = oracle.uniform_buckets(n, d)
    streams = []
    for j, v in enumerate(vs):
        norms = oracle.bucket_norms(v, bst)
        if j == 1:
            mx = oracle.bucket_max_norms(v, bst)
            norms[[1, 3]] = mx[[1, 3]]
        _, _, words, offs, _ = oracle.compress(v, bst, s, seed + j, norms=norms)
        streams.append((words, offs))
    per_bucket = np.diff(streams[1][1].astype(np.int64)) / d
    assert per_bucket[1] > 8 and per_bucket[3] > 8 and per_bucket[0] < 4
    acc0 = _start_acc(n, seed)
    got = _run(streams, bst, n, s, d, acc0)
    rc, exp = oracle.decode_accumulate(streams, bst, s, acc0)
    assert rc == oracle.OK
    assert np.array_equal(got.view(np.uint32), exp.view(np.uint32))


def test_accumulate_sparse_and_mixed_values():
    vs = [wl.mixed_values(40000, 30 + j) for j in range(3)]
    _check(vs, 8, 512, 30)


def test_accumulate_ragged():
    rng = np.random.default_rng(40)
    seg = rng.integers(0, 3000, size=25)
    seg[[3, 11]] = 0
    n = int(seg.sum())
    vs = [wl.small_gaussian(n, 400 + j) for j in range(3)]
    _check(vs, 8, 512, 40, seg_len=seg)


def test_zero_streams_leave_acc_unchanged():
    acc0 = _start_acc(1000, 50)
    acc = to_dev(acc0.copy())
    q.decode_accumulate([], [], 1000, 4, 64, acc)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().view(np.uint32), acc0.view(np.uint32))


def test_too_many_streams_rejected():
    v = to_dev(wl.small_gaussian(100, 1))
    out, _, offs = q.encode(v, 4, 16, 1)
    acc = torch.zeros(100, dtype=torch.float32, device="cuda")
    with pytest.raises(q.QsgdError):
        q.decode_accumulate([out] * 33, [offs] * 33, 100, 4, 16, acc)


def test_full_size_config3_four_streams():
    w = wl.config3()
    vs = [w.v] + [wl.peer_gradient(3, j) for j in range(1, 4)]
    _check(vs, w.s, w.d, w.seed)


def test_full_size_config2_four_streams():
    # eight buckets of 512 per group and s = 16: the folded sum forms each value
    # directly, the whole round in one pass
    w = wl.config2()
    vs = [w.v] + [wl.peer_gradient(2, j) for j in range(1, 4)]
    print(f"decode-accumulate full size n={w.n} d={w.d} s={w.s} k=4", flush=True)
    _check(vs, w.s, w.d, w.seed)


@pytest.mark.parametrize("n,d,s,k", [(50000, 512, 16, 3), (30000, 4096, 64, 2), (20000, 1000, 300, 4),
                                     (200000, 50000, 8, 2)])
def test_gamma_streams(n, d, s, k):
    # streams of the Elias gamma record code, through qsgd_decode_accumulate_ex
    vs = [wl.small_gaussian(n, 60 + j) for j in range(k)]
    bst = oracle.uniform_buckets(n, d)
    streams = []
    for j, v in enumerate(vs):
        _, _, words, offs, _ = oracle.compress(v, bst, s, 70 + j, code=oracle.GAMMA)
        streams.append((words, offs))
    acc0 = _start_acc(n, 80)
    wd = [to_dev(np.ascontiguousarray(w).view(np.int64)) for w, _ in streams]
    od = [to_dev(np.ascontiguousarray(o).view(np.int64)) for _, o in streams]
    acc = to_dev(acc0.copy())
    print(f"gamma accumulate n={n} d={d} s={s} k={k}", flush=True)
    q.decode_accumulate(wd, od, n, s, d, acc, code=q.GAMMA)
    torch.cuda.synchronize()
    rc, want = oracle.decode_accumulate(streams, bst, s, acc0.copy(), code=oracle.GAMMA)
    assert rc == oracle.OK
    assert np.array_equal(acc.cpu().numpy().view(np.uint32), want.view(np.uint32))
