"""GPU parity: the HIP path (through the C ABI) against the oracle.

Every comparison is element by element: norms within 1e-6 relative; levels,
stream words, bucket bit offsets, bit counts and decoded values bit-exact given
the GPU's norms (see tests/parity.py). Sizes span several tiles and a ragged
tail; the full-size workloads run in the launch configuration the benchmark uses.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_sgd_amd as q
from quantized_sgd_amd import workloads as wl
from tests.parity import check_parity, gpu_run, to_dev, u64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


def test_config1_exact():
    w = wl.config1()
    g, info = check_parity(w.v, w.s, w.d, w.seed)
    assert info["norms_exact"] == 1


SMALL = [
    # n, d, s, seed
    (1, 1, 1, 1), (5, 2, 4, 2), (17, 16, 3, 3), (100, 7, 2, 4), (4095, 4096, 4, 5),
    (4096, 4096, 64, 6), (4097, 4096, 64, 7), (9000, 4096, 64, 8), (20000, 512, 16, 9),
    (20001, 513, 8, 10), (33333, 100, 1, 11), (50000, 1, 5, 12), (12345, 3, 1000, 13),
    (70000, 2048, 1 << 24, 14), (40000, 4081, 2, 15), (123457, 64, 7, 16), (8192, 16, 255, 17),
]


@pytest.mark.parametrize("n,d,s,seed", SMALL)
def test_small_gaussian(n, d, s, seed):
    v = wl.small_gaussian(n, seed)
    check_parity(v, s, d, seed)


@pytest.mark.parametrize("n,d,s,seed", [(30000, 512, 16, 21), (9999, 37, 3, 22), (4096, 4096, 1, 23),
                                        (65536, 1024, 64, 24)])
def test_mixed_edge_values(n, d, s, seed):
    v = wl.mixed_values(n, seed)
    check_parity(v, s, d, seed)


@pytest.mark.parametrize("n,d,s,seed", [(4096 + 37, 16, 64, 41), (20000, 64, 64, 42), (3000, 32, 50, 43)])
def test_long_records_per_thread(n, d, s, seed):
    # near-constant magnitudes put the levels near s / sqrt(d): records of 9-15
    # bits, so the records of 8 consecutive coordinates pass 64 bits
    rng = np.random.default_rng(seed)
    v = (rng.choice([-1.0, 1.0], n) * (1.0 + 0.01 * rng.standard_normal(n))).astype(np.float32)
    check_parity(v, s, d, seed)


@pytest.mark.parametrize("code", [0, 1])
def test_long_halves_from_spikes(code):
    # buckets of 1024 with s = 64: levels are small on average (the encoder keeps
    # no level bytes for such launches), but 16 spikes of equal size per bucket
    # get k = 16 and records of 13+ bits, so their thread halves pass 64 bits
    rng = np.random.default_rng(44)
    n, d = 64 * 1024 + 100, 1024
    v = (1e-6 * rng.standard_normal(n)).astype(np.float32)
    for b0 in range(0, n - 336, d):
        v[b0 + 320:b0 + 336] = rng.choice([-1.0, 1.0], 16).astype(np.float32)
    check_parity(v, 64, d, 44, code=code)


def test_zero_buckets_and_spikes():
    n, d = 40000, 512
    v = np.zeros(n, np.float32)
    v[::1000] = 3.0          # isolated spikes: r = s exactly
    v[5000:5512] = -0.0      # a bucket of negative zeros
    v[20000:20512] = 1.0     # constant bucket
    check_parity(v, 16, d, 3)


def test_chain_repairs_out_of_phase():
    """Streams on which the decoder's speculative chains never meet the true one.
    Under the max-norm with s = 1 a constant positive bucket has level 1 at every
    coordinate (r = 1 exactly), so each record is the three bits 000 and the
    payload is all zeros: a chain started 1 or 2 bits off a record boundary stays
    off it to the end. With a segment length that is not a multiple of 3, lanes
    start in all three phases, so most lanes are restarted, and a lane restarted
    from a predecessor that is itself restarted must be restarted again. The
    bucket lengths below (ragged, buckets of at most 4000) give 7 to 64 lanes of
    129 to 188 bits, seven buckets out of phase."""
    s, d = 1, 4000
    seg = np.array([1000, 4096, 1001, 333, 3100, 650, 2500, 4000, 2731], dtype=np.int64)
    v = np.full(int(seg.sum()), 0.5, dtype=np.float32)
    v[4096 + 1000:4096 + 1000 + 1001] = 2.0   # a second constant
    bst = oracle.ragged_buckets(seg, d)
    _, _, _, offs, _ = oracle.compress(v, bst, s, 7, norms=oracle.bucket_max_norms(v, bst))
    # the payload lengths give decoder segments that are not multiples of 3 bits
    out_of_phase = 0
    for b in range(len(bst) - 1):
        lp = int(offs[b + 1] - offs[b]) - 32
        assert lp == 3 * int(bst[b + 1] - bst[b])
        nl = max(1, min(64, lp // 128))
        out_of_phase += ((lp + nl - 1) // nl) % 3 != 0
    assert out_of_phase >= 5
    check_parity(v, s, d, 7, seg_len=seg, norm=q.MAXNORM)
    check_parity(v, s, d, 8, seg_len=seg, norm=q.MAXNORM, code=oracle.GAMMA)


def test_integer_valued_norms_are_exact():
    # small integers: every partial sum is exact in fp64, so GPU and oracle norms
    # must agree bit for bit whatever the summation order
    rng = np.random.default_rng(1)
    v = rng.integers(-50, 50, size=4096 * 5 + 100).astype(np.float32)
    g, info = check_parity(v, 8, 4096, 9)
    assert info["norms_exact"] == info["nb"]


@pytest.mark.parametrize("seed", [31, 32])
def test_ragged_small(seed):
    rng = np.random.default_rng(seed)
    seg = rng.integers(1, 3000, size=40).astype(np.uint64)
    seg[3] = 1
    seg[7] = 16
    v = wl.small_gaussian(int(seg.sum()), seed)
    check_parity(v, 8, 512, seed, seg_len=seg)


def test_ragged_with_empty_segments():
    seg = np.array([0, 5, 0, 513, 1, 0, 4096, 7], np.uint64)
    v = wl.small_gaussian(int(seg.sum()), 7)
    check_parity(v, 4, 512, 7, seg_len=seg)


def test_empty_input():
    v = torch.empty(0, dtype=torch.float32, device="cuda")
    out, bits, offs = q.encode(v, 4, 512, 1)
    torch.cuda.synchronize()
    assert int(bits.item()) == 0 and int(offs[0].item()) == 0


def test_deterministic_and_repeatable():
    v = wl.chunked_gaussian(300_000, 5)
    a = gpu_run(v, 16, 512, 2)
    for _ in range(20):
        b = gpu_run(v, 16, 512, 2)
        assert a["bits"] == b["bits"]
        assert np.array_equal(a["words"], b["words"])
        assert np.array_equal(a["norms"].view(np.uint32), b["norms"].view(np.uint32))


def test_decode_writes_exactly_n():
    n, d, s = 10000, 512, 16
    v = wl.small_gaussian(n, 3)
    vd = to_dev(v)
    out, bits, offs = q.encode(vd, s, d, 4)
    guard = torch.full((n + 64,), 7.0, dtype=torch.float32, device="cuda")
    q.decode(out, offs, n, s, d, v_hat=guard[:n])
    torch.cuda.synchronize()
    assert torch.all(guard[n:] == 7.0)


def test_decode_of_oracle_stream():
    # the GPU decoder on a stream built entirely by the oracle
    n, d, s, seed = 50000, 4096, 64, 5
    v = wl.small_gaussian(n, seed)
    bst = oracle.uniform_buckets(n, d)
    lev, nrm, words, offs, nbits = oracle.compress(v, bst, s, seed)
    wd = to_dev(np.concatenate([words, np.zeros(1, np.uint64)]).view(np.int64))
    od = to_dev(offs.view(np.int64))
    vh = q.decode(wd, od, n, s, d).cpu().numpy()
    want = oracle.dequantize(lev, nrm, bst, s)
    assert np.array_equal(vh.view(np.uint32), want.view(np.uint32))


def test_invalid_arguments():
    v = torch.zeros(64, dtype=torch.float32, device="cuda")
    with pytest.raises(q.QsgdError):
        q.quantize(v, 0, 16, 1)
    with pytest.raises(q.QsgdError):
        q.quantize(v, 4, 0, 1)
    with pytest.raises(q.QsgdError):
        q.quantize(v, (1 << 24) + 1, 16, 1)
    with pytest.raises(q.QsgdError):
        q.quantize(v[1:], 4, 16, 1)  # misaligned
    cap = q.encode_capacity_words(64, 4, 16)
    out = torch.empty(cap + 1, dtype=torch.int64, device="cuda")
    with pytest.raises(q.QsgdError):
        q.encode(v, 4, 16, 1, out=out[1:])  # out misaligned


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_full_size_configs(cfg):
    w = wl.CONFIGS[cfg]()
    g, info = check_parity(w.v, w.s, w.d, w.seed, seg_len=w.seg_len)
    print(f"{w.name}: bits/coord {g['bits'] / w.n:.4f}, norms exact {info['norms_exact']}/{info['nb']}")


def test_full_size_config4():
    w = wl.config4()
    g, info = check_parity(w.v, w.s, w.d, w.seed)
    print(f"{w.name}: bits/coord {g['bits'] / w.n:.4f}, norms exact {info['norms_exact']}/{info['nb']}")
