"""GPU parity of the Elias gamma variant (qsgd_encode_ex / qsgd_decode_ex with
QSGD_CODE_GAMMA) against the oracle: the page names "Elias recursive
gamma/omega" coding; the stream layout is the omega one with gamma codewords.
Same rules as tests/parity.py: norms within 1e-6 relative, everything else
bit-exact given the GPU's norms. Cases cover the aligned and general encoders,
the staged and per-lane decoders, ragged batches, records past 64 bits per
thread half, edge values, and config 3 at full size."""
import numpy as np
import pytest
import torch

import oracle
import quantized_sgd_amd as q
from quantized_sgd_amd import workloads as wl
from tests.parity import check_parity, to_dev, u64

pytestmark = pytest.mark.gpu
G = oracle.GAMMA


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


@pytest.mark.parametrize("n,d,s,seed", [
    (1, 1, 1, 1), (17, 16, 3, 3), (4095, 4096, 4, 5), (4096, 4096, 64, 6), (9000, 4096, 64, 8),
    (20000, 512, 16, 9), (20001, 513, 8, 10), (33333, 100, 1, 11), (50000, 1, 5, 12),
    (12345, 3, 1000, 13), (70000, 2048, 1 << 24, 14), (123457, 64, 7, 16), (8192, 16, 255, 17),
])
def test_gamma_small(n, d, s, seed):
    check_parity(wl.small_gaussian(n, seed), s, d, seed, code=G)


@pytest.mark.parametrize("n,d,s,seed", [(30000, 512, 16, 21), (9999, 37, 3, 22), (65536, 1024, 64, 24)])
def test_gamma_mixed_values(n, d, s, seed):
    check_parity(wl.mixed_values(n, seed), s, d, seed, code=G)


@pytest.mark.parametrize("n,d,s,seed", [(4096 + 37, 16, 64, 41), (20000, 64, 64, 42)])
def test_gamma_long_records_per_thread(n, d, s, seed):
    rng = np.random.default_rng(seed)
    v = (rng.choice([-1.0, 1.0], n) * (1.0 + 0.01 * rng.standard_normal(n))).astype(np.float32)
    check_parity(v, s, d, seed, code=G)


def test_gamma_ragged():
    rng = np.random.default_rng(31)
    seg = rng.integers(0, 5000, size=40)
    seg[[4, 17]] = 0
    v = wl.small_gaussian(int(seg.sum()), 31)
    check_parity(v, 8, 512, 31, seg_len=seg, code=G)


def test_gamma_decode_of_oracle_stream():
    # a stream the oracle wrote, decoded by the GPU
    v = wl.small_gaussian(50000, 7)
    bst = oracle.uniform_buckets(v.size, 512)
    lev, nrm, words, offs, nbits = oracle.compress(v, bst, 16, 7, code=G)
    vh = q.decode(to_dev(words.view(np.int64)), to_dev(offs.view(np.int64)), v.size, 16, 512, code=G)
    torch.cuda.synchronize()
    want = oracle.dequantize(lev, nrm, bst, 16)
    assert np.array_equal(vh.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_gamma_full_size_config3():
    w = wl.config3()
    g, info = check_parity(w.v, w.s, w.d, w.seed, code=G)
    # gamma streams of this workload are longer than omega ones (gamma spends
    # 2 floor(log2 N) + 1 bits, omega fewer for N >= 4 except a few values)
    assert g["bits"] > 0
