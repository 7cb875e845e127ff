"""GPU parity of the decode of buckets longer than 16384 coordinates, which is
cut into chunks of 16384 stream bits, one wave each (page "QSGD (Quantized
Stochastic Gradient Descent) with Elias Coding", definition paragraph: the
coding is lossless, for the whole vector v in R^n as for buckets).

Cases: the whole-vector operator d = n at n = 4097, 10^6 and 60,192,808 (the
ResNet-152-sized gradient as one bucket); streams on which chunk chains never
meet, decoded by the whole-bucket fallback (constant vectors with
s = sqrt(n), where every record is the same 3 bits, so chains started a
multiple of 3 bits apart never meet); a mix of such buckets with Gaussian
ones; the gamma code; decode-accumulate over long buckets; payloads a few bits
longer than a multiple of the chunk (the last chunk takes the rest, so that a
chain started in it has a whole chunk to meet the exact one); buckets without
records among long ones (written, and accumulated, as zeros); and very sparse
whole vectors, whose outputs are zeroed first and then get the records'
values."""
import numpy as np
import pytest
import torch

import oracle
import quantized_sgd_amd as q
from quantized_sgd_amd import workloads as wl
from tests.parity import check_parity, to_dev, u64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


@pytest.mark.parametrize("n,s,seed", [(4097, 4, 1), (1_000_000, 1000, 2), (1_000_000, 64, 3)])
def test_whole_vector(n, s, seed):
    print(f"whole vector n={n} s={s}", flush=True)
    check_parity(wl.small_gaussian(n, seed), s, n, seed)


@pytest.mark.parametrize("s", [64, 7759])
def test_whole_vector_config3_gradient(s):
    # the ResNet-152-sized gradient as one bucket, at the config's s and at
    # s ~ sqrt(n), where the stream spans tens of thousands of chunks
    w = wl.config3()
    print(f"whole vector n={w.n} s={s} (config-3 gradient as one bucket)", flush=True)
    g, _ = check_parity(w.v, s, w.n, w.seed)
    print(f"  stream bits {g['bits']}", flush=True)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_out_of_phase_chunks_take_the_fallback(sign):
    # n = 65536 and s = 256 = sqrt(n): r = 1 exactly, every record is the same
    # 3 bits, and chunk 1 starts 16384 = 1 (mod 3) bits after chunk 0
    n, s = 65536, 256
    v = np.full(n, sign, np.float32)
    print(f"constant vector sign={sign}", flush=True)
    g, _ = check_parity(v, s, n, 5)
    assert g["bits"] == 32 + 3 * n


def test_mixed_buckets_some_falling_back():
    d, s = 65536, 256
    v = np.concatenate([np.full(d, 1.0, np.float32), wl.small_gaussian(d, 6),
                        np.full(d, -2.0, np.float32), wl.small_gaussian(d + 123, 7)])
    print("mixed buckets", flush=True)
    check_parity(v, s, d, 8)


def test_chunked_gamma_and_maxnorm():
    print("chunked gamma / maxnorm", flush=True)
    check_parity(wl.small_gaussian(300000, 9), 16, 100000, 9, code=oracle.GAMMA)
    check_parity(wl.small_gaussian(300000, 10), 64, 150000, 10, norm=q.MAXNORM)


def test_chunked_decode_accumulate():
    n, d, s = 400000, 200000, 64
    bst = oracle.uniform_buckets(n, d)
    streams, dev = [], []
    for j in range(3):
        v = wl.small_gaussian(n, 20 + j)
        lev, nrm = oracle.quantize(v, bst, s, 30 + j)
        words, offs, _ = oracle.encode(lev, nrm, bst, s)
        streams.append((words, offs))
        dev.append((to_dev(words.view(np.int64)), to_dev(offs.view(np.int64))))
    acc0 = wl.small_gaussian(n, 40)
    acc = to_dev(acc0.copy())
    print("chunked decode-accumulate", flush=True)
    q.decode_accumulate([w for w, _ in dev], [o for _, o in dev], n, s, d, acc)
    torch.cuda.synchronize()
    rc, want = oracle.decode_accumulate(streams, bst, s, acc0.copy())
    assert rc == oracle.OK
    assert np.array_equal(acc.cpu().numpy().view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("s,seed,n", [(64, 11, 61620), (16, 12, 61970)])
def test_payload_just_past_whole_chunks(s, seed, n):
    v = wl.small_gaussian(120000, seed)[:n]
    bst = oracle.uniform_buckets(n, n)
    _, _, _, _, nbits = oracle.compress(v, bst, s, seed)
    payload = nbits - 32
    assert payload > 16384 and 0 < payload % 16384 < 8
    print(f"whole vector n={n} s={s}: payload {payload} bits", flush=True)
    check_parity(v, s, n, seed)


def test_long_buckets_without_records():
    # a zero bucket (norm 0: its stream is the 32-bit norm alone) between long
    # Gaussian buckets, decoded into a buffer of sentinels, and accumulated
    # into -0.0f accumulators there
    d, s = 20000, 64
    rng = np.random.default_rng(31)
    v = np.concatenate([rng.standard_normal(d), np.zeros(d), rng.standard_normal(d + 5)]).astype(np.float32)
    n = v.size
    bst = oracle.uniform_buckets(n, d)
    lev, nrm = oracle.quantize(v, bst, s, 32)
    words, offs, _ = oracle.encode(lev, nrm, bst, s)
    assert offs[2] - offs[1] == 32
    want = oracle.dequantize(lev, nrm, bst, s)
    wd, od = to_dev(words.view(np.int64)), to_dev(offs.view(np.int64))
    print("long buckets without records", flush=True)
    vh = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    q.decode(wd, od, n, s, d, v_hat=vh)
    torch.cuda.synchronize()
    assert np.array_equal(vh.cpu().numpy().view(np.uint32), want.view(np.uint32))
    acc0 = rng.standard_normal(n).astype(np.float32)
    acc0[d:2 * d] = -0.0
    acc = to_dev(acc0.copy())
    q.decode_accumulate([wd], [od], n, s, d, acc)
    torch.cuda.synchronize()
    rc, exp = oracle.decode_accumulate([(words, offs)], bst, s, acc0.copy())
    assert rc == oracle.OK
    got = acc.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), exp.view(np.uint32))
    assert np.all(got[d:2 * d].view(np.uint32) == 0)     # -0.0 + +0.0 = +0.0


@pytest.mark.parametrize("n,s", [(1_000_000, 1), (3_000_000, 2)])
def test_very_sparse_whole_vectors(n, s):
    # few records with gaps of thousands of coordinates: the output is zeroed by
    # a parallel fill and the chunk writers store only the records' values
    v = wl.small_gaussian(n, 41 + s)
    print(f"sparse whole vector n={n} s={s}", flush=True)
    g, _ = check_parity(v, s, n, 42)
    assert g["bits"] < n // 50
