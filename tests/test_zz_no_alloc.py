"""GPU test of qsgd_encode_noalloc, the encode entry point for callers that
cannot allocate: its workspace lives in the library's fixed scratch array. Its
stream, bit count and bucket offsets must be bit-identical to qsgd_encode's on
the same inputs, on consecutive calls (the second smaller, so it runs over the
scratch the first one left behind), and an input whose workspace exceeds the
scratch must be refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import quantized_sgd_amd as q
from quantized_sgd_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


def _both(v: np.ndarray, s: int, d: int, seed: int):
    vd = torch.from_numpy(v).to("cuda")
    n = v.size
    nb = q.num_buckets(n, d)
    cap = q.encode_noalloc_capacity_words(n, s, d)
    assert cap > 0
    out = torch.zeros(cap, dtype=torch.int64, device="cuda")
    bits = torch.zeros(1, dtype=torch.int64, device="cuda")
    offs = torch.zeros(nb + 1, dtype=torch.int64, device="cuda")
    q.encode_noalloc(vd, s, d, seed, out, bits, offs)
    ref_out, ref_bits, ref_offs = q.encode(vd, s, d, seed)
    torch.cuda.synchronize()
    nbits = int(bits.item())
    assert nbits == int(ref_bits.item())
    w = (nbits + 63) // 64
    assert torch.equal(out[:w], ref_out[:w])
    assert torch.equal(offs, ref_offs)
    return nbits


def test_noalloc_matches_encode_on_consecutive_calls():
    print("noalloc: n=3000000 s=16 d=512", flush=True)
    b1 = _both(wl.small_gaussian(3_000_000, 41), 16, 512, 5)
    print("noalloc: n=100003 s=64 d=4096 (smaller, after the larger call)", flush=True)
    b2 = _both(wl.small_gaussian(100_003, 42), 64, 4096, 6)
    print("noalloc: n=7777 s=3 d=100", flush=True)
    b3 = _both(wl.small_gaussian(7_777, 43), 3, 100, 7)
    assert b1 > b2 > b3 > 0


def test_noalloc_refuses_inputs_beyond_the_scratch():
    s, d = 64, 4096
    n = 40_000_000
    assert q.encode_noalloc_capacity_words(n, s, d) == 0
    v = torch.zeros(n, dtype=torch.float32, device="cuda")
    out = torch.zeros(16, dtype=torch.int64, device="cuda")
    bits = torch.zeros(1, dtype=torch.int64, device="cuda")
    offs = torch.zeros(q.num_buckets(n, d) + 1, dtype=torch.int64, device="cuda")
    with pytest.raises(q.QsgdError) as e:
        q.encode_noalloc(v, s, d, 1, out, bits, offs)
    assert e.value.status == q.QSGD_ERR_SCRATCH
    assert int(bits.item()) == 0


def test_noalloc_empty_input():
    v = torch.zeros(0, dtype=torch.float32, device="cuda")
    out = torch.zeros(1, dtype=torch.int64, device="cuda")
    bits = torch.full((1,), 7, dtype=torch.int64, device="cuda")
    offs = torch.full((1,), 7, dtype=torch.int64, device="cuda")
    q.encode_noalloc(v, 4, 16, 1, out, bits, offs)
    torch.cuda.synchronize()
    assert int(bits.item()) == 0 and int(offs[0].item()) == 0
