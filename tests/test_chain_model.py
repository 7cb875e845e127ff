"""What the decoder's parallel parse does on given inputs, from the CPU model in
tests/chain_model.py over oracle streams: which inputs make speculative chains
fail to meet (and so exercise the repair rounds the GPU tests then check), and
how far past a segment start chains meet on Gaussian buckets."""
import numpy as np

import oracle
from quantized_sgd_amd import workloads as wl
from tests.chain_model import Bucket, model_bucket, stream_bits, SYNC_BITS


def buckets_of(v, d, s, seg_len=None, maxnorm=False, code=oracle.OMEGA):
    bst = oracle.uniform_buckets(v.size, d) if seg_len is None else oracle.ragged_buckets(seg_len, d)
    norms = oracle.bucket_max_norms(v, bst) if maxnorm else None
    _, _, words, offs, _ = oracle.compress(v, bst, s, 7, norms=norms, code=code)
    bits = stream_bits(words)
    return [Bucket(bits, int(offs[b]), int(offs[b + 1]), int(bst[b + 1] - bst[b]), s, code)
            for b in range(len(bst) - 1)]


def test_out_of_phase_stream_forces_repeated_restarts():
    # the input of the GPU test test_chain_repairs_out_of_phase: constant buckets
    # under the max-norm with s = 1, all-zero payloads of 3-bit records
    seg = np.array([1000, 4096, 1001, 333, 3100, 650, 2500, 4000, 2731], dtype=np.int64)
    v = np.full(int(seg.sum()), 0.5, dtype=np.float32)
    res = [model_bucket(b) for b in buckets_of(v, 4000, 1, seg, maxnorm=True)]
    phase = [(b.seg % 3 != 0) for b in buckets_of(v, 4000, 1, seg, maxnorm=True)]
    for r, off in zip(res, phase):
        if off:
            assert r["restarts"] > 0 and r["rounds"] >= 2, r
        else:
            assert r["restarts"] == 0, r
    assert sum(r["rerestarts"] for r in res) > 100
    assert max(r["rounds"] for r in res) > 10


def test_gaussian_buckets_meet_within_the_window():
    # buckets like the ResNet-152 workload's (d = 4096, s = 64, L2 norm): every
    # lane's chain meets its successor within the noted window, no restarts
    v = wl.small_gaussian(6 * 4096, 11)
    res = [model_bucket(b) for b in buckets_of(v, 4096, 64)]
    for r in res:
        assert r["lanes"] == 64 and r["restarts"] == 0, r
        assert max(r["sync"]) < SYNC_BITS
        assert 15 <= max(r["steps_a"]) <= 40


def test_maxnorm_buckets_need_restarts():
    # the max-norm at s = 64 gives long records that often miss the table; some
    # chains then meet their successor only past the window and are restarted
    v = wl.small_gaussian(4 * 4096, 12)
    bks = buckets_of(v, 4096, 64, maxnorm=True)
    res = [model_bucket(b) for b in bks]
    assert all(not b.guess for b in bks)  # more than 4 payload bits per coordinate
    assert sum(r["restarts"] for r in res) > 0


def test_guess_steps_delay_sync_on_maxnorm_streams():
    # long records miss the table on the true chain too, where a guess step's
    # one-bit move derails the chain: without guess steps speculative chains
    # join the true one sooner, and fewer need more than the noted window
    from tests.chain_model import sync_distances
    v = wl.small_gaussian(6 * 4096, 13)
    no_g, with_g = [], []
    for b in buckets_of(v, 4096, 64, maxnorm=True):
        no_g += [x if x is not None else 10**6 for x in sync_distances(b, False)]
        with_g += [x if x is not None else 10**6 for x in sync_distances(b, True)]
    no_g, with_g = np.array(no_g), np.array(with_g)
    assert np.median(no_g) < np.median(with_g)
    assert np.mean(no_g > SYNC_BITS) < np.mean(with_g > SYNC_BITS)
