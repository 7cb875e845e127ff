"""GPU parity of the ragged calls that take host tensor lengths
(qsgd_quantize_seglen / qsgd_encode_seglen / qsgd_decode_seglen: the layout
travels in the kernel arguments). Per-tensor quantization is the curated
page's bucketed training ("QSGD (Quantized Stochastic Gradient Descent) with
Elias Coding", claim on multi-GPU bucketed training, paper Section 3.3). Their
results must equal the oracle's and the table-form calls' bit for bit, on
batches with empty tensors, tensors shorter than a bucket, and the 150-tensor
ragged workload at full size."""
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


def _seglen_run(v, seg, s, d, seed):
    vd = to_dev(v)
    lev, nrm = q.quantize_seglen(vd, seg, s, d, seed)
    out, bits, offs = q.encode_seglen(vd, seg, s, d, seed)
    torch.cuda.synchronize()
    nbits = int(bits.item())
    vh = q.decode_seglen(out, offs, seg, s, d)
    torch.cuda.synchronize()
    return dict(levels=lev.cpu().numpy(), norms=nrm.cpu().numpy(), words=u64(out[: (nbits + 63) // 64]),
                offsets=u64(offs), bits=nbits, v_hat=vh.cpu().numpy(), out=out)


@pytest.mark.parametrize("nseg,hi,s,d,seed", [(40, 5000, 8, 512, 1), (160, 3000, 16, 100, 2),
                                              (7, 100000, 64, 4081, 3), (1, 70000, 4, 1024, 4)])
def test_seglen_matches_oracle_and_table_form(nseg, hi, s, d, seed):
    rng = np.random.default_rng(seed)
    seg = rng.integers(0, hi, size=nseg)
    if nseg > 3:
        seg[[1, nseg // 2]] = 0
        seg[2] = 3
    v = wl.small_gaussian(int(seg.sum()), seed)
    print(f"seglen nseg={nseg} n={v.size} s={s} d={d}", flush=True)
    g = _seglen_run(v, seg, s, d, seed)
    check_parity(v, s, d, seed, seg_len=seg, g=g)
    # the table form on the same layout gives the same words
    lay = q.RaggedLayout(seg, d)
    out, bits, offs = q.encode_ragged(to_dev(v), lay, s, seed)
    torch.cuda.synchronize()
    assert int(bits.item()) == g["bits"]
    assert np.array_equal(u64(out[: (g["bits"] + 63) // 64]), g["words"])
    assert np.array_equal(u64(offs), g["offsets"])


def test_seglen_ragged_workload_full_size():
    w = wl.config5()
    print(f"seglen ragged workload n={w.n} tensors={len(w.seg_len)}", flush=True)
    g = _seglen_run(w.v, w.seg_len, w.s, w.d, w.seed)
    lay = q.RaggedLayout(w.seg_len, w.d)
    vd = to_dev(w.v)
    out, bits, offs = q.encode_ragged(vd, lay, w.s, w.seed)
    vh = q.decode_ragged(out, offs, lay, w.s)
    torch.cuda.synchronize()
    assert int(bits.item()) == g["bits"]
    assert np.array_equal(u64(out[: (g["bits"] + 63) // 64]), g["words"])
    assert np.array_equal(u64(offs), g["offsets"])
    assert np.array_equal(vh.cpu().numpy().view(np.uint32), g["v_hat"].view(np.uint32))
