"""GPU parity on streams whose gaps and levels take every structure of the Elias
omega code: page "QSGD (Quantized Stochastic Gradient Descent) with Elias
Coding", encoding paragraph (the distances between non-zero coordinates and the
levels are coded with Elias's recursive code).

Both record codes are run (the Elias gamma code of the same page as well). Each
bucket holds equal non-zero magnitudes at chosen distances and exact zeros
elsewhere. Under the max-norm scale every non-zero has ratio s exactly, so its
level is s whatever the random words, and the gaps are the distances placed:
1 to 16384, across the boundaries where an omega codeword
gains a group (3, 4, 7, 8, 15, 16, 31, 32, ...), with levels whose codewords are
1 bit (s = 1) up to 33 bits (s = 2^24 - 1). Short records decode from the
decoder's 12-bit table, records past it from the table's partial field groups
and the general omega loop; buckets of 512 coordinates take the lane-per-bucket
decode, of 4096 the team decode (with per-lane writers for s > 127), and of
65536 the chunked decode. Everything is compared bit for bit with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_sgd_amd as q
from tests.parity import check_parity

pytestmark = pytest.mark.gpu

GAPS = [1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256,
        511, 512, 1023, 1024, 2047, 2048, 4095, 8192, 16383, 16384]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


def gapped_vector(nb, d, seed):
    """nb buckets of d coordinates: +-1.5 at positions whose distances cycle
    through GAPS (those that fit the bucket, rotated per bucket), 0 elsewhere."""
    rng = np.random.default_rng(seed)
    v = np.zeros(nb * d, dtype=np.float32)
    fit = [g for g in GAPS if g <= d]
    for b in range(nb):
        k = b % len(fit)
        pos = -1
        while True:
            pos += fit[k % len(fit)]
            if pos >= d:
                break
            v[b * d + pos] = 1.5 if rng.random() < 0.5 else -1.5
            k += 1
    return v


@pytest.mark.parametrize("code", [oracle.OMEGA, oracle.GAMMA])
@pytest.mark.parametrize("d,nb", [(512, 256), (4096, 40), (65536, 3)])
@pytest.mark.parametrize("s", [1, 15, 16, 64, 65535, (1 << 24) - 1])
def test_every_gap_and_level_structure(d, nb, s, code):
    v = gapped_vector(nb, d, 1000 + d + s % 997)
    print(f"long gaps d={d} nb={nb} s={s} code={code} nonzeros={int(np.count_nonzero(v))}", flush=True)
    g, info = check_parity(v, s, d, 5, code=code, norm=q.MAXNORM)
    assert info["norms_exact"] == info["nb"]
    # every non-zero decodes to +-1.5 (level s of scale 1.5) and the rest to +0
    want = np.where(v != 0, v, np.float32(0)).astype(np.float32)
    assert np.array_equal(g["v_hat"].view(np.uint32), want.view(np.uint32))
