"""GPU parity of buckets longer than a tile, up to the whole-vector operator
d = n (page "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding",
definition paragraph: Q_s is defined on a whole vector v in R^n; bucketing is
the paper's Section 3.3 extension). Such buckets span several 4096-coordinate
windows: their norms are folded from per-window partial sums, and a window's
first gap can reach back over earlier windows, across the pass-1 workgroups'
runs. Cases: d just over 4096, unaligned and aligned d, several buckets,
d = n up to a million coordinates, sparse vectors whose gaps cross many
windows, the max-norm scale and the gamma code."""
import numpy as np
import pytest
import torch

import oracle
import quantized_sgd_amd as q
from quantized_sgd_amd import workloads as wl
from tests.parity import check_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()


def sparse_vector(n, density, seed):
    rng = np.random.default_rng(seed)
    v = np.zeros(n, np.float32)
    idx = rng.choice(n, size=max(1, int(n * density)), replace=False)
    v[idx] = rng.standard_normal(idx.size).astype(np.float32)
    return v


@pytest.mark.parametrize("n,d,s,seed", [
    (4097, 4097, 4, 1),          # d = n, one coordinate past a tile
    (10000, 10000, 8, 2),
    (50000, 4097, 16, 3),        # several buckets, unaligned starts
    (100000, 8192, 64, 4),       # aligned
    (200003, 65536, 1, 5),
    (123457, 5000, 3, 6),        # s not a power of two
    (1_000_000, 1_000_000, 1000, 7),
])
def test_span_gaussian(n, d, s, seed):
    print(f"span gaussian n={n} d={d} s={s}", flush=True)
    check_parity(wl.small_gaussian(n, seed), s, d, seed)


@pytest.mark.parametrize("n,d,s,density,seed", [
    (300000, 300000, 1, 1e-4, 11),   # gaps of thousands of coordinates
    (600000, 150000, 4, 3e-5, 12),   # buckets with no non-zero level at all
    (500000, 500000, 2, 2e-3, 13),
])
def test_span_sparse(n, d, s, density, seed):
    print(f"span sparse n={n} d={d} s={s} density={density}", flush=True)
    check_parity(sparse_vector(n, density, seed), s, d, seed)


def test_span_maxnorm_and_gamma():
    print("span maxnorm / gamma", flush=True)
    check_parity(wl.small_gaussian(90000, 21), 64, 4500, 21, norm=q.MAXNORM)
    check_parity(wl.small_gaussian(70000, 22), 8, 20000, 22, code=oracle.GAMMA)
    check_parity(wl.mixed_values(60000, 23), 16, 60000, 23)
