"""Seeded synthetic gradients shaped like the pages' workloads.

The pages ("QSGD: Communication-Efficient SGD via Gradient Quantization and
Encoding" abstract; the curated page's claim on bucketed training, Table 1 and
Figures 1-2) train ResNet-50/152-class CNNs and speech LSTMs on ImageNet,
CIFAR-10 and AN4; those datasets and trained gradients are not available, so
these generators stand in for them with gradients of the same sizes and value
mix. Nothing here computes any part of the compressor: these are only inputs
(numpy PCG64, drawn in float64 and cast to float32), shared by the tests, the
smoke check and the benchmark.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

CHUNK = 1 << 20  # "1M-element chunks": 2^20, so chunk edges fall on bucket edges


@dataclasses.dataclass
class Workload:
    name: str
    v: np.ndarray            # float32 gradient (flat)
    s: int                   # quantization levels
    d: int                   # bucket size
    seed: int                # Philox seed
    seg_len: np.ndarray | None = None  # per-tensor lengths (ragged batch) or None
    description: str = ""

    @property
    def n(self) -> int:
        return int(self.v.size)

    def sha256(self) -> str:
        return hashlib.sha256(self.v.tobytes()).hexdigest()


def chunked_gaussian(n: int, seed: int, lo_exp: float = -4.0, hi_exp: float = -1.0) -> np.ndarray:
    """Chunks of 2^20 coordinates, each N(0, sigma_c^2) with sigma_c log-uniform
    in [10^lo_exp, 10^hi_exp] (the last chunk is partial)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nchunks = (n + CHUNK - 1) // CHUNK
    sig = 10.0 ** rng.uniform(lo_exp, hi_exp, size=nchunks)
    out = np.empty(n, dtype=np.float32)
    for c in range(nchunks):
        a, b = c * CHUNK, min(n, (c + 1) * CHUNK)
        out[a:b] = (sig[c] * rng.standard_normal(b - a)).astype(np.float32)
    return out


def config1() -> Workload:
    rng = np.random.Generator(np.random.PCG64(0))
    v = rng.standard_normal(4096).astype(np.float32)
    return Workload("c1_n4096_s4_single_bucket", v, s=4, d=4096, seed=1,
                    description="one vector n=4096, N(0,1) from seed 0; s=4, d=n")


def config2() -> Workload:
    return Workload("c2_resnet50_n25557032_d512_s16", chunked_gaussian(25_557_032, 2), s=16, d=512,
                    seed=1, description="ResNet-50-sized gradient, chunked Gaussian, d=512, s=16")


def config3() -> Workload:
    return Workload("c3_resnet152_n60192808_d4096_s64", chunked_gaussian(60_192_808, 3), s=64,
                    d=4096, seed=1,
                    description="ResNet-152-sized gradient, chunked Gaussian, d=4096, s=64")


def config4(n: int = 1 << 28) -> Workload:
    rng = np.random.Generator(np.random.PCG64(4))
    v = np.empty(n, dtype=np.float32)
    step = 1 << 24
    for a in range(0, n, step):
        b = min(n, a + step)
        v[a:b] = (1e-3 * rng.standard_t(3, size=b - a)).astype(np.float32)
    return Workload("c4_heavytail_n268435456_d512_s1", v, s=1, d=512, seed=1,
                    description="2^28 coords, Student-t nu=3 scaled 1e-3; d=512, s=1")


def ragged_sizes(seed: int = 5, count: int = 150, lo: int = 64, hi: int = 4_194_304):
    rng = np.random.Generator(np.random.PCG64(seed))
    sizes = np.rint(np.exp(rng.uniform(np.log(lo), np.log(hi), size=count))).astype(np.int64)
    return rng, sizes


def config5() -> Workload:
    rng, sizes = ragged_sizes()
    sig = 10.0 ** rng.uniform(-5.0, -1.0, size=len(sizes))
    v = np.empty(int(sizes.sum()), dtype=np.float32)
    pos = 0
    for t, m in enumerate(sizes):
        v[pos:pos + m] = (sig[t] * rng.standard_normal(int(m))).astype(np.float32)
        pos += int(m)
    return Workload("c5_ragged150_d512_s8", v, s=8, d=512, seed=1, seg_len=sizes.astype(np.uint64),
                    description="150 tensors, sizes log-uniform in [64, 4194304], per-tensor sigma; d=512, s=8")


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def peer_gradient(cfg: int, j: int) -> np.ndarray:
    """Gradient of worker j for the decode-accumulate workloads (the gradients a
    receiver sums): same size and value mix as config 2 or 3, worker 0 being the
    config's own gradient."""
    n = {2: 25_557_032, 3: 60_192_808}[cfg]
    return chunked_gaussian(n, cfg + 100 * j)


def small_gaussian(n: int, seed: int, scale: float = 1.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return (scale * rng.standard_normal(n)).astype(np.float32)


def mixed_values(n: int, seed: int) -> np.ndarray:
    """Gaussian values with scales from 1e-38 to 1e30, exact zeros, negative zeros
    and fp32 subnormals: edge-case inputs for the parity tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    v = rng.standard_normal(n) * 10.0 ** rng.uniform(-30, 30, size=n)
    v = v.astype(np.float32)
    idx = rng.integers(0, n, size=max(1, n // 8))
    v[idx] = 0.0
    idx = rng.integers(0, n, size=max(1, n // 16))
    v[idx] = -0.0
    idx = rng.integers(0, n, size=max(1, n // 32))
    v[idx] = (rng.standard_normal(idx.size) * 1e-42).astype(np.float32)
    return v
