"""Parity helpers: run the HIP path through the C ABI and the oracle on the same
inputs and compare.

Comparison rules (the pages fix no precision; these follow from the arithmetic):
  * norms: fp64 sums of the same fp32 squares in a different order, rounded once
    to fp32 -- relative difference <= 1e-6 (in practice almost always 0 ulp);
  * given the GPU's norms, the oracle's levels, stream words, bucket offsets and
    bit count must be bit-identical to the GPU's;
  * decode output must be bit-identical to the oracle's dequantization.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import quantized_sgd_amd as q


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def u64(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint64)


def bucket_table(n, d, seg_len):
    if seg_len is None:
        return oracle.uniform_buckets(n, d)
    return oracle.ragged_buckets(seg_len, d)


def gpu_run(v: np.ndarray, s: int, d: int, seed: int, seg_len=None, code=oracle.OMEGA, norm=q.L2):
    vd = to_dev(v)
    if seg_len is None:
        lev, nrm = q.quantize(vd, s, d, seed, norm=norm)
        out, bits, offs = q.encode(vd, s, d, seed, code=code, norm=norm)
        torch.cuda.synchronize()
        nbits = int(bits.item())
        words = out[: (nbits + 63) // 64]
        vh = q.decode(out, offs, v.size, s, d, code=code)
    else:
        lay = q.RaggedLayout(seg_len, d)
        lev, nrm = q.quantize_ragged(vd, lay, s, seed, norm=norm)
        out, bits, offs = q.encode_ragged(vd, lay, s, seed, code=code, norm=norm)
        torch.cuda.synchronize()
        nbits = int(bits.item())
        words = out[: (nbits + 63) // 64]
        vh = q.decode_ragged(out, offs, lay, s, code=code)
    torch.cuda.synchronize()
    return dict(levels=lev.cpu().numpy(), norms=nrm.cpu().numpy(), words=u64(words),
                offsets=u64(offs), bits=nbits, v_hat=vh.cpu().numpy(), out=out)


def check_parity(v: np.ndarray, s: int, d: int, seed: int, seg_len=None, g=None, code=oracle.OMEGA,
                 norm=q.L2):
    """Full element-by-element parity of quantize, encode and decode (code: the
    integer code of the record fields; norm: the bucket scale, the max-norm
    being exact and so compared bit for bit)."""
    if g is None:
        g = gpu_run(v, s, d, seed, seg_len, code, norm)
    bst = bucket_table(v.size, d, seg_len)
    # norms
    on = oracle.bucket_norms(v, bst) if norm == q.L2 else oracle.bucket_max_norms(v, bst)
    gn = g["norms"]
    assert gn.shape == on.shape
    if norm != q.L2:
        assert np.array_equal(gn.view(np.uint32), on.view(np.uint32))
    rel = np.abs(gn.astype(np.float64) - on) / np.maximum(np.abs(on.astype(np.float64)), 1e-45)
    assert np.all(rel <= 1e-6), float(rel.max())
    # levels given the GPU norms
    olev, _ = oracle.quantize(v, bst, s, seed, norms=gn)
    assert np.array_equal(g["levels"], olev), np.flatnonzero(g["levels"] != olev)[:10]
    # stream given the GPU norms
    words, offs, nbits = oracle.encode(olev, gn, bst, s, code)
    assert g["bits"] == nbits
    assert np.array_equal(g["offsets"], offs)
    assert np.array_equal(g["words"], words), np.flatnonzero(g["words"] != words)[:10]
    # decode
    want = oracle.dequantize(olev, gn, bst, s)
    assert np.array_equal(g["v_hat"].view(np.uint32), want.view(np.uint32))
    rc, ovh = oracle.decode(words, offs, bst, s, code)
    assert rc == oracle.OK and np.array_equal(ovh.view(np.uint32), want.view(np.uint32))
    return g, dict(norms_exact=int(np.sum(gn == on)), nb=len(on))
