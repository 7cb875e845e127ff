"""MI355X-native QSGD compressor: thin Python binding over libqsgd.so.

Every step of the compressor runs in the HIP kernels behind the C ABI of
include/qsgd.h; this module only marshals torch tensors (device memory and the
current HIP stream) into those calls. There is no CPU fallback: if the library
is not built, every entry point raises.

Method: page "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding"
(definition paragraph; claims on Elias coding and on bucketed training).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "QsgdError", "lib", "num_buckets", "encode_capacity_words", "quantize", "encode",
    "decode", "RaggedLayout", "quantize_ragged", "encode_ragged", "decode_ragged",
    "max_bucket", "max_streams", "decode_accumulate", "decode_accumulate_ragged", "OMEGA", "GAMMA",
    "L2", "MAXNORM", "encode_noalloc", "encode_noalloc_capacity_words", "quantize_seglen", "encode_seglen",
    "decode_seglen",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsgd.so")
_lib = None

_u64 = ctypes.c_uint64
_u32 = ctypes.c_uint32
_vp = ctypes.c_void_p

QSGD_OK, QSGD_ERR_INVALID_ARG, QSGD_ERR_LAUNCH, QSGD_ERR_UNSUPPORTED, QSGD_ERR_SCRATCH = 0, 1, 2, 3, 4
OMEGA, GAMMA = 0, 1  # integer code of the record fields (qsgd_code)
L2, MAXNORM = 0, 1   # bucket scale (qsgd_norm): ||v||_2, or max|v_i| (QSGDinf)


class QsgdError(RuntimeError):
    def __init__(self, status: int, what: str):
        name = lib().qsgd_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{what}: {name}")
        self.status = status


def lib():
    """Loads libqsgd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m quantized_sgd_amd.build` "
                "(the QSGD compressor has no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        L.qsgd_status_string.argtypes = [ctypes.c_int]
        L.qsgd_status_string.restype = ctypes.c_char_p
        L.qsgd_num_buckets.argtypes = [_u64, _u32]
        L.qsgd_num_buckets.restype = _u64
        L.qsgd_max_bucket.argtypes = []
        L.qsgd_max_bucket.restype = _u32
        L.qsgd_encode_capacity_words.argtypes = [_u64, _u32, _u32]
        L.qsgd_encode_capacity_words.restype = _u64
        L.qsgd_encode_capacity_words_ragged.argtypes = [_u64, _u64, _u32, _u32]
        L.qsgd_encode_capacity_words_ragged.restype = _u64
        L.qsgd_quantize.argtypes = [_vp, _u64, _u32, _u32, _u64, _vp, _vp, _vp]
        L.qsgd_encode.argtypes = [_vp, _u64, _u32, _u32, _u64, _vp, _vp, _vp, _vp]
        L.qsgd_decode.argtypes = [_vp, _vp, _u64, _u32, _u32, _vp, _vp]
        L.qsgd_num_buckets_ragged.argtypes = [_vp, _u32, _u32]
        L.qsgd_num_buckets_ragged.restype = _u64
        L.qsgd_ragged_bucket_table.argtypes = [_vp, _u32, _u32, _vp, _u64]
        L.qsgd_quantize_ragged.argtypes = [_vp, _u64, _vp, _u64, _u32, _u32, _u64, _vp, _vp, _vp]
        L.qsgd_encode_ragged.argtypes = [_vp, _u64, _vp, _u64, _u32, _u32, _u64, _vp, _vp, _vp, _vp]
        L.qsgd_decode_ragged.argtypes = [_vp, _vp, _u64, _vp, _u64, _u32, _u32, _vp, _vp]
        L.qsgd_encode_capacity_words_ex.argtypes = [_u64, _u64, _u32, _u32, ctypes.c_int]
        L.qsgd_encode_capacity_words_ex.restype = _u64
        L.qsgd_encode_ex.argtypes = [_vp, _u64, _vp, _u64, _u32, _u32, _u64, ctypes.c_int, ctypes.c_int,
                                     _vp, _vp, _vp, _vp]
        L.qsgd_quantize_ex.argtypes = [_vp, _u64, _vp, _u64, _u32, _u32, _u64, ctypes.c_int, _vp, _vp, _vp]
        L.qsgd_decode_ex.argtypes = [_vp, _vp, _u64, _vp, _u64, _u32, _u32, ctypes.c_int, _vp, _vp]
        L.qsgd_max_streams.argtypes = []
        L.qsgd_max_streams.restype = _u32
        L.qsgd_decode_accumulate.argtypes = [_vp, _vp, _u32, _u64, _u32, _u32, _vp, _vp]
        L.qsgd_decode_accumulate_ragged.argtypes = [_vp, _vp, _u32, _u64, _vp, _u64, _u32, _u32, _vp, _vp]
        L.qsgd_decode_accumulate_ex.argtypes = [_vp, _vp, _u32, _u64, _vp, _u64, _u32, _u32, ctypes.c_int, _vp, _vp]
        L.qsgd_quantize_seglen.argtypes = [_vp, _vp, _u32, _u32, _u32, _u64, _vp, _vp, _vp]
        L.qsgd_encode_seglen.argtypes = [_vp, _vp, _u32, _u32, _u32, _u64, _vp, _vp, _vp, _vp]
        L.qsgd_decode_seglen.argtypes = [_vp, _vp, _vp, _u32, _u32, _u32, _vp, _vp]
        L.qsgd_encode_noalloc_capacity_words.argtypes = [_u64, _u32, _u32]
        L.qsgd_encode_noalloc_capacity_words.restype = _u64
        L.qsgd_encode_noalloc.argtypes = [_vp, _u64, _u32, _u32, _u64, _vp, _vp, _vp, _vp]
        for name in ("qsgd_encode_noalloc", "qsgd_decode_accumulate_ex", "qsgd_quantize_seglen",
                     "qsgd_encode_seglen", "qsgd_decode_seglen", "qsgd_quantize", "qsgd_encode", "qsgd_decode", "qsgd_ragged_bucket_table",
                     "qsgd_quantize_ragged", "qsgd_encode_ragged", "qsgd_decode_ragged",
                     "qsgd_decode_accumulate", "qsgd_decode_accumulate_ragged", "qsgd_encode_ex",
                     "qsgd_decode_ex", "qsgd_quantize_ex"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != QSGD_OK:
        raise QsgdError(status, what)


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _need(t: torch.Tensor, count: int, name: str):
    """Raises before any device work when a buffer holds fewer than `count`
    elements (the kernels would write past it)."""
    if t.numel() < count:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {count}")


def _dev(t: torch.Tensor, dtype, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def num_buckets(n: int, d: int) -> int:
    return int(lib().qsgd_num_buckets(n, d))


def max_bucket() -> int:
    return int(lib().qsgd_max_bucket())


def encode_capacity_words(n: int, s: int, d: int, code: int = OMEGA) -> int:
    if code == OMEGA:
        return int(lib().qsgd_encode_capacity_words(n, s, d))
    return int(lib().qsgd_encode_capacity_words_ex(n, num_buckets(n, d), s, d, code))


def quantize(v: torch.Tensor, s: int, d: int, seed: int, levels=None, norms=None, stream=None,
             norm: int = L2):
    """Q_s per bucket: returns (levels int32 = sgn * k, norms float32). norm:
    L2 (qsgd_quantize) or MAXNORM (qsgd_quantize_ex, the QSGDinf reading)."""
    n = v.numel()
    nb = num_buckets(n, d)
    if levels is None:
        levels = torch.empty(n, dtype=torch.int32, device=v.device)
    if norms is None:
        norms = torch.empty(max(nb, 1), dtype=torch.float32, device=v.device)
    _need(levels, n, "levels")
    _need(norms, nb, "norms")
    if norm == L2:
        _check(lib().qsgd_quantize(_dev(v, torch.float32, "v"), n, s, d, seed,
                                   _dev(levels, torch.int32, "levels"),
                                   _dev(norms, torch.float32, "norms"), _stream(stream)),
               "qsgd_quantize")
    else:
        _check(lib().qsgd_quantize_ex(_dev(v, torch.float32, "v"), n, None, nb, s, d, seed, norm,
                                      _dev(levels, torch.int32, "levels"),
                                      _dev(norms, torch.float32, "norms"), _stream(stream)),
               "qsgd_quantize_ex")
    return levels, norms[:nb]


def encode(v: torch.Tensor, s: int, d: int, seed: int, out=None, out_bits=None, offsets=None,
           stream=None, code: int = OMEGA, norm: int = L2):
    """Returns (out words, out_bits [1], bucket bit offsets [nb + 1]) as device
    tensors (uint64 data in int64 tensors). The stream is out[: ceil(bits/64)].
    code OMEGA and norm L2 use qsgd_encode; other choices qsgd_encode_ex."""
    n = v.numel()
    nb = num_buckets(n, d)
    cap = encode_capacity_words(n, s, d, code)
    if cap == 0:
        raise QsgdError(QSGD_ERR_UNSUPPORTED, "qsgd_encode_capacity_words")
    if out is None:
        out = torch.empty(cap, dtype=torch.int64, device=v.device)
    elif out.numel() < cap:
        raise ValueError(f"out holds {out.numel()} words, needs {cap}")
    if out_bits is None:
        out_bits = torch.empty(1, dtype=torch.int64, device=v.device)
    if offsets is None:
        offsets = torch.empty(nb + 1, dtype=torch.int64, device=v.device)
    _need(out_bits, 1, "out_bits")
    _need(offsets, nb + 1, "offsets")
    if code == OMEGA and norm == L2:
        _check(lib().qsgd_encode(_dev(v, torch.float32, "v"), n, s, d, seed,
                                 _dev(out, torch.int64, "out"), _dev(out_bits, torch.int64, "out_bits"),
                                 _dev(offsets, torch.int64, "offsets"), _stream(stream)),
               "qsgd_encode")
    else:
        _check(lib().qsgd_encode_ex(_dev(v, torch.float32, "v"), n, None, nb, s, d, seed, code, norm,
                                    _dev(out, torch.int64, "out"), _dev(out_bits, torch.int64, "out_bits"),
                                    _dev(offsets, torch.int64, "offsets"), _stream(stream)),
               "qsgd_encode_ex")
    return out, out_bits, offsets


def decode(words: torch.Tensor, offsets: torch.Tensor, n: int, s: int, d: int, v_hat=None,
           stream=None, code: int = OMEGA):
    """Decodes a stream written by encode (with the same code) back to Q_s(v)
    (float32 [n])."""
    if v_hat is None:
        v_hat = torch.empty(n, dtype=torch.float32, device=words.device)
    _need(v_hat, n, "v_hat")
    _need(offsets, num_buckets(n, d) + 1, "offsets")
    if code == OMEGA:
        _check(lib().qsgd_decode(_dev(words, torch.int64, "words"), _dev(offsets, torch.int64, "offsets"),
                                 n, s, d, _dev(v_hat, torch.float32, "v_hat"), _stream(stream)),
               "qsgd_decode")
    else:
        _check(lib().qsgd_decode_ex(_dev(words, torch.int64, "words"), _dev(offsets, torch.int64, "offsets"),
                                    n, None, num_buckets(n, d), s, d, code,
                                    _dev(v_hat, torch.float32, "v_hat"), _stream(stream)),
               "qsgd_decode_ex")
    return v_hat


def max_streams() -> int:
    return int(lib().qsgd_max_streams())


def _pointer_arrays(words_list, offsets_list):
    if len(words_list) != len(offsets_list):
        raise ValueError("one offsets tensor per stream")
    k = len(words_list)
    ins = (ctypes.c_uint64 * max(k, 1))(*[_dev(w, torch.int64, "words") for w in words_list])
    offs = (ctypes.c_uint64 * max(k, 1))(*[_dev(o, torch.int64, "offsets") for o in offsets_list])
    return k, ins, offs


def decode_accumulate(words_list, offsets_list, n: int, s: int, d: int, acc: torch.Tensor,
                      stream=None, code: int = OMEGA):
    """acc += the decodes of the streams (all of record code `code`), added in
    list order per coordinate (one fp32 rounding per addition); returns acc."""
    k, ins, offs = _pointer_arrays(words_list, offsets_list)
    _need(acc, n, "acc")
    for o in offsets_list:
        _need(o, num_buckets(n, d) + 1, "offsets")
    if code == OMEGA:
        _check(lib().qsgd_decode_accumulate(ctypes.addressof(ins), ctypes.addressof(offs), k, n, s, d,
                                            _dev(acc, torch.float32, "acc"), _stream(stream)),
               "qsgd_decode_accumulate")
    else:
        _check(lib().qsgd_decode_accumulate_ex(ctypes.addressof(ins), ctypes.addressof(offs), k, n, None,
                                               num_buckets(n, d), s, d, code, _dev(acc, torch.float32, "acc"),
                                               _stream(stream)),
               "qsgd_decode_accumulate_ex")
    return acc


class RaggedLayout:
    """Bucket layout of a batch of tensors laid out back to back in one buffer:
    buckets of at most d coordinates that restart at every tensor."""

    def __init__(self, seg_len, d: int, device="cuda"):
        import numpy as np
        sl = np.ascontiguousarray(np.asarray(seg_len, dtype=np.uint64))
        self.d = int(d)
        self.n = int(sl.sum())
        self.nseg = len(sl)
        nb = int(lib().qsgd_num_buckets_ragged(sl.ctypes.data, len(sl), d))
        table = np.zeros(nb + 1, dtype=np.uint64)
        _check(lib().qsgd_ragged_bucket_table(sl.ctypes.data, len(sl), d, table.ctypes.data, nb),
               "qsgd_ragged_bucket_table")
        self.nb = nb
        self.bucket_start_host = table
        self.bucket_start = torch.from_numpy(table.view(np.int64)).to(device)

    def capacity_words(self, s: int, code: int = OMEGA) -> int:
        if code == OMEGA:
            return int(lib().qsgd_encode_capacity_words_ragged(self.n, self.nb, s, self.d))
        return int(lib().qsgd_encode_capacity_words_ex(self.n, self.nb, s, self.d, code))


def quantize_ragged(v: torch.Tensor, layout: RaggedLayout, s: int, seed: int, stream=None,
                    norm: int = L2):
    _need(v, layout.n, "v")
    levels = torch.empty(layout.n, dtype=torch.int32, device=v.device)
    norms = torch.empty(max(layout.nb, 1), dtype=torch.float32, device=v.device)
    bs = _dev(layout.bucket_start, torch.int64, "bucket_start")
    if norm == L2:
        _check(lib().qsgd_quantize_ragged(_dev(v, torch.float32, "v"), layout.n, bs, layout.nb, s,
                                          layout.d, seed, _dev(levels, torch.int32, "levels"),
                                          _dev(norms, torch.float32, "norms"), _stream(stream)),
               "qsgd_quantize_ragged")
    else:
        _check(lib().qsgd_quantize_ex(_dev(v, torch.float32, "v"), layout.n, bs, layout.nb, s, layout.d,
                                      seed, norm, _dev(levels, torch.int32, "levels"),
                                      _dev(norms, torch.float32, "norms"), _stream(stream)),
               "qsgd_quantize_ex")
    return levels, norms[: layout.nb]


def encode_ragged(v: torch.Tensor, layout: RaggedLayout, s: int, seed: int, out=None, out_bits=None,
                  offsets=None, stream=None, code: int = OMEGA, norm: int = L2):
    cap = layout.capacity_words(s, code)
    if cap == 0:
        raise QsgdError(QSGD_ERR_UNSUPPORTED, "qsgd_encode_capacity_words_ragged")
    if out is None:
        out = torch.empty(cap, dtype=torch.int64, device=v.device)
    if out_bits is None:
        out_bits = torch.empty(1, dtype=torch.int64, device=v.device)
    if offsets is None:
        offsets = torch.empty(layout.nb + 1, dtype=torch.int64, device=v.device)
    _need(out, cap, "out")
    _need(out_bits, 1, "out_bits")
    _need(offsets, layout.nb + 1, "offsets")
    _need(v, layout.n, "v")
    if code == OMEGA and norm == L2:
        _check(lib().qsgd_encode_ragged(_dev(v, torch.float32, "v"), layout.n,
                                        _dev(layout.bucket_start, torch.int64, "bucket_start"), layout.nb,
                                        s, layout.d, seed, _dev(out, torch.int64, "out"),
                                        _dev(out_bits, torch.int64, "out_bits"),
                                        _dev(offsets, torch.int64, "offsets"), _stream(stream)),
               "qsgd_encode_ragged")
    else:
        _check(lib().qsgd_encode_ex(_dev(v, torch.float32, "v"), layout.n,
                                    _dev(layout.bucket_start, torch.int64, "bucket_start"), layout.nb,
                                    s, layout.d, seed, code, norm, _dev(out, torch.int64, "out"),
                                    _dev(out_bits, torch.int64, "out_bits"),
                                    _dev(offsets, torch.int64, "offsets"), _stream(stream)),
               "qsgd_encode_ex")
    return out, out_bits, offsets


def decode_ragged(words: torch.Tensor, offsets: torch.Tensor, layout: RaggedLayout, s: int,
                  v_hat=None, stream=None, code: int = OMEGA):
    if v_hat is None:
        v_hat = torch.empty(layout.n, dtype=torch.float32, device=words.device)
    _need(v_hat, layout.n, "v_hat")
    _need(offsets, layout.nb + 1, "offsets")
    bs = _dev(layout.bucket_start, torch.int64, "bucket_start")
    if code == OMEGA:
        _check(lib().qsgd_decode_ragged(_dev(words, torch.int64, "words"),
                                        _dev(offsets, torch.int64, "offsets"), layout.n, bs, layout.nb,
                                        s, layout.d, _dev(v_hat, torch.float32, "v_hat"), _stream(stream)),
               "qsgd_decode_ragged")
    else:
        _check(lib().qsgd_decode_ex(_dev(words, torch.int64, "words"), _dev(offsets, torch.int64, "offsets"),
                                    layout.n, bs, layout.nb, s, layout.d, code,
                                    _dev(v_hat, torch.float32, "v_hat"), _stream(stream)),
               "qsgd_decode_ex")
    return v_hat


def decode_accumulate_ragged(words_list, offsets_list, layout: RaggedLayout, s: int, acc: torch.Tensor,
                             stream=None):
    """Ragged decode_accumulate."""
    k, ins, offs = _pointer_arrays(words_list, offsets_list)
    _need(acc, layout.n, "acc")
    for o in offsets_list:
        _need(o, layout.nb + 1, "offsets")
    _check(lib().qsgd_decode_accumulate_ragged(ctypes.addressof(ins), ctypes.addressof(offs), k, layout.n,
                                               _dev(layout.bucket_start, torch.int64, "bucket_start"),
                                               layout.nb, s, layout.d, _dev(acc, torch.float32, "acc"),
                                               _stream(stream)),
           "qsgd_decode_accumulate_ragged")
    return acc


def encode_noalloc_capacity_words(n: int, s: int, d: int) -> int:
    """Words `out` must hold for encode_noalloc (0: the workspace of (n, s, d)
    exceeds the library's fixed scratch)."""
    return int(lib().qsgd_encode_noalloc_capacity_words(n, s, d))


def encode_noalloc(v: torch.Tensor, s: int, d: int, seed: int, out: torch.Tensor, out_bits: torch.Tensor,
                   offsets: torch.Tensor, stream=None):
    """qsgd_encode_noalloc: encode with the workspace in the library's fixed
    scratch; every buffer is the caller's (out: encode_noalloc_capacity_words
    words, out_bits: 1, offsets: num_buckets + 1)."""
    n = v.numel()
    cap = encode_noalloc_capacity_words(n, s, d)
    if cap and out.numel() < cap:
        raise ValueError(f"out holds {out.numel()} words, needs {cap}")
    if out_bits.numel() < 1:
        raise ValueError("out_bits needs 1 word")
    if offsets.numel() < num_buckets(n, d) + 1:
        raise ValueError(f"offsets holds {offsets.numel()} words, needs {num_buckets(n, d) + 1}")
    _check(lib().qsgd_encode_noalloc(_dev(v, torch.float32, "v"), n, s, d, seed,
                                     _dev(out, torch.int64, "out"), _dev(out_bits, torch.int64, "out_bits"),
                                     _dev(offsets, torch.int64, "offsets"), _stream(stream)),
           "qsgd_encode_noalloc")
    return out, out_bits, offsets


def _seg_lengths(seg_len):
    import numpy as np
    return np.ascontiguousarray(np.asarray(seg_len, dtype=np.uint64))


def quantize_seglen(v: torch.Tensor, seg_len, s: int, d: int, seed: int, stream=None):
    """qsgd_quantize_seglen: the ragged quantize with the layout given by the
    host tensor lengths (at most 160 tensors). Returns (levels, norms)."""
    sl = _seg_lengths(seg_len)
    n = int(sl.sum())
    if v.numel() < n:
        raise ValueError(f"v holds {v.numel()} values, the lengths sum to {n}")
    nb = int(lib().qsgd_num_buckets_ragged(sl.ctypes.data, len(sl), d))
    levels = torch.empty(max(n, 1), dtype=torch.int32, device=v.device)
    norms = torch.empty(max(nb, 1), dtype=torch.float32, device=v.device)
    _check(lib().qsgd_quantize_seglen(_dev(v, torch.float32, "v"), sl.ctypes.data, len(sl), s, d, seed,
                                      _dev(levels, torch.int32, "levels"), _dev(norms, torch.float32, "norms"),
                                      _stream(stream)), "qsgd_quantize_seglen")
    return levels[:n], norms[:nb]


def encode_seglen(v: torch.Tensor, seg_len, s: int, d: int, seed: int, stream=None):
    """qsgd_encode_seglen: returns (out words, out_bits [1], offsets [nb + 1])."""
    sl = _seg_lengths(seg_len)
    n = int(sl.sum())
    if v.numel() < n:
        raise ValueError(f"v holds {v.numel()} values, the lengths sum to {n}")
    nb = int(lib().qsgd_num_buckets_ragged(sl.ctypes.data, len(sl), d))
    cap = int(lib().qsgd_encode_capacity_words_ragged(n, nb, s, d))
    if cap == 0:
        raise QsgdError(QSGD_ERR_UNSUPPORTED, "qsgd_encode_capacity_words_ragged")
    out = torch.empty(cap, dtype=torch.int64, device=v.device)
    out_bits = torch.empty(1, dtype=torch.int64, device=v.device)
    offsets = torch.empty(nb + 1, dtype=torch.int64, device=v.device)
    _check(lib().qsgd_encode_seglen(_dev(v, torch.float32, "v"), sl.ctypes.data, len(sl), s, d, seed,
                                    _dev(out, torch.int64, "out"), _dev(out_bits, torch.int64, "out_bits"),
                                    _dev(offsets, torch.int64, "offsets"), _stream(stream)), "qsgd_encode_seglen")
    return out, out_bits, offsets


def decode_seglen(words: torch.Tensor, offsets: torch.Tensor, seg_len, s: int, d: int, stream=None):
    """qsgd_decode_seglen: the ragged decode with host tensor lengths."""
    sl = _seg_lengths(seg_len)
    n = int(sl.sum())
    nb = int(lib().qsgd_num_buckets_ragged(sl.ctypes.data, len(sl), d))
    if offsets.numel() < nb + 1:
        raise ValueError(f"offsets holds {offsets.numel()} words, needs {nb + 1}")
    v_hat = torch.empty(max(n, 1), dtype=torch.float32, device=words.device)
    _check(lib().qsgd_decode_seglen(_dev(words, torch.int64, "words"), _dev(offsets, torch.int64, "offsets"),
                                    sl.ctypes.data, len(sl), s, d, _dev(v_hat, torch.float32, "v_hat"),
                                    _stream(stream)), "qsgd_decode_seglen")
    return v_hat[:n]
