"""QSGD oracle (test infrastructure only).

A plain, single-threaded CPU statement of the QSGD compressor, written in C
(`qsgd_oracle.c`) and wrapped here with ctypes + numpy. Only the test suite,
`__graft_entry__.smoke()` and the CPU-baseline leg of `bench.py` may use it; the
GPU library (`quantized_sgd_amd`) never imports it and shares no code with it.

What it computes, cited by page title and part of the page:
  * "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding" (AIMech
    curated page), definition paragraph: Q_s(v)_i = ||v||_2 sgn(v_i) xi_i(v, s)
    with xi_i = (l_i + 1)/s w.p. p_i else l_i/s, and Elias recursive coding of
    (norm, signs, non-zero gaps, levels k_i).
  * same page, claim on Elias coding: F = 32 bit norm, levels k_i in {1..s}.
  * same page, claim on bucketed training (paper Section 3.3): Q_s per bucket of
    d coordinates.
The floating-point and stream-layout readings are listed in `qsgd_oracle.h`.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsgd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u64p = ctypes.POINTER(ctypes.c_uint64)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)


def build() -> str:
    """Compile the oracle with gcc (single-threaded, IEEE, no contraction)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(
        ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
         "-fno-fast-math", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"],
        check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.or_philox4x32_10.argtypes = [_u32p, _u32p, _u32p]
        L.or_random_word.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.or_random_word.restype = ctypes.c_uint32
        L.or_random_words.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, _u32p]
        L.or_omega_length.argtypes = [ctypes.c_uint64]
        L.or_omega_length.restype = ctypes.c_uint
        L.or_omega_codeword.argtypes = [ctypes.c_uint64, ctypes.c_char_p]
        L.or_omega_codeword.restype = ctypes.c_uint
        L.or_uniform_buckets.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p]
        L.or_uniform_buckets.restype = ctypes.c_uint64
        L.or_ragged_buckets.argtypes = [_u64p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p]
        L.or_ragged_buckets.restype = ctypes.c_uint64
        L.or_bucket_norms.argtypes = [_f32p, _u64p, ctypes.c_uint64, _f32p]
        L.or_bucket_max_norms.argtypes = [_f32p, _u64p, ctypes.c_uint64, _f32p]
        L.or_quantize.argtypes = [_f32p, _u64p, ctypes.c_uint64, ctypes.c_uint32,
                                  ctypes.c_uint64, ctypes.c_void_p, _i32p, _f32p]
        L.or_quantize.restype = ctypes.c_int
        L.or_quantize_u24.argtypes = [_f32p, _u64p, ctypes.c_uint64, ctypes.c_uint32,
                                      _u32p, ctypes.c_void_p, _i32p, _f32p]
        L.or_quantize_u24.restype = ctypes.c_int
        L.or_dequantize.argtypes = [_i32p, _f32p, _u64p, ctypes.c_uint64, ctypes.c_uint32, _f32p]
        L.or_encode.argtypes = [_i32p, _f32p, _u64p, ctypes.c_uint64, ctypes.c_uint32,
                                _u64p, ctypes.c_uint64, _u64p, _u64p]
        L.or_encode.restype = ctypes.c_int
        L.or_decode.argtypes = [_u64p, ctypes.c_uint64, _u64p, _u64p, ctypes.c_uint64,
                                ctypes.c_uint32, _f32p]
        L.or_decode.restype = ctypes.c_int
        L.or_gamma_length.argtypes = [ctypes.c_uint64]
        L.or_gamma_length.restype = ctypes.c_uint
        L.or_gamma_codeword.argtypes = [ctypes.c_uint64, ctypes.c_char_p]
        L.or_gamma_codeword.restype = ctypes.c_uint
        L.or_encode_code.argtypes = [_i32p, _f32p, _u64p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int,
                                     _u64p, ctypes.c_uint64, _u64p, _u64p]
        L.or_encode_code.restype = ctypes.c_int
        L.or_decode_code.argtypes = [_u64p, ctypes.c_uint64, _u64p, _u64p, ctypes.c_uint64,
                                     ctypes.c_uint32, ctypes.c_int, _f32p]
        L.or_decode_code.restype = ctypes.c_int
        L.or_decode_accumulate.argtypes = [ctypes.c_void_p, _u64p, ctypes.c_void_p, ctypes.c_uint64,
                                           _u64p, ctypes.c_uint64, ctypes.c_uint32, _f32p, _f32p]
        L.or_decode_accumulate.restype = ctypes.c_int
        L.or_decode_accumulate_code.argtypes = [ctypes.c_void_p, _u64p, ctypes.c_void_p, ctypes.c_uint64,
                                                _u64p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, _f32p,
                                                _f32p]
        L.or_decode_accumulate_code.restype = ctypes.c_int
        _lib = L
    return _lib


OK, ERR_ARG, ERR_MALFORMED, ERR_CAPACITY = 0, 1, 2, 3


def _p(a, t):
    return a.ctypes.data_as(t)


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().or_philox4x32_10(_p(c, _u32p), _p(k, _u32p), _p(out, _u32p))
    return out


def random_word(seed: int, i: int) -> int:
    return int(lib().or_random_word(seed, i))


def random_words(seed: int, first: int, count: int) -> np.ndarray:
    out = np.zeros(count, dtype=np.uint32)
    lib().or_random_words(seed, first, count, _p(out, _u32p))
    return out


def omega_length(N: int) -> int:
    return int(lib().or_omega_length(N))


def omega_codeword(N: int) -> str:
    buf = ctypes.create_string_buffer(160)
    lib().or_omega_codeword(N, buf)
    return buf.value.decode()


def uniform_buckets(n: int, d: int) -> np.ndarray:
    nb = lib().or_uniform_buckets(n, d, None)
    b = np.zeros(nb + 1, dtype=np.uint64)
    lib().or_uniform_buckets(n, d, b.ctypes.data)
    return b


def ragged_buckets(seg_len, d: int) -> np.ndarray:
    sl = np.ascontiguousarray(seg_len, dtype=np.uint64)
    nb = lib().or_ragged_buckets(_p(sl, _u64p), len(sl), d, None)
    b = np.zeros(nb + 1, dtype=np.uint64)
    lib().or_ragged_buckets(_p(sl, _u64p), len(sl), d, b.ctypes.data)
    return b


def bucket_norms(v, bstart) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    bstart = np.ascontiguousarray(bstart, dtype=np.uint64)
    nb = len(bstart) - 1
    out = np.zeros(nb, dtype=np.float32)
    lib().or_bucket_norms(_p(v, _f32p), _p(bstart, _u64p), nb, _p(out, _f32p))
    return out


def bucket_max_norms(v, bstart) -> np.ndarray:
    """max|v_i| per bucket (the QSGDinf reading's scale)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    bstart = np.ascontiguousarray(bstart, dtype=np.uint64)
    nb = len(bstart) - 1
    out = np.zeros(max(nb, 1), dtype=np.float32)
    lib().or_bucket_max_norms(_p(v, _f32p), _p(bstart, _u64p), nb, _p(out, _f32p))
    return out[:nb]


def quantize(v, bstart, s: int, seed: int, norms=None, u24=None):
    """Returns (levels int32 = sgn * k, norms float32). Raises on bad input."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    bstart = np.ascontiguousarray(bstart, dtype=np.uint64)
    nb = len(bstart) - 1
    levels = np.zeros(len(v), dtype=np.int32)
    norms_out = np.zeros(nb, dtype=np.float32)
    given = None
    if norms is not None:
        norms = np.ascontiguousarray(norms, dtype=np.float32)
        given = norms.ctypes.data
    if u24 is None:
        rc = lib().or_quantize(_p(v, _f32p), _p(bstart, _u64p), nb, s, seed, given,
                               _p(levels, _i32p), _p(norms_out, _f32p))
    else:
        u = np.ascontiguousarray(u24, dtype=np.uint32)
        rc = lib().or_quantize_u24(_p(v, _f32p), _p(bstart, _u64p), nb, s, _p(u, _u32p),
                                   given, _p(levels, _i32p), _p(norms_out, _f32p))
    if rc != OK:
        raise ValueError(f"oracle quantize failed with status {rc}")
    return levels, norms_out


def dequantize(levels, norms, bstart, s: int) -> np.ndarray:
    levels = np.ascontiguousarray(levels, dtype=np.int32)
    norms = np.ascontiguousarray(norms, dtype=np.float32)
    bstart = np.ascontiguousarray(bstart, dtype=np.uint64)
    out = np.zeros(len(levels), dtype=np.float32)
    lib().or_dequantize(_p(levels, _i32p), _p(norms, _f32p), _p(bstart, _u64p),
                        len(bstart) - 1, s, _p(out, _f32p))
    return out


OMEGA, GAMMA = 0, 1  # integer codes of the record fields


def gamma_length(N: int) -> int:
    return int(lib().or_gamma_length(N))


def gamma_codeword(N: int) -> str:
    buf = ctypes.create_string_buffer(160)
    lib().or_gamma_codeword(N, buf)
    return buf.value.decode()


def code_length(N: int, code: int = OMEGA) -> int:
    return gamma_length(N) if code == GAMMA else omega_length(N)


def capacity_words(bstart, s: int, code: int = OMEGA) -> int:
    """A bound on the stream size: 32 bits per bucket plus, per coordinate, one
    code of a gap (at most the longest bucket), a sign and the code of s."""
    bstart = np.asarray(bstart, dtype=np.uint64)
    nb = len(bstart) - 1
    n = int(bstart[-1])
    dmax = int(np.max(np.diff(bstart))) if nb else 1
    bits = 32 * nb + n * (code_length(max(dmax, 1), code) + 1 + code_length(s, code))
    return bits // 64 + 2


def encode(levels, norms, bstart, s: int, code: int = OMEGA):
    """Returns (words uint64, offsets uint64[nb+1], out_bits)."""
    levels = np.ascontiguousarray(levels, dtype=np.int32)
    norms = np.ascontiguousarray(norms, dtype=np.float32)
    bstart = np.ascontiguousarray(bstart, dtype=np.uint64)
    nb = len(bstart) - 1
    cap = capacity_words(bstart, s, code)
    words = np.zeros(cap, dtype=np.uint64)
    offsets = np.zeros(nb + 1, dtype=np.uint64)
    out_bits = np.zeros(1, dtype=np.uint64)
    rc = lib().or_encode_code(_p(levels, _i32p), _p(norms, _f32p), _p(bstart, _u64p), nb, s, code,
                              _p(words, _u64p), cap, _p(offsets, _u64p), _p(out_bits, _u64p))
    if rc != OK:
        raise ValueError(f"oracle encode failed with status {rc}")
    nbits = int(out_bits[0])
    return words[: (nbits + 63) // 64].copy(), offsets, nbits


def decode(words, offsets, bstart, s: int, code: int = OMEGA):
    """Returns (status, v_hat float32)."""
    words = np.ascontiguousarray(words, dtype=np.uint64)
    if len(words) == 0:
        words = np.zeros(1, dtype=np.uint64)
        nwords = 0
    else:
        nwords = len(words)
    offsets = np.ascontiguousarray(offsets, dtype=np.uint64)
    bstart = np.ascontiguousarray(bstart, dtype=np.uint64)
    out = np.zeros(int(bstart[-1]), dtype=np.float32)
    if len(out) == 0:
        out = np.zeros(1, dtype=np.float32)
    rc = lib().or_decode_code(_p(words, _u64p), nwords, _p(offsets, _u64p), _p(bstart, _u64p),
                              len(bstart) - 1, s, code, _p(out, _f32p))
    return int(rc), out[: int(bstart[-1])]


def decode_accumulate(streams, bstart, s: int, acc, code: int = OMEGA):
    """streams: list of (words, offsets) of the record code `code`. Returns
    (status, acc + the decodes added in list order, one fp32 addition per
    stream and coordinate)."""
    bstart = np.ascontiguousarray(bstart, dtype=np.uint64)
    n = int(bstart[-1])
    out = np.array(acc, dtype=np.float32, copy=True)
    if n == 0:
        return OK, out
    ws = [np.ascontiguousarray(w, dtype=np.uint64) if len(w) else np.zeros(1, np.uint64) for w, _ in streams]
    nwords = np.array([len(w) for w, _ in streams] or [0], dtype=np.uint64)
    offs = [np.ascontiguousarray(o, dtype=np.uint64) for _, o in streams]
    k = len(streams)
    wp = (ctypes.c_void_p * max(k, 1))(*[w.ctypes.data for w in ws])
    op = (ctypes.c_void_p * max(k, 1))(*[o.ctypes.data for o in offs])
    scratch = np.zeros(n, dtype=np.float32)
    rc = lib().or_decode_accumulate_code(ctypes.addressof(wp), _p(nwords, _u64p), ctypes.addressof(op), k,
                                         _p(bstart, _u64p), len(bstart) - 1, s, code, _p(out, _f32p),
                                         _p(scratch, _f32p))
    return int(rc), out


def compress(v, bstart, s: int, seed: int, norms=None, code: int = OMEGA):
    """quantize + encode: (levels, norms, words, offsets, out_bits)."""
    levels, nrm = quantize(v, bstart, s, seed, norms=norms)
    words, offsets, nbits = encode(levels, nrm, bstart, s, code)
    return levels, nrm, words, offsets, nbits
