"""The C-ABI library loads and exports every entry point include/qsgd.h declares
(no compute calls: this runs without a GPU). Host-only helpers (bucket counts,
capacities, the ragged bucket table, argument checks) are exercised too."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import quantized_sgd_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "qsgd.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsgd_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(q.LIB_PATH)
    names = declared_functions()
    assert len(names) == 26
    for name in names:
        assert hasattr(lib, name), name


def test_library_is_built_for_gfx950():
    data = open(q.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_host_helpers_match_oracle_bucketing():
    for n, d in [(0, 4), (1, 1), (10, 3), (4096, 4096), (25_557_032, 512), (60_192_808, 4096)]:
        assert q.num_buckets(n, d) == len(oracle.uniform_buckets(n, d)) - 1
    rng = np.random.default_rng(3)
    seg = rng.integers(0, 5000, size=60)
    seg[[2, 9]] = 0
    lay_host = np.zeros(1)
    lib = q.lib()
    sl = np.ascontiguousarray(seg.astype(np.uint64))
    nb = lib.qsgd_num_buckets_ragged(sl.ctypes.data, len(sl), 512)
    tab = np.zeros(nb + 1, np.uint64)
    assert lib.qsgd_ragged_bucket_table(sl.ctypes.data, len(sl), 512, tab.ctypes.data, nb) == 0
    assert np.array_equal(tab, oracle.ragged_buckets(seg, 512))
    # a wrong nb is rejected
    assert lib.qsgd_ragged_bucket_table(sl.ctypes.data, len(sl), 512, tab.ctypes.data, nb + 1) == 1


def test_decode_accumulate_argument_checks():
    # rejected (or a no-op) on the host before anything touches a device
    lib = q.lib()
    assert lib.qsgd_max_streams() == 32
    k = 33
    ptrs = (ctypes.c_uint64 * k)(*([16] * k))
    addr = ctypes.addressof(ptrs)
    assert lib.qsgd_decode_accumulate(addr, addr, k, 100, 4, 16, 16, None) == 1    # too many streams
    assert lib.qsgd_decode_accumulate(None, None, 2, 100, 4, 16, 16, None) == 1    # no pointer arrays
    zero = (ctypes.c_uint64 * 2)(16, 0)
    assert lib.qsgd_decode_accumulate(ctypes.addressof(zero), addr, 2, 100, 4, 16, 16, None) == 1  # NULL entry
    assert lib.qsgd_decode_accumulate(addr, addr, 2, 100, 0, 16, 16, None) == 1    # s == 0
    assert lib.qsgd_decode_accumulate(addr, addr, 0, 100, 4, 16, 16, None) == 0    # k == 0: nothing to do
    assert lib.qsgd_decode_accumulate(addr, addr, 2, 0, 4, 16, 16, None) == 0      # n == 0: nothing to do
    assert lib.qsgd_decode_accumulate(addr, addr, 2, 100, 4, 16, 18, None) == 1    # acc not 16-byte aligned


def test_code_choice_argument_checks():
    # host-side rejections of the code-selecting calls (nothing is enqueued)
    lib = q.lib()
    assert lib.qsgd_encode_capacity_words_ex(1000, 2, 4, 512, 2) == 0          # unknown code
    assert lib.qsgd_encode_capacity_words_ex(1000, 2, 4, 512, q.GAMMA) > 0
    assert lib.qsgd_encode_ex(16, 1000, None, 3, 4, 512, 1, q.GAMMA, 0, 16, 16, 16, None) == 1  # nb != ceil(n/d)
    assert lib.qsgd_encode_ex(16, 1000, None, 2, 4, 512, 1, 7, 0, 16, 16, 16, None) == 1        # unknown code
    assert lib.qsgd_encode_ex(16, 1000, None, 2, 4, 512, 1, 0, 5, 16, 16, 16, None) == 1        # unknown norm
    assert lib.qsgd_quantize_ex(16, 1000, None, 2, 4, 512, 1, 5, 16, 16, None) == 1             # unknown norm
    assert lib.qsgd_quantize_ex(16, 1000, None, 3, 4, 512, 1, q.MAXNORM, 16, 16, None) == 1     # nb != ceil(n/d)
    assert lib.qsgd_decode_ex(16, 16, 1000, None, 3, 4, 512, q.GAMMA, 16, None) == 1        # nb != ceil(n/d)
    assert lib.qsgd_decode_ex(16, 16, 1000, None, 2, 4, 512, 9, 16, None) == 1              # unknown code


def test_capacity_bounds_oracle_streams():
    # the capacity helper bounds the worst case; check it against oracle streams
    for n, d, s in [(4096, 4096, 64), (5000, 1, 1 << 24), (10000, 7, 3), (20000, 512, 16),
                    # buckets longer than a tile (the span path), and d around its threshold
                    (100, 5000, 4), (20000, 5000, 3), (9000, 9000, 64), (13000, 4081, 8),
                    (13000, 4082, 8), (13000, 4095, 8), (13000, 4096, 8), (40000, 40000, 1)]:
        bst = oracle.uniform_buckets(n, d)
        for code in (oracle.OMEGA, oracle.GAMMA):
            cap = q.encode_capacity_words(n, s, d, code)
            for v in (np.full(n, 1.0, np.float32), np.random.default_rng(n).standard_normal(n).astype(np.float32)):
                _, _, _, _, nbits = oracle.compress(v, bst, s, 1, code=code)
                assert cap * 64 > nbits
    # uniform buckets of any length are served; ragged batches up to 4081
    assert q.encode_capacity_words(100, 4, 5000) > 0
    assert q.max_bucket() == 4081
    lib = q.lib()
    assert lib.qsgd_encode_capacity_words_ragged(100000, 20, 4, 5000) == 0
    assert lib.qsgd_encode_capacity_words_ragged(100000, 30, 4, 4081) > 0


def test_seglen_calls_refuse_more_tensors_than_the_arguments_hold():
    # more than 160 tensors: refused on the host before anything is enqueued
    lib = q.lib()
    seg = np.full(161, 100, np.uint64)
    assert lib.qsgd_quantize_seglen(16, seg.ctypes.data, 161, 4, 64, 1, 16, 16, None) == q.QSGD_ERR_UNSUPPORTED
    assert lib.qsgd_encode_seglen(16, seg.ctypes.data, 161, 4, 64, 1, 16, 16, 16, None) == q.QSGD_ERR_UNSUPPORTED
    assert lib.qsgd_decode_seglen(16, 16, seg.ctypes.data, 161, 4, 64, 16, None) == q.QSGD_ERR_UNSUPPORTED
    assert lib.qsgd_encode_seglen(16, None, 3, 4, 64, 1, 16, 16, 16, None) == q.QSGD_ERR_INVALID_ARG
    assert lib.qsgd_encode_seglen(16, seg.ctypes.data, 3, 4, 0, 1, 16, 16, 16, None) == q.QSGD_ERR_INVALID_ARG


def test_status_strings():
    lib = q.lib()
    assert lib.qsgd_status_string(0) == b"QSGD_OK"
    assert lib.qsgd_status_string(1) == b"QSGD_ERR_INVALID_ARG"


def test_no_cpu_fallback_in_product(monkeypatch, tmp_path):
    # the binding refuses to run without the HIP library
    monkeypatch.setattr(q, "_lib", None)
    monkeypatch.setattr(q, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        q.lib()


def test_product_does_not_import_oracle():
    pkg = os.path.join(ROOT, "quantized_sgd_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "qsgd_oracle" not in text, f


def test_binding_refuses_short_buffers_before_any_device_work():
    # the wrappers compare buffer sizes with what the call writes; a CPU tensor
    # is enough to see the refusal, which comes before the device check
    import torch
    v = torch.zeros(1000)
    with pytest.raises(ValueError):
        q.quantize(v, 4, 100, 1, levels=torch.zeros(999, dtype=torch.int32), norms=torch.zeros(10))
    with pytest.raises(ValueError):
        q.quantize(v, 4, 100, 1, levels=torch.zeros(1000, dtype=torch.int32), norms=torch.zeros(9))
    with pytest.raises(ValueError):
        q.encode(v, 4, 100, 1, offsets=torch.zeros(10, dtype=torch.int64))
    with pytest.raises(ValueError):
        q.decode(torch.zeros(4, dtype=torch.int64), torch.zeros(11, dtype=torch.int64), 1000, 4, 100,
                 v_hat=torch.zeros(999))
    with pytest.raises(ValueError):
        q.decode(torch.zeros(4, dtype=torch.int64), torch.zeros(10, dtype=torch.int64), 1000, 4, 100,
                 v_hat=torch.zeros(1000))
