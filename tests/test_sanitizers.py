"""CPU builds of the oracle and of the library's host-side planning under
AddressSanitizer and UndefinedBehaviorSanitizer, each driven by a small program
in tests/sanitize/ (no kernel is launched). The sanitizers abort on any
out-of-bounds access, use after free or undefined behaviour; the drivers also
check their results. The host build compiles the whole library (device code
included), so this test takes a minute or two."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    return r.stdout


@pytest.mark.slow
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"), os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "qsgd_oracle.c"), "-lm", "-o", exe])
    assert "ok" in _run([exe])


@pytest.mark.slow
@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not available")
def test_host_planning_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "host_san")
    csrc = os.path.join(ROOT, "quantized_sgd_amd", "csrc")
    _run(["/opt/rocm/bin/hipcc", "-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all",
          "-I", os.path.join(ROOT, "include"), "-I", csrc,
          os.path.join(csrc, "qsgd_api.hip"), os.path.join(SAN, "host_driver.cpp"), "-o", exe], timeout=900)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")  # the HIP runtime keeps its allocations to exit
    assert "ok" in _run([exe], env=env)
