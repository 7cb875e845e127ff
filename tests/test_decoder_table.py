"""The decoder's record table (quantized_sgd_amd/csrc/qsgd_decode.h, built at
compile time) against the oracle's codewords (page "QSGD (Quantized Stochastic
Gradient Descent) with Elias Coding": the record of a non-zero coordinate is
c(gap), its sign, c(level), with c Elias omega, or gamma).

A host program prints the 4096 entries of both codes; each is compared with the
entry derived here from the oracle's codeword functions: the window's bits are
parsed with the prefix-free code those functions define. The layout checked is
the one the table's comment states: one or two records of gap and level at most
16 that end within the 12 bits (total length, first length, gap - 1 and level
byte of each), or, with total length 0, the first field alone (its length and
value) when that codeword ends within the window, or, for an omega codeword
longer than the window, the bits and the value of its whole groups within it."""
import os
import shutil
import subprocess

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
W = 12

PROGRAM = r"""
#include "qsgd_decode.h"
#include <cstdio>
int main() {
    static constexpr qsgd::RecordLut t0 = qsgd::make_record_lut<0>();
    static constexpr qsgd::RecordLut t1 = qsgd::make_record_lut<1>();
    for (unsigned i = 0; i < (1u << qsgd::kLutBits); ++i) std::printf("%u %u\n", t0.e[i], t1.e[i]);
    return 0;
}
"""


@pytest.fixture(scope="module")
def tables(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    d = tmp_path_factory.mktemp("lut")
    src = d / "dump.hip"
    src.write_text(PROGRAM)
    exe = d / "dump"
    r = subprocess.run([HIPCC, "-std=c++17", "-O1", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
                        "-I", os.path.join(ROOT, "quantized_sgd_amd", "csrc"), "-o", str(exe), str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    rows = [tuple(int(x) for x in line.split()) for line in out if line.strip()]
    assert len(rows) == 1 << W
    return {oracle.OMEGA: [r[0] for r in rows], oracle.GAMMA: [r[1] for r in rows]}


def codewords(code):
    """Codeword (stream order) -> value, for the codewords of at most W bits."""
    out = {}
    for n in range(1, 300):
        cw = oracle.omega_codeword(n) if code == oracle.OMEGA else oracle.gamma_codeword(n)
        if len(cw) <= W:
            out[cw] = n
    return out


def expected_entry(i, cws):
    bits = "".join(str((i >> j) & 1) for j in range(W))  # stream bit j of the window is bit j of i

    def field(pos):
        for end in range(pos + 1, W + 1):
            if bits[pos:end] in cws:
                return cws[bits[pos:end]], end
        return None

    def record(pos):
        g = field(pos)
        if g is None or g[1] >= W:
            return None
        sign, q = int(bits[g[1]]), g[1] + 1
        k = field(q)
        if k is None or g[0] > 16 or k[0] > 16:
            return None
        return g[0], sign, k[0], k[1]

    r1 = record(0)
    if r1 is None:
        f = field(0)
        if f is not None:
            return (f[0] << 8) | (f[1] << 4)
        if cws is OMEGA_CWS:
            # an omega field past the window: the whole groups within it (a
            # group is a 1 bit and n more bits, n the value so far, starting at
            # 1; its bits are the new value), their length and the value they leave
            n, pos = 1, 0
            while pos < W and bits[pos] == "1" and pos + n + 1 <= W:
                n, pos = int(bits[pos:pos + n + 1], 2), pos + n + 1
            return (n << 20) | (pos << 16) if pos else 0
        return 0
    g, sg, k, l1 = r1
    e = l1 | (l1 << 4) | (((g - 1) | (((sg << 7) | k) << 4)) << 8)
    r2 = record(l1)
    if r2 is not None:
        g2, sg2, k2, end = r2
        e = (e & ~15) | end | (((g2 - 1) | (((sg2 << 7) | k2) << 4)) << 20)
    return e


OMEGA_CWS = codewords(oracle.OMEGA)


@pytest.mark.parametrize("code", [oracle.OMEGA, oracle.GAMMA])
def test_record_table_matches_the_codewords(tables, code):
    cws = OMEGA_CWS if code == oracle.OMEGA else codewords(code)
    # the codewords within the window: values up to 63 for both codes
    assert max(cws.values()) == 63
    got = tables[code]
    bad = [i for i in range(1 << W) if got[i] != expected_entry(i, cws)]
    assert not bad, [(i, got[i], expected_entry(i, cws)) for i in bad[:5]]
    # every kind of entry occurs: two records, one record, a field alone, nothing
    kinds = {("two" if (e & 15) > ((e >> 4) & 15) else "one") if e & 15 else
             ("field" if (e >> 4) & 15 else ("groups" if e else "none")) for e in got}
    assert kinds == ({"two", "one", "field", "groups"} if code == oracle.OMEGA else
                     {"two", "one", "field", "none"})
