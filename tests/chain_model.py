"""A CPU model of the decoder's parallel parse of one bucket: the 12-bit record
table (one or two records of gap and level at most 16), the general-path
record, the guess steps of speculative starts, the positions noted in the
first 128 bits of a segment, the meet search and the parallel repair rounds,
replayed on a stream the oracle built. It counts what the parse does (steps
per lane, sync distances, restarts, rounds) so that a test can show which of
the decoder's paths an input exercises. It follows the step rules of
quantized_sgd_amd/csrc/qsgd_decode.h; it decodes no values and checks none.

Test infrastructure: used by tests only.
"""
from __future__ import annotations

import os
import re

import numpy as np

_DECODER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "quantized_sgd_amd", "csrc", "qsgd_decode.h")


def _decoder_constant(pattern: str) -> int:
    """A constant of the decoder's source, so that the model follows it."""
    with open(_DECODER) as f:
        m = re.search(pattern, f.read())
    if m is None:
        raise RuntimeError(f"decoder constant not found: {pattern}")
    return int(m.group(1))


TABLE_BITS = _decoder_constant(r"constexpr int kLutBits = (\d+);")
FIELD_MAX = 16  # the table's largest gap and level: four bits each in an entry
SYNC_BITS = _decoder_constant(r"constexpr int kSyncWin = (\d+);")
GUESS_STEPS = _decoder_constant(r"#define QSGD_GUESS_STEPS (\d+)")
GUESS_BITS_PER_COORD = _decoder_constant(r"constexpr uint32_t kGuessBits = (\d+);")
GUESS_MIN_BITS_PER_COORD = _decoder_constant(r"constexpr uint32_t kGuessMinBits = (\d+);")


def stream_bits(words) -> list:
    """Stream bit t (MSB-first in uint64 words) at index t, with zero padding."""
    b = np.unpackbits(np.asarray(words, dtype=np.uint64).byteswap().view(np.uint8))
    return np.concatenate([b, np.zeros(4096, np.uint8)]).tolist()


def _field(bits, p, code, lim=None, cap=None):
    """Elias omega (code 0) or gamma (code 1) value at p: (N, end), or None when
    it runs past lim or exceeds cap."""
    if code == 0:
        n = 1
        while True:
            if lim is not None and p >= lim:
                return None
            if bits[p] == 0:
                return n, p + 1
            g = n + 1
            if lim is not None and p + g > lim:
                return None
            v = 0
            for i in range(g):
                v = (v << 1) | bits[p + i]
            n, p = v, p + g
            if cap is not None and n > cap:
                return None
    z = 0
    while True:
        if lim is not None and p + z >= lim:
            return None
        if bits[p + z]:
            break
        z += 1
        if z > 31:
            return None
    if lim is not None and p + 2 * z + 1 > lim:
        return None
    v = 0
    for i in range(z + 1):
        v = (v << 1) | bits[p + z + i]
    if cap is not None and v > cap:
        return None
    return v, p + 2 * z + 1


class Bucket:
    """One bucket's payload [P0, E) in a stream, with the decoder's parameters."""

    def __init__(self, bits, start, end, length, s, code=0, team=64):
        self.bits, self.E, self.len, self.s, self.code = bits, end, length, s, code
        self.P0 = start + 32
        lp = end - self.P0
        self.nl = max(1, min(team, lp // SYNC_BITS)) if lp > 0 else 0
        self.seg = (lp + self.nl - 1) // self.nl if self.nl else 0
        self.guess = GUESS_MIN_BITS_PER_COORD * length <= lp <= GUESS_BITS_PER_COORD * length
        self.gbits = max(1, int(length).bit_length())
        self.kbits = int(s).bit_length()
        self._table = {}

    def entry(self, p):
        """Table entry at p: (total length, first length, gap1, gap2) or None."""
        if p not in self._table:
            lim = p + TABLE_BITS

            def rec(q):
                g = _field(self.bits, q, self.code, lim, FIELD_MAX)
                if g is None or g[1] >= lim:
                    return None
                k = _field(self.bits, g[1] + 1, self.code, lim, FIELD_MAX)
                return None if k is None else (g[0], k[1])

            r1 = rec(p)
            e = None
            if r1 is not None:
                r2 = rec(r1[1])
                e = (r1[1] - p, r1[1] - p, r1[0], 0) if r2 is None else (r2[1] - p, r1[1] - p, r1[0], r2[0])
            self._table[p] = e
        return self._table[p]

    def slow(self, p):
        """General-path record at p: (end, gap), or (0, 0) if none parses."""
        if self.code == 0:
            def f(q, mb):
                n = 1
                while True:
                    if self.bits[q] == 0:
                        return n, q + 1
                    g = n + 1
                    if g > mb:
                        return 0, q
                    v = 0
                    for i in range(g):
                        v = (v << 1) | self.bits[q + i]
                    n, q = v, q + g
        else:
            def f(q, mb):
                z = 0
                while self.bits[q + z] == 0 and z < 32:
                    z += 1
                if z + 1 > mb:
                    return 0, q
                v = 0
                for i in range(z + 1):
                    v = (v << 1) | self.bits[q + z + i]
                return v, q + 2 * z + 1
        g, q = f(p, self.gbits)
        if g == 0:
            return 0, 0
        k, q = f(q + 1, self.kbits)
        if k == 0 or k > self.s:
            return 0, 0
        return q, g

    def step(self, p, lim):
        """One chain step from p below lim: (next position, positions visited)."""
        e = self.entry(p)
        if e is None:
            q, _ = self.slow(p)
            return (q if q else p + 1), [p]
        tot, l1 = e[0], e[1]
        if l1 < tot and p + l1 < lim:
            return p + tot, [p, p + l1]
        return p + l1, [p]


def model_bucket(b: Bucket):
    """Replays the parse of one bucket; returns counts of what it did."""
    nl, E = b.nl, b.E
    out = dict(lanes=nl, steps_a=[], steps_b=[], sync=[], restarts=0, rerestarts=0, rounds=0)
    if nl == 0:
        return out
    sq = [b.P0 + q * b.seg for q in range(nl)]
    sn = [E if q == nl - 1 else sq[q] + b.seg for q in range(nl)]
    marks, cx = [], []
    for q in range(nl):
        p, n = sq[q], 0
        if q and b.guess:
            for _ in range(GUESS_STEPS):
                e = b.entry(p)
                if p < sn[q]:
                    if e is None:
                        p += 1
                    else:
                        p += e[0] if (e[1] < e[0] and p + e[1] < sn[q]) else e[1]
        noted = set()
        for lim in (min(sn[q], sq[q] + 64), min(sn[q], sq[q] + SYNC_BITS)):
            while p < lim:
                p, vis = b.step(p, lim)
                noted.update(vis)
                n += 1
        while p < sn[q]:
            p, _ = b.step(p, sn[q])
            n += 1
        marks.append(noted)
        cx.append(p)
        out["steps_a"].append(n)

    def meet(q, x0):
        def stop(p):
            if p == E or p in marks[q + 1]:
                return True, True
            return p - sn[q] >= SYNC_BITS or p > E, False

        p, n = x0, 0
        while True:
            done, hit = stop(p)
            if done:
                return hit, p, n
            e = b.entry(p)
            n += 1
            if e is None:
                p, _ = b.slow(p)
                if p == 0:
                    return False, p, n
                continue
            # the second record too, unless its start already ends the walk
            p1 = p + e[1]
            p = p + e[0] if e[1] < e[0] and not stop(p1)[0] else p1

    found = [True] * nl
    for q in range(nl - 1):
        f, y, n = meet(q, cx[q])
        found[q] = f
        out["steps_b"].append(n)
        if f:
            out["sync"].append(y - sn[q])
    repaired, rstart = [False] * nl, [0] * nl
    while True:
        broken = [q >= 1 and not found[q - 1] for q in range(nl)]
        if not any(broken):
            break
        out["rounds"] += 1
        px = list(cx)
        for q in range(nl):
            if broken[q]:
                out["restarts"] += 1
                out["rerestarts"] += repaired[q]
                p = px[q - 1]
                while p < sn[q]:
                    p, _ = b.step(p, sn[q])
                cx[q] = p
                found[q] = True if q == nl - 1 else meet(q, p)[0]
                repaired[q], rstart[q] = True, px[q - 1]
        for q in range(nl - 1):
            if repaired[q + 1]:
                found[q] = cx[q] == rstart[q + 1]
    return out


def sync_distances(b: Bucket, guess: bool):
    """For each lane q >= 1: bits from its segment start to the first position
    its speculative chain (with or without the guess steps) shares with the true
    chain of the bucket, or None if they share none before the bucket's end."""
    true, p = set(), b.P0
    while p < b.E:
        p, vis = b.step(p, b.E)
        true.update(vis)
    out = []
    for q in range(1, b.nl):
        sq = b.P0 + q * b.seg
        p = sq
        if guess:
            for _ in range(GUESS_STEPS):
                e = b.entry(p)
                p += 1 if e is None else (e[0] if e[1] < e[0] and p + e[1] < b.E else e[1])
        met = None
        while p < b.E and met is None:
            p, vis = b.step(p, b.E)
            met = next((y for y in vis if y in true), None)
        out.append(met - sq if met is not None else None)
    return out
