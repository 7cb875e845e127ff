// Decoder: parses the Elias-omega (or Elias-gamma) stream and dequantizes.
//
// Page "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding",
// definition paragraph: the coding is lossless, so decode inverts it exactly;
// Q_s(v)_i = ||v|| sgn(v_i) k_i / s, the binary32 value nearest to the exact
// quotient (dequant_value).
//
// Work split. A wave64 owns a group of consecutive buckets and a team of T lanes
// (T = 1..64, chosen from the bucket size) decodes each bucket. The wave first
// copies the group's stream words into LDS with coalesced loads.
//
// Parallel parse of one bucket. Its records form a chain that can only be
// followed serially, so the team splits the payload into equal bit segments
// (each at least 128 bits) and lane q starts a chain at its segment start s_q,
// a guess at a record boundary (lane 0 starts at a true boundary). A chain that
// meets an invalid code restarts one bit later.
//   phase A: lane q follows its chain to the first position >= s_{q+1} and notes
//            the positions it visits in the first 128 bits of its segment.
//   phase B: lane q keeps following its chain until it lands on one of lane
//            q+1's noted positions. Two chains that meet coincide from then on,
//            and the chain that reached s_{q+1} from a true boundary is the true
//            chain, so that position is the first true boundary of lane q+1's
//            chain: lane q+1's records are exact from there.
//   repair:  if lane q's chain does not meet lane q+1's within 128 bits, lane q+1
//            restarts from lane q's exit; all such lanes restart together, and
//            again while a restarted predecessor exits elsewhere.
//   count:   each lane's index span is the sum of the gaps of its exact records
//            (phase A + B sums minus those before its sync point, from the gap
//            sums noted in phase A or parsed again); a team prefix sum gives
//            absolute indices.
//   write:   each lane parses its exact range again. For levels that fit a byte
//            and groups of at most 4096 coordinates, it stores (sign, k) bytes
//            in an LDS copy of the group, which the wave then dequantizes and
//            writes with coalesced 16-byte stores; otherwise each lane writes
//            its own index range directly.
// Record parsing looks the next 12 stream bits up in a table that decodes one or
// two whole records (gap <= 16, k <= 16) at once; other records take the
// general omega (or gamma) loop. A walk keeps a 64-bit window of the stream,
// read from LDS at its current position together with that position's table
// entry, which holds the next step's table bits. Groups whose stream passes the
// stage are staged over the stage and the level buffer together, or read from
// global memory.
#pragma once

#include "qsgd_device.h"

namespace qsgd {

constexpr int kLutBits = 12;
constexpr int kSyncWin = 128;       // bits
constexpr int kDecWaves = 8;        // waves per decode workgroup
constexpr int kDecWG = 64 * kDecWaves;
constexpr int kStageWords = 320;    // 64-bit stream words staged per wave
constexpr int kStagePad = 4;        // zero words after the staged stream
constexpr int kGroupCoords = 4096;  // coordinates of a group whose levels are staged in LDS
constexpr uint32_t kLevelSpare = kGroupCoords + 16;  // level byte for out-of-range writes
// Sparse streams: a unit of kSoloBuckets consecutive buckets whose stream fits
// the stage and whose payloads are at most kSoloMaxBits bits each is decoded by
// one wave, a lane per bucket (decode_kernel).
constexpr uint32_t kSoloBuckets = 64;
constexpr uint32_t kSoloMaxBits = 1024;
// Streams of more bits per bucket on average (a unit of them would not fit the
// stage) skip the per-group test for such units altogether.
constexpr uint32_t kSoloAvgBits = (uint32_t)kStageWords * 64u / kSoloBuckets;

// Streams that one decode-accumulate call sums.
constexpr uint32_t kMaxStreams = 32;

struct DecodeParams {
    // the streams to decode (one for a plain decode) and their bucket offsets
    const uint64_t *in[kMaxStreams];
    const uint64_t *offsets[kMaxStreams];
    uint32_t nstreams;
    const uint64_t *bstart;  // ragged table or nullptr
    float *v_hat;
    uint64_t n;
    uint64_t nb;
    uint32_t s;
    uint32_t d;
    uint32_t team;           // lanes per bucket (power of two, 1..64)
    uint32_t tpw;            // buckets per wave group (tpw * team <= 64)
    uint32_t lds_out;        // 1: levels staged in LDS (s <= 127, tpw * d <= kGroupCoords)
    uint32_t s_pow2;         // s is a power of two (norm / s exact)
    uint32_t solo;           // 1: units of sparse buckets are decoded a lane per bucket (decode_kernel)
    double inv_s;            // 1 / s (exact when s_pow2)
    SegTable seg;            // ragged layout by tensor lengths (nseg > 0) instead of bstart
};

// ---- record table -------------------------------------------------------
// Entry for the next 12 stream bits, indexed with the first of them in bit 0.
// It decodes the first record, and the second one if it also ends within the
// 12 bits, when each has gap and level at most 16:
//   bits  0-3   total length of the decoded records (0: take the general path)
//   bits  4-7   length of the first record (== total: one record)
//   bits  8-11  gap - 1 of the first record
//   bits 12-19  level byte sign << 7 | k of the first record
//   bits 20-23  gap - 1 of the second record
//   bits 24-31  level byte of the second record
// With total length 0, the first field alone (any value) if it ends within the
// 12 bits: bits 4-7 its length, bits 8-15 its value; else, for an omega field
// that starts with whole groups within the 12 bits, bits 16-19 the bits those
// groups take and bits 20-31 the value they leave (the next group's length - 1);
// else 0. The general path decodes from it. Computed at compile time.
struct alignas(16) RecordLut {
    uint32_t e[1 << kLutBits];
};

struct LutCursor {
    uint32_t bits;
    int pos;
};

constexpr int lut_take(LutCursor &c, int nbits) {
    if (c.pos + nbits > kLutBits) return -1;
    const int v = (int)((c.bits >> (kLutBits - c.pos - nbits)) & ((1u << nbits) - 1u));
    c.pos += nbits;
    return v;
}

// Elias omega (Elias 1975) for values up to 16: N = 1; while the next bit is 1,
// that bit and the N bits after it are the new N; a 0 bit ends the codeword.
constexpr int lut_omega(LutCursor &c) {
    int N = 1;
    while (true) {
        const int b = lut_take(c, 1);
        if (b < 0) return -1;
        if (b == 0) return N;
        const int v = lut_take(c, N);
        if (v < 0) return -1;
        N = (1 << N) | v;
        if (N > 16) return -1;
    }
}

// Elias gamma (Elias 1975) for values up to 16: z zero bits, then the z + 1 bits
// of N from its leading 1.
constexpr int lut_gamma(LutCursor &c) {
    int z = 0;
    while (true) {
        const int b = lut_take(c, 1);
        if (b < 0) return -1;
        if (b == 1) break;
        if (++z > 4) return -1;
    }
    int N = 1;
    for (int i = 0; i < z; ++i) {
        const int b = lut_take(c, 1);
        if (b < 0) return -1;
        N = (N << 1) | b;
    }
    return N > 16 ? -1 : N;
}

// A record field (gap or level) in the code of the stream: omega or gamma.
template <int CODE>
constexpr int lut_field(LutCursor &c) {
    return CODE ? lut_gamma(c) : lut_omega(c);
}

// One record at the cursor: (gap - 1) | level byte << 4, or -1.
template <int CODE>
constexpr int lut_record(LutCursor &c) {
    const int gap = lut_field<CODE>(c);
    if (gap <= 0) return -1;
    const int sg = lut_take(c, 1);
    if (sg < 0) return -1;
    const int k = lut_field<CODE>(c);
    if (k <= 0) return -1;
    return (gap - 1) | (((sg << 7) | k) << 4);
}

constexpr uint32_t reverse_bits(uint32_t v, int n) {
    uint32_t r = 0;
    for (int b = 0; b < n; ++b) r |= ((v >> b) & 1u) << (n - 1 - b);
    return r;
}

// One field (omega or gamma, any value) at the cursor, or -1 if it does not
// end within the window; a codeword of at most kLutBits bits holds N <= 63.
template <int CODE>
constexpr int lut_field_any(LutCursor &c) {
    if (CODE) {
        int z = 0;
        while (true) {
            const int b = lut_take(c, 1);
            if (b < 0) return -1;
            if (b == 1) break;
            ++z;
        }
        int N = 1;
        for (int i = 0; i < z; ++i) {
            const int b = lut_take(c, 1);
            if (b < 0) return -1;
            N = (N << 1) | b;
        }
        return N;
    }
    int N = 1;
    while (true) {
        const int b = lut_take(c, 1);
        if (b < 0) return -1;
        if (b == 0) return N;
        const int v = lut_take(c, N);
        if (v < 0) return -1;
        N = (1 << N) | v;
    }
}

// Entry of window i: one or two records (total length in bits 0-3, see above);
// where no record ends within the window, total length 0 and, if the first
// field does, N << 8 | its length << 4 (0 if not).
template <int CODE>
constexpr RecordLut make_record_lut() {
    RecordLut t{};
    for (uint32_t i = 0; i < (1u << kLutBits); ++i) {
        LutCursor c{reverse_bits(i, kLutBits), 0};  // the cursor reads the first bit from the top
        uint32_t e = 0;
        const int r1 = lut_record<CODE>(c);
        if (r1 >= 0) {
            const uint32_t l1 = (uint32_t)c.pos;
            e = l1 | (l1 << 4) | ((uint32_t)r1 << 8);
            LutCursor c2 = c;
            const int r2 = lut_record<CODE>(c2);
            if (r2 >= 0) e = (e & ~15u) | (uint32_t)c2.pos | ((uint32_t)r2 << 20);
        } else {
            LutCursor cf{reverse_bits(i, kLutBits), 0};
            const int N = lut_field_any<CODE>(cf);
            if (N > 0) {
                e = ((uint32_t)N << 8) | ((uint32_t)cf.pos << 4);
            } else if (!CODE) {
                // an omega field longer than the window: its whole groups within it
                LutCursor cp{reverse_bits(i, kLutBits), 0};
                int Np = 1, m = 0;
                while (lut_take(cp, 1) == 1) {
                    const int v = lut_take(cp, Np);
                    if (v < 0) break;
                    Np = (1 << Np) | v;
                    m = cp.pos;
                }
                if (m > 0) e = ((uint32_t)Np << 20) | ((uint32_t)m << 16);
            }
        }
        t.e[i] = e;
    }
    return t;
}

// record tables of the omega (code 0) and gamma (code 1) streams
__constant__ RecordLut kRecordLut = make_record_lut<0>();
__constant__ RecordLut kRecordLutGamma = make_record_lut<1>();


// ---- bit access -----------------------------------------------------------
// Bit positions fit 32 bits (a group spans fewer than 2^31 bits: buckets of at
// most 2^24 coordinates). LDS mode: a position is an LDS bit address; the
// wave's staged copy of the group's stream words sits bit-reversed, so that
// the dword at byte address 4h holds stream bits [32h, 32h + 32) with the first
// in bit 0, and kStagePad zero words follow it, so no bound check is needed.
// Global mode: positions count from the group's first stream word (bits
// [32h, 32h + 32) are dword h ^ 1, first bit on top); dwords past `hlast` read
// as zero.
typedef __attribute__((address_space(3))) const uint32_t lds_cu32;

// LDS byte address of a pointer into LDS.
__device__ __forceinline__ uint32_t lds_address(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

template <bool LDS>
struct Bits {
    const uint32_t *src;
    uint32_t hlast;

    // Stream bits [32h, 32h + 64), bit 32h in bit 0.
    __device__ __forceinline__ uint64_t pair(uint32_t h) const {
        if (LDS) {
            const lds_cu32 *lds = (const lds_cu32 *)(uintptr_t)0;
            return ((uint64_t)lds[h + 1u] << 32) | (uint64_t)lds[h];
        }
        const uint32_t a = h <= hlast ? src[h ^ 1u] : 0u;
        const uint32_t b = h + 1u <= hlast ? src[(h + 1u) ^ 1u] : 0u;
        return ((uint64_t)__builtin_bitreverse32(b) << 32) | (uint64_t)__builtin_bitreverse32(a);
    }

    // The 64 stream bits from bit p on, stream bit p in bit 0; at least the
    // first 33 of them lie within the two dwords read (zeros above).
    __device__ __forceinline__ uint64_t at(uint32_t p) const { return pair(p >> 5) >> (p & 31u); }
};

// Read-ahead window of a chain walk: stream bits [32h, 32h + 64). A walk reads
// the window of its current position together with that position's table
// entry; the next position is at most 12 bits on (one table step), so its 12
// table bits lie in that window (p - 32h <= 43). The walk thus waits for one
// LDS read per step instead of two dependent ones. After a general-path record
// the window is read again at the new position.
struct Win {
    uint64_t w;
    uint32_t h;
};

template <bool LDS>
__device__ __forceinline__ Win win_at(const Bits<LDS> &r, uint32_t p) {
    return Win{r.pair(p >> 5), p >> 5};
}

__device__ __forceinline__ uint32_t win_index(const Win &W, uint32_t p) {
    return (uint32_t)(W.w >> (p - (W.h << 5))) & ((1u << kLutBits) - 1u);
}

// CODE: integer code of the record fields, 0 Elias omega, 1 Elias gamma.
template <int CODE>
struct RecordCtx {
    static constexpr int code = CODE;
    const uint32_t *lut;
    uint32_t gbits, kbits, s;
};

__device__ __forceinline__ uint32_t bitlen32(uint32_t x) { return 32u - (uint32_t)__clz(x); }

// General omega decoding from bit p: returns N and advances p, or 0 if a group
// is longer than maxbits (<= 25, so each group lies in one 64-bit read). N: the
// value left by the groups before p (1 at a codeword's start).
// One read serves the groups and the final bit that lie within its first 33
// bits; the stream is read again only where a group passes them.
template <bool LDS>
__device__ __forceinline__ uint32_t omega_at(const Bits<LDS> &r, uint32_t &p, uint32_t maxbits,
                                             uint32_t N = 1u) {
    uint64_t w = r.at(p);
    uint32_t have = 33u;  // bits of w that are stream bits from p on
    while (true) {
        if ((w & 1u) == 0) {
            p += 1u;
            return N;
        }
        const uint32_t g = N + 1u;
        if (g > maxbits) return 0;
        if (g >= have) {
            w = r.at(p);
            have = 33u;
        }
        N = __builtin_bitreverse32((uint32_t)w) >> (32u - g);
        p += g;
        w >>= g;
        have -= g;
    }
}

// General Elias gamma decoding from bit p: returns N and advances p, or 0 if N
// has more than maxbits (<= 25) binary digits.
template <bool LDS>
__device__ __forceinline__ uint32_t gamma_at(const Bits<LDS> &r, uint32_t &p, uint32_t maxbits) {
    const uint32_t w = (uint32_t)r.at(p);
    const uint32_t z = w ? (uint32_t)__builtin_ctz(w) : 32u;  // zero bits before the leading 1
    if (z + 1u > maxbits) return 0;
    const uint32_t v = (uint32_t)r.at(p + z);
    p += 2u * z + 1u;
    return __builtin_bitreverse32(v) >> (31u - z);
}

// One record c(gap) | sign | c(k) at bit p by general decoding of the code c.
// Returns the position after it, or 0 if it does not parse (a record never
// ends at 0): a group longer than the bound, or k > s.
// The first field of the window a table entry was made from: its value N and
// length, or false if it does not end within the window. A record entry's first
// field is its gap (N <= 16); an entry without a record keeps the field itself.
template <int CODE>
__device__ __forceinline__ bool entry_field(uint32_t e, uint32_t &N, uint32_t &len) {
    if (e & 15u) {
        N = ((e >> 8) & 15u) + 1u;
        const uint32_t b = 32u - (uint32_t)__clz(N);
        len = CODE ? 2u * b - 1u : (N == 1u ? 1u : (N < 4u ? 3u : (N < 8u ? 6u : (N < 16u ? 7u : 11u))));
        return true;
    }
    N = e >> 8;
    len = (e >> 4) & 15u;
    return len != 0u;
}

// e0: the table entry at p (one without a record).
template <bool LDS, class X>
__device__ __forceinline__ uint32_t record_slow(const Bits<LDS> &r, const X &x, uint32_t p,
                                                uint32_t &gap, uint32_t &neg, uint32_t &k,
                                                uint32_t e0) {
    // both fields of at most kLutBits bits: the first from e0, the table entry at
    // p, the second from the entry at its start (one read of the stream, 33 bits
    // or more from p, and one of the table). The bounds below are those of the
    // general decoding: every group of a codeword is at most as long as the
    // binary form of its value.
    {
        uint32_t v1, l1, v2, l2;
        if (entry_field<X::code>(e0, v1, l1)) {
            const uint64_t w = r.at(p);
            const uint32_t e2 = x.lut[(uint32_t)(w >> (l1 + 1u)) & ((1u << kLutBits) - 1u)];
            if (entry_field<X::code>(e2, v2, l2) && 32u - (uint32_t)__clz(v1) <= x.gbits &&
                32u - (uint32_t)__clz(v2) <= x.kbits && v2 <= x.s) {
                gap = v1;
                neg = (uint32_t)(w >> l1) & 1u;
                k = v2;
                return p + l1 + 1u + l2;
            }
        }
    }
    uint32_t q = p;
    if (X::code) {
        gap = gamma_at(r, q, x.gbits);
    } else {
        // an omega gap field longer than the window goes on from the groups e0
        // holds; their longest group is the last, as long as the value they leave
        const uint32_t m = (e0 >> 16) & 15u, N0 = e0 >> 20;
        if (m == 0u) {
            gap = omega_at(r, q, x.gbits);
        } else if (bitlen32(N0) <= x.gbits) {
            q += m;
            gap = omega_at(r, q, x.gbits, N0);
        } else {
            gap = 0;
        }
    }
    if (gap == 0) return 0;
    neg = (uint32_t)r.at(q) & 1u;
    q += 1u;
    k = X::code ? gamma_at(r, q, x.kbits) : omega_at(r, q, x.kbits);
    if (k == 0 || k > x.s) return 0;
    return q;
}

// Table entry of the 12 stream bits at p (length 0: take record_slow). The
// table covers records of at most 12 bits with gap, k <= 16; it does not check
// k <= s or gap <= bucket length: on the true chain those hold anyway, and a
// speculative chain only has to be a deterministic function of its start. A
// two-record entry is the same as two one-record steps, so every walker of a
// chain visits the same positions. The entry is looked up in the window W (read
// at a position at most 12 bits before p, or at p); W moves on to p's own
// window for the next step.
template <bool LDS, class X>
__device__ __forceinline__ uint32_t lut_step(const Bits<LDS> &r, const X &x, uint32_t p, Win &W) {
    const uint32_t e = x.lut[win_index(W, p)];
    W = win_at(r, p);
    return e;
}

// The general path of a chain step at p (e: the table entry there): past the
// record at p adding its gap to sum, or one bit on if no record parses there;
// W follows p.
template <bool LDS, class X>
__device__ __forceinline__ void slow_step(const Bits<LDS> &r, const X &x, uint32_t &p, uint32_t &sum,
                                          Win &W, uint32_t e) {
    uint32_t gap, neg, k;
    const uint32_t q = record_slow(r, x, p, gap, neg, k, e);
    sum += q ? gap : 0u;
    p = q ? q : p + 1u;
    W = win_at(r, p);
}

// One step of a chain: past the record at p adding its gap to sum, or one bit
// on if no record parses there.
template <bool LDS, class X>
__device__ __forceinline__ void chain_step(const Bits<LDS> &r, const X &x, uint32_t &p,
                                           uint32_t &sum, Win &W) {
    const uint32_t e = lut_step(r, x, p, W);
    if (e & 15u) {
        p += (e >> 4) & 15u;
        sum += ((e >> 8) & 15u) + 1u;
    } else {
        slow_step(r, x, p, sum, W, e);
    }
}

// One record of the true chain at p: its end (0 if it does not parse), gap and
// level byte sign << 7 | k (k <= 127 when the caller uses the byte).
// W is the walk's read-ahead window (lut_step).
template <bool LDS, class X>
__device__ __forceinline__ uint32_t record_at(const Bits<LDS> &r, const X &x, uint32_t p,
                                              uint32_t &gap, uint32_t &neg, uint32_t &k, Win &W) {
    const uint32_t e = lut_step(r, x, p, W);
    if (e & 15u) {
        gap = ((e >> 8) & 15u) + 1u;
        k = (e >> 12) & 127u;
        neg = (e >> 19) & 1u;
        return p + ((e >> 4) & 15u);
    }
    const uint32_t q = record_slow(r, x, p, gap, neg, k, e);
    if (q) W = win_at(r, q);
    return q;
}


// Slots of a lane's gap-prefix table (bytes, in the wave's level buffer while
// the chains are being synchronised); positions past the table are not looked up.
// An odd count keeps the lanes' tables in different LDS banks.
constexpr uint32_t kCumSlots = 63;

// Steps at the start of a guessed chain that skip a bit at a table miss.
#ifndef QSGD_GUESS_STEPS
#define QSGD_GUESS_STEPS 6
#endif
constexpr int kGuessSteps = QSGD_GUESS_STEPS;
// Buckets whose payload averages more bits per coordinate than kGuessBits, or
// fewer than kGuessMinBits, take no guess steps: their long records (large
// levels, or long gaps between sparse non-zeros) miss the table on the true
// chain too, where moving one bit on derails the chain.
constexpr uint32_t kGuessBits = 4;
constexpr uint32_t kGuessMinBits = 1;

// Whether a bucket of len coordinates and payload bits takes guess steps.
__device__ __forceinline__ bool guess_bucket(uint64_t bits, uint64_t len) {
    return bits <= (uint64_t)kGuessBits * len && bits >= (uint64_t)kGuessMinBits * len;
}

// The first steps of a chain whose start is only a guess at a record boundary.
// Such a start lands on bits that are not a record start as often as not, and
// those often miss the table; so for kGuessSteps steps a table miss moves one
// bit on instead of decoding a long record. follow_chain notes no position
// during these steps, so another chain can only meet this one where it follows
// the exact rule, and both continue alike from there.
template <bool LDS, class X>
__device__ __forceinline__ void guess_steps(const Bits<LDS> &r, const X &x, uint32_t &p,
                                            uint32_t sn, uint32_t &sum, Win &W) {
#pragma unroll
    for (int i = 0; i < kGuessSteps; ++i) {
        const uint32_t e = lut_step(r, x, p, W);
        const uint32_t len1 = (e >> 4) & 15u;
        const bool two = len1 < (e & 15u) && p + len1 < sn;
        const uint32_t adv = (e & 15u) == 0 ? 1u : two ? (e & 15u) : len1;
        const uint32_t g =
            (e & 15u) == 0 ? 0u : ((e >> 8) & 15u) + 1u + (two ? ((e >> 20) & 15u) + 1u : 0u);
        const bool go = p < sn;
        sum += go ? g : 0u;
        p += go ? adv : 0u;
    }
}

// Phase A: follows a chain from `start` to its first position >= sn and returns
// that position (the exit), with the gap sum of the records passed. MARK: sets
// bit (p - start) of own0:own1 for each chain position p in [start, start + 128)
// and, with CUM, stores in cum[i] the low byte of the gap sum before the i-th of
// them (i < kCumSlots - 1; cum_top: the gap sum after the last noted position, so
// a table entry is exact when cum_top < 256). Two-record table entries advance
// two records at once when the second starts before the current limit (the
// end of the 64-bit mark word being filled, or sn).
template <bool LDS, bool MARK, bool CUM, class X>
__device__ __forceinline__ uint32_t follow_chain(const Bits<LDS> &r, const X &x, uint32_t start,
                                                 uint32_t sn, uint32_t &ga, uint64_t &own0,
                                                 uint64_t &own1, uint8_t *cum, uint32_t &cum_top,
                                                 bool guess = false) {
    uint32_t p = start, sum = 0;
    Win W = win_at(r, p);
    if (MARK && guess) guess_steps(r, x, p, sn, sum, W);
    if (MARK) {
        uint32_t i = 0;
        // one step from p below lim: returns the step's chain positions
        // relative to p (bit 0, and bit len1 for a second record)
        auto step = [&](uint32_t lim) -> uint32_t {
            const uint32_t e = lut_step(r, x, p, W);
            if (CUM) cum[i] = (uint8_t)sum;
            uint32_t m = 1u;
            if (e & 15u) {
                const uint32_t len1 = (e >> 4) & 15u;
                const uint32_t s1 = sum + ((e >> 8) & 15u) + 1u;
                const bool two = len1 < (e & 15u) && p + len1 < lim;
                if (CUM) cum[i + 1u] = (uint8_t)s1;
                m = ((uint32_t)two << len1) | 1u;
                sum = two ? s1 + ((e >> 20) & 15u) + 1u : s1;
                p += two ? (e & 15u) : len1;
                i += two ? 2u : 1u;
            } else {
                slow_step(r, x, p, sum, W, e);
                i += 1u;
            }
            i = i < kCumSlots - 2u ? i : kCumSlots - 2u;
            return m;
        };
        const uint32_t l1 = sn < start + 64u ? sn : start + 64u;
        while (p < l1) {
            const uint32_t rel = p - start;
            own0 |= (uint64_t)step(l1) << rel;
        }
        const uint32_t l2 = sn < start + 128u ? sn : start + 128u;
        while (p < l2) {
            const uint32_t rel = p - start - 64u;
            own1 |= (uint64_t)step(l2) << rel;
        }
        cum_top = sum;
    }
    while (p < sn) {
        const uint32_t e = lut_step(r, x, p, W);
        if (e & 15u) {
            const uint32_t len1 = (e >> 4) & 15u;
            const bool two = len1 < (e & 15u) && p + len1 < sn;
            sum += ((e >> 8) & 15u) + 1u + (two ? ((e >> 20) & 15u) + 1u : 0u);
            p += two ? (e & 15u) : len1;
        } else {
            slow_step(r, x, p, sum, W, e);
        }
    }
    ga = sum;
    return p;
}

// Gap sum of a lane's speculative chain before its position y, from the table
// follow_chain<MARK> filled; false if the table cannot tell (y not a noted
// position, past the table, or sums past a byte).
__device__ __forceinline__ bool cum_lookup(const uint8_t *cum, uint32_t cum_top, uint64_t own0,
                                           uint64_t own1, uint32_t rel, uint32_t &g) {
    if (rel >= 128u || cum_top > 255u) return false;
    const uint64_t m = rel < 64u ? own0 : own1;
    if (((m >> (rel & 63u)) & 1u) == 0) return false;
    const uint32_t i = rel < 64u
                           ? (uint32_t)__popcll(own0 & ((1ull << rel) - 1ull))
                           : (uint32_t)__popcll(own0) +
                                 (uint32_t)__popcll(own1 & ((1ull << (rel - 64u)) - 1ull));
    if (i >= kCumSlots - 2u) return false;
    g = cum[i];
    return true;
}

// Phase B: continues the chain from its exit x0 (>= sn) until it lands on a
// position noted by the next lane (nxt0:nxt1, relative to sn) or on E. Gives up
// 128 bits past sn, past E, or at a record that does not parse.
__device__ __forceinline__ bool meet_stop(uint32_t p, uint32_t sn, uint32_t E, uint64_t nxt0,
                                          uint64_t nxt1, bool &found) {
    if (p == E) { found = true; return true; }
    const uint32_t rel = p - sn;
    if (rel >= (uint32_t)kSyncWin || p > E) return true;
    const uint64_t m = rel < 64u ? nxt0 : nxt1;
    if ((m >> (rel & 63u)) & 1u) { found = true; return true; }
    return false;
}

template <bool LDS, class X>
__device__ __forceinline__ bool extend_chain(const Bits<LDS> &r, const X &x, uint32_t x0,
                                             uint32_t sn, uint32_t E, uint64_t nxt0, uint64_t nxt1,
                                             uint32_t &y, uint32_t &gb) {
    uint32_t p = x0, sum = 0;
    bool found = false;
    Win W = win_at(r, p);
    while (!meet_stop(p, sn, E, nxt0, nxt1, found)) {
        const uint32_t e = lut_step(r, x, p, W);
        if (e & 15u) {
            const uint32_t p1 = p + ((e >> 4) & 15u);
            sum += ((e >> 8) & 15u) + 1u;
            p = p1;
            // take the second record too unless its start already ends the walk
            bool f1 = false;
            if ((e & 15u) > ((e >> 4) & 15u) && !meet_stop(p1, sn, E, nxt0, nxt1, f1)) {
                sum += ((e >> 20) & 15u) + 1u;
                p = p1 + ((e & 15u) - ((e >> 4) & 15u));
            }
        } else {
            uint32_t gap, neg, k;
            const uint32_t q = record_slow(r, x, p, gap, neg, k, e);
            if (!q) break;
            p = q;
            sum += gap;
            W = win_at(r, p);
        }
    }
    y = found ? p : E;
    gb = sum;
    return found;
}

// Writes one lane's output range [lo, hi) in index order, exactly once: values
// and the zeros between them, 16-byte stores for whole aligned quads inside the
// range, single floats for the partial quads at its ends. ACC: adds them to the
// output instead (the zeros too: -0.0f + +0.0f is +0.0f).
template <bool ACC>
struct QuadWriter {
    float *out;
    uint64_t lo, hi, q;
    float v0, v1, v2, v3;

    __device__ __forceinline__ void init(float *o, uint64_t l, uint64_t h) {
        out = o; lo = l; hi = h; q = l >> 2;
        v0 = v1 = v2 = v3 = 0.0f;
    }
    __device__ __forceinline__ static void put1(float *p, float v) { *p = ACC ? *p + v : v; }
    __device__ __forceinline__ static void put4(float *p, float4 v) {
        float4 *p4 = reinterpret_cast<float4 *>(p);
        if (ACC) {
            const float4 o = *p4;
            v = make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w);
        }
        *p4 = v;
    }
    // The elements of the quad v at out[a, a + 4) that lie in [l, h), one by one
    // (a quad cut by a range end). The empty asm keeps the compiler from merging
    // the last of these stores with the 16-byte store of a whole quad in the
    // caller's other branch, which it would then split into 12- and 4-byte stores.
    __device__ __forceinline__ static void put_part(float *out, uint64_t a, uint64_t l, uint64_t h, float4 v) {
        if (a >= l && a < h) put1(out + a, v.x);
        if (a + 1 >= l && a + 1 < h) put1(out + a + 1, v.y);
        if (a + 2 >= l && a + 2 < h) put1(out + a + 2, v.z);
        if (a + 3 >= l && a + 3 < h) put1(out + a + 3, v.w);
        asm volatile("" ::: "memory");
    }
    __device__ __forceinline__ void flush() const {
        const uint64_t a = q << 2;
        if (a >= lo && a + 4 <= hi)
            put4(out + a, make_float4(v0, v1, v2, v3));
        else
            put_part(out, a, lo, hi, make_float4(v0, v1, v2, v3));
    }
    // moves to quad nq > q: writes the current quad and the all-zero quads between
    __device__ __forceinline__ void advance(uint64_t nq) {
        flush();
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
        for (uint64_t t = q + 1; t < nq; ++t) put4(out + (t << 2), z);
        q = nq;
        v0 = v1 = v2 = v3 = 0.0f;
    }
    __device__ __forceinline__ void put(uint64_t g, float val) {
        const uint64_t nq = g >> 2;
        if (nq != q) advance(nq);
        const uint32_t c = (uint32_t)(g & 3u);
        v0 = c == 0 ? val : v0;
        v1 = c == 1 ? val : v1;
        v2 = c == 2 ? val : v2;
        v3 = c == 3 ? val : v3;
    }
    __device__ __forceinline__ void finish() {
        const uint64_t nq = hi >> 2;
        if (nq != q) advance(nq);
        if (hi & 3u) flush();
    }
};

template <bool RAGGED>
__device__ __forceinline__ uint64_t bucket_first(const DecodeParams &D, uint64_t b) {
    if (RAGGED) return ragged_start(D.bstart, D.seg, b);
    const uint64_t g = b * D.d;
    return g < D.n ? g : D.n;
}

// Orders the wave's LDS accesses before this point before those after it, for
// data that other lanes of the same wave read or overwrite.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


// Decodes the buckets [b0, b1) of one wave group of a stream with bucket
// offsets `offs`; `r` reads the group's stream, bit 0 being stream bit `gbit`.
// LDS_OUT: each record's level byte (sign << 7 | k) goes to the group's LDS
// buffer `lvl` (index = coordinate - lbase, cleared here) and each bucket's
// norm to ebs[team]; otherwise every lane writes (ACC: adds) its own
// output range with a QuadWriter. CUM: the lanes' gap-prefix tables live in
// `lvl` (without them, the gap sum before a sync point is found by walking the
// speculative chain again).
// A piece of one bucket decoded outside the bucket tables (buckets longer
// than a chunk): its payload [P0, E) in the reader's positions, the first
// output coordinate c0 and the output length len (MODE 2), the bucket's length
// blen (the bound of its gaps), its norm, whether guessed starts take guess
// steps, and whether lane 0's start is itself a guess (MODE 1, chunks after the
// first).
struct GroupView {
    uint32_t P0, E;
    uint64_t c0, len, blen;
    double norm;
    bool guess, lane0_guess;
};

// MODE 1 result: the gap sum from P0 along the chunk's chain to its exit X
// (the first chain position at or past E).
struct ChunkOut {
    uint32_t T, X;
};

// MODE 0: the buckets [b0, b1) of a wave group. MODE 1: parse a chunk of a long
// bucket with one team (no output; lane 0 may start on a guess). MODE 2: decode
// a piece [P0, E) of a long bucket that starts on an exact record boundary,
// with one team, into [c0, c0 + len) (lane writers). MODE 3: as MODE 2 into an
// output already zeroed, writing only the records' values.
template <bool RAGGED, bool LDS_IN, bool LDS_OUT, bool ACC, int CODE, bool CUM, int MODE = 0>
__device__ __forceinline__ void decode_group(const DecodeParams &D, const uint64_t *offs,
                                             const uint32_t *lut,
                                             const Bits<LDS_IN> &r, uint64_t gbit, uint64_t b0,
                                             uint64_t b1, uint8_t *lvl, double *ebs, uint64_t lbase,
                                             uint32_t nclear16, const GroupView *gv = nullptr,
                                             ChunkOut *co = nullptr) {
    const int lane = lane_id();
    const uint32_t T = D.team;
    const uint32_t q = (uint32_t)lane % T;
    const uint32_t team = (uint32_t)lane / T;

    const uint64_t b = b0 + team;
    const bool tactive = MODE ? team == 0 : (team < D.tpw && b < b1);
    uint32_t A = 0, E = 0;
    uint64_t c0 = 0, len = 0;
    double e_b = 0.0;
    uint32_t nl = 0;
    bool guess = false;
    if (MODE && tactive) {
        A = gv->P0 - 32u;
        E = gv->E;
        c0 = gv->c0;
        len = gv->len;
        e_b = gv->norm;
        if (E > gv->P0) {
            const uint32_t m = (E - gv->P0) / (uint32_t)kSyncWin;
            nl = m < T ? m : T;
            if (nl == 0) nl = 1;
        }
        guess = gv->guess;
    } else if (tactive) {
        A = (uint32_t)(offs[b] - gbit);
        E = (uint32_t)(offs[b + 1] - gbit);
        c0 = bucket_first<RAGGED>(D, b);
        len = bucket_first<RAGGED>(D, b + 1) - c0;
        if (E >= A + 32u && len > 0) {
            const float norm = __uint_as_float(__builtin_bitreverse32((uint32_t)r.at(A)));
            e_b = (double)norm;
            const uint32_t Lp = E - (A + 32u);
            if (Lp > 0) {
                const uint32_t m = Lp / (uint32_t)kSyncWin;
                nl = m < T ? m : T;
                if (nl == 0) nl = 1;
            }
            // guess steps pay where table misses are rare on the true chain:
            // short records, kGuessMinBits to kGuessBits payload bits per coordinate
            guess = guess_bucket(Lp, len);
        }
    }
    if (LDS_OUT && tactive && q == 0) ebs[team] = e_b;
    const RecordCtx<CODE> x{lut, tactive ? bitlen32((uint32_t)(MODE ? gv->blen : len)) : 1u, bitlen32(D.s), D.s};
    const uint32_t P0 = A + 32u;
    const uint32_t seg = nl ? ((E - P0) + nl - 1u) / nl : 0u;
    const bool act = q < nl;
    const bool last = q + 1u >= nl;
    const uint32_t sq = act ? P0 + q * seg : E;
    const uint32_t sn = act ? (last ? E : sq + seg) : E;

    // phase A on every lane's own segment, noting its first 128 bits
    uint64_t own0 = 0, own1 = 0;
    uint32_t cx = E, ga = 0, gb = 0, ynext = E;
    bool found = false;
    uint8_t *cum = lvl + (uint32_t)lane * kCumSlots;
    uint32_t cum_top = 0;
    const bool lguess = guess && (q != 0 || (MODE == 1 && gv->lane0_guess));
    if (act) cx = follow_chain<LDS_IN, true, CUM>(r, x, sq, sn, ga, own0, own1, cum, cum_top, lguess);
    if (act && last) found = true;
    // phase B against the next lane's window
    const uint64_t nxt0 = lane_next64(own0, T);
    const uint64_t nxt1 = lane_next64(own1, T);
    if (act && !last) found = extend_chain(r, x, cx, sn, E, nxt0, nxt1, ynext, gb);

    // repair: every lane whose predecessor's chain does not reach its start
    // (did not meet it) restarts from the predecessor's exit, all such lanes in
    // the same round. A restarted lane's start is consistent with its
    // predecessor only while it equals the predecessor's exit; a predecessor
    // that itself restarts in the same round and exits elsewhere breaks it
    // again. In each round the lowest broken lane of a team restarts from an
    // exact predecessor that no longer changes, so the lowest broken lane only
    // moves up and the loop ends after at most T rounds; then every lane's start
    // lies on its predecessor's chain, so all chains are exact from lane 0 on.
    bool repaired = false;
    uint32_t rstart = 0;
    while (true) {
        const bool pf = lane_prev(found ? 1u : 0u, T) != 0u;
        const uint32_t px = lane_prev(cx, T);
        const bool broken = act && q >= 1 && !pf;
        if (__ballot(broken) == 0) break;
        if (broken) {
            uint64_t d0 = 0, d1 = 0;
            uint32_t dtop = 0;
            cx = follow_chain<LDS_IN, false, false>(r, x, px, sn, ga, d0, d1, nullptr, dtop);
            if (last) {
                found = true;
                ynext = E;
                gb = 0;
            } else {
                found = extend_chain(r, x, cx, sn, E, nxt0, nxt1, ynext, gb);
            }
            repaired = true;
            rstart = px;
        }
        // a restarted successor's records begin at its restart point: this
        // lane's records end at its exit, which must be that point
        const bool srep = lane_next(repaired ? 1u : 0u, T) != 0u && !last;
        const uint32_t srs = lane_next(rstart, T);
        if (act && srep) {
            found = cx == srs;
            ynext = cx;
            gb = 0;
        }
    }

    // exact start of each lane's records
    const uint32_t py = lane_prev(ynext, T);
    uint32_t ystart = E;
    if (act) {
        if (q == 0) ystart = P0;
        else if (repaired) ystart = rstart;
        else ystart = py;
    }
    // gaps of the records before the sync point: from the phase A table, else
    // by following the same speculative chain again
    uint32_t gpre = 0;
    if (act && q >= 1 && !repaired && !(CUM && cum_lookup(cum, cum_top, own0, own1, ystart - sq, gpre))) {
        gpre = 0;
        uint32_t p = sq;
        Win W = win_at(r, p);
        if (guess) guess_steps(r, x, p, sn, gpre, W);
        while (p < ystart) chain_step(r, x, p, gpre, W);
    }
    const uint32_t G = act ? ga + gb - gpre : 0u;
    // team-exclusive prefix sum of the index spans
    uint32_t incl = G;
    if (T == 64u) {
        incl = wave_incl_add_u32(G);
    } else {
        for (uint32_t off = 1; off < T; off <<= 1) {
            const uint32_t y = __shfl_up(incl, off, (int)T);
            if (q >= off) incl += y;
        }
    }
    const uint32_t basej = incl - G;

    if (MODE == 1) {
        // the team's total and the last lane's exit
        const uint32_t src = (uint32_t)__builtin_amdgcn_readfirstlane((int)(nl ? nl - 1u : 0u));
        co->T = nl ? (uint32_t)__builtin_amdgcn_readlane((int)incl, (int)src) : 0u;
        co->X = nl ? (uint32_t)__builtin_amdgcn_readlane((int)cx, (int)src) : P0;
        return;
    }

    if (LDS_OUT) {
        // the gap-prefix tables are done with: clear the group's level bytes
        wave_sync();
        uint4 *l4 = reinterpret_cast<uint4 *>(lvl);
        for (uint32_t i = (uint32_t)lane; i < nclear16; i += 64) l4[i] = make_uint4(0u, 0u, 0u, 0u);
        wave_sync();
        if (act) {
            // tix: the record's index in the group's level bytes; indices past the
            // bucket (only in a malformed stream) go to a spare byte
            uint32_t tix = (uint32_t)(c0 - lbase) + basej - 1u;
            const uint32_t tend = (uint32_t)(c0 - lbase) + (uint32_t)len;
            uint32_t p = ystart;
            Win W = win_at(r, p);
            while (p < ynext) {
                const uint32_t e = lut_step(r, x, p, W);
                if (e & 15u) {
                    const uint32_t len1 = (e >> 4) & 15u;
                    tix += ((e >> 8) & 15u) + 1u;
                    lvl[tix < tend ? tix : kLevelSpare] = (uint8_t)(e >> 12);
                    const bool two = len1 < (e & 15u) && p + len1 < ynext;
                    const uint32_t t2 = tix + ((e >> 20) & 15u) + 1u;
                    lvl[two && t2 < tend ? t2 : kLevelSpare] = (uint8_t)(e >> 24);
                    tix = two ? t2 : tix;
                    p += two ? (e & 15u) : len1;
                } else {
                    uint32_t gap, neg, k;
                    const uint32_t nq = record_slow(r, x, p, gap, neg, k, e);
                    if (!nq) break;
                    tix += gap;
                    lvl[tix < tend ? tix : kLevelSpare] = (uint8_t)((neg << 7) | k);
                    p = nq;
                    W = win_at(r, p);
                }
            }
        }
        return;
    }
    // output: lane q owns [basej, basej + G), the last lane up to the bucket end;
    // a bucket without records is written by its team's first lane
    if (tactive && (act || (nl == 0 && q == 0))) {
        uint64_t lo = basej, hi = (last || nl == 0) ? len : (uint64_t)basej + G;
        if (lo > len) lo = len;
        if (hi > len) hi = len;
        if (hi < lo) hi = lo;
        if (MODE == 3) {
            if (act) {
                uint32_t p = ystart;
                uint64_t jj = (uint64_t)basej - 1u;
                Win W = win_at(r, p);
                while (p < ynext) {
                    uint32_t gap, neg, k;
                    const uint32_t nq = record_at(r, x, p, gap, neg, k, W);
                    if (!nq) break;
                    jj += gap;
                    if (jj >= hi) break;
                    const float m = dequant_value(e_b, k, D.s, D.s_pow2 != 0u, D.inv_s);
                    D.v_hat[c0 + jj] = neg ? -m : m;
                    p = nq;
                }
            }
            return;
        }
        QuadWriter<ACC> w;
        w.init(D.v_hat, c0 + lo, c0 + hi);
        if (act) {
            uint32_t p = ystart;
            uint64_t jj = (uint64_t)basej - 1u;
            Win W = win_at(r, p);
            while (p < ynext) {
                uint32_t gap, neg, k;
                const uint32_t nq = record_at(r, x, p, gap, neg, k, W);
                if (!nq) break;
                jj += gap;
                if (jj >= hi) break;
                const float m = dequant_value(e_b, k, D.s, D.s_pow2 != 0u, D.inv_s);
                w.put(c0 + jj, neg ? -m : m);
                p = nq;
            }
        }
        w.finish();
    }
}

// Writes the group's buckets from the LDS level bytes: RN32(norm k / s)
// (dequant_value) with the byte's sign (+0.0f for k = 0), 16-byte stores for whole aligned
// quads of a bucket, single floats for quads that a bucket boundary cuts (ACC:
// added to the output). The value of each of the 256 level bytes is tabulated
// per bucket in `tbl` first.
template <bool RAGGED, bool ACC>
__device__ __forceinline__ void store_group(const DecodeParams &D, const uint8_t *lvl, const double *ebs,
                                            float *tbl, uint64_t lbase, uint64_t b0, uint64_t b1) {
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t *lw = reinterpret_cast<const uint32_t *>(lvl);
    for (uint64_t b = b0; b < b1; ++b) {
        const uint64_t A = bucket_first<RAGGED>(D, b), B = bucket_first<RAGGED>(D, b + 1);
        const double e = ebs[b - b0];
#pragma unroll
        for (uint32_t t = lane; t < 256u; t += 64u) {
            const float m = dequant_value(e, t & 127u, D.s, D.s_pow2 != 0u, D.inv_s);
            tbl[t] = __uint_as_float(__float_as_uint(m) | ((t & 128u) << 24));
        }
        wave_sync();
        const uint64_t qa = A >> 2, qb = (B + 3) >> 2;
        if (((A | B) & 3u) == 0) {
            // whole quads only: 32-bit quad indices from the bucket's first quad
            const uint32_t nq = (uint32_t)(qb - qa);
            const uint32_t *lq = lw + ((A - lbase) >> 2);
            float4 *oq = reinterpret_cast<float4 *>(D.v_hat + A);
            for (uint32_t i = lane; i < nq; i += 64) {
                const uint32_t word = lq[i];
                const float4 v = make_float4(tbl[word & 0xffu], tbl[(word >> 8) & 0xffu],
                                             tbl[(word >> 16) & 0xffu], tbl[word >> 24]);
                QuadWriter<ACC>::put4(reinterpret_cast<float *>(oq + i), v);
            }
        } else {
            for (uint64_t qd = qa + lane; qd < qb; qd += 64) {
                const uint64_t a = qd << 2;
                const uint32_t word = lw[(a - lbase) >> 2];
                const float v0 = tbl[word & 0xffu], v1 = tbl[(word >> 8) & 0xffu];
                const float v2 = tbl[(word >> 16) & 0xffu], v3 = tbl[word >> 24];
                if (a >= A && a + 4 <= B)
                    QuadWriter<ACC>::put4(D.v_hat + a, make_float4(v0, v1, v2, v3));
                else
                    QuadWriter<ACC>::put_part(D.v_hat, a, A, B, make_float4(v0, v1, v2, v3));
            }
        }
        // the table is rebuilt for the next bucket
        wave_sync();
    }
}

// Dynamic LDS: per wave the staged stream words, the group's level bytes and
// the per-bucket dequantization factors; then the record
// table.
constexpr size_t kStageBytes = (size_t)(kStageWords + kStagePad) * 8;
constexpr size_t kLevelBytes = (size_t)kGroupCoords + 32;
constexpr size_t kWaveLdsBytes = kStageBytes + kLevelBytes + 64 * 8;
static_assert(kStageBytes % 16 == 0 && kLevelBytes % 16 == 0, "LDS carve-out alignment");
// stream words of a group staged over the stage and the level buffer together
constexpr int kBigStageWords = (int)((kStageBytes + kLevelBytes) / 8) - kStagePad;
static_assert(kStageBytes >= 256 * sizeof(float), "the value table reuses the stage");
// two workgroups per CU (160 KB of LDS)
static_assert(2 * ((size_t)kDecWaves * kWaveLdsBytes + 16384) <= 160 * 1024, "decode LDS budget");

constexpr size_t decode_lds_bytes() { return (size_t)kDecWaves * kWaveLdsBytes + sizeof(RecordLut); }

// Whether the unit of buckets [ub0, ub1) of stream `offs` is decoded a lane per
// bucket: its stream words fit the stage and every bucket's bit length is at
// most kSoloMaxBits (which also makes its offsets non-decreasing). Uniform.
__device__ __forceinline__ bool solo_unit_ok(const uint64_t *offs, uint64_t ub0, uint64_t ub1,
                                             uint64_t total_words) {
    const uint64_t A0 = offs[ub0], E1 = offs[ub1];
    if (E1 < A0) return false;
    const uint64_t w0 = A0 >> 6;
    uint64_t w1 = (E1 + 63) >> 6;
    if (w1 > total_words) w1 = total_words;
    if (w1 > w0 && w1 - w0 > (uint64_t)kStageWords) return false;
    const uint64_t b = ub0 + (uint64_t)lane_id();
    bool bad = false;
    if (b < ub1) {
        const uint64_t A = offs[b], E = offs[b + 1];
        bad = E < A || E - A > (uint64_t)kSoloMaxBits;
    }
    return __ballot(bad) == 0;
}

// Coordinates of one bucket per window of the sparse-unit decode: a lane's row
// of the wave's tile (64 rows of fp32 in the level buffer).
constexpr uint32_t kSoloWin = 16;
static_assert(kSoloBuckets * kSoloWin * 4 <= kLevelBytes, "sparse-unit tile in the level buffer");

// Float index in the tile of coordinate i (0..15) of row `row`: the row's four
// quads rotated by the row number, so that lanes writing the same i of
// neighbouring rows hit different LDS banks.
__device__ __forceinline__ uint32_t solo_slot(uint32_t row, uint32_t i) {
    return row * kSoloWin + ((((i >> 2) ^ row) & 3u) << 2) + (i & 3u);
}

// Decodes the unit [ub0, ub1) (solo_unit_ok) of a plain decode. Lane i follows
// bucket ub0 + i from its first record; the value of each record is
// RN32(norm k / s) with its sign, every other coordinate +0.0f. Each bucket's
// coordinates are taken in windows of kSoloWin from its first 16-byte quad on:
// per window, each lane puts the values of its records in the window into its
// tile row (otherwise zero), and the wave stores the 64 rows with 16-byte
// stores, the quads a bucket shares with a neighbour element by element. Every
// output is thus written once, by coalesced stores.
template <bool RAGGED, int CODE>
__device__ __forceinline__ void solo_unit(const DecodeParams &D, const uint64_t *in, const uint64_t *offs,
                                          const uint32_t *lut, uint64_t *stage, float *tile, uint64_t ub0,
                                          uint64_t ub1, uint64_t total_words) {
    const uint32_t lane = (uint32_t)lane_id();
    const uint64_t w0 = offs[ub0] >> 6;
    uint64_t w1 = (offs[ub1] + 63) >> 6;
    if (w1 > total_words) w1 = total_words;
    const uint64_t nw = w1 > w0 ? w1 - w0 : 0;
    for (uint64_t i = lane; i < nw + kStagePad; i += 64)
        stage[i] = i < nw ? __builtin_bitreverse64(in[w0 + i]) : 0ull;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    {
        float4 *row4 = reinterpret_cast<float4 *>(tile + lane * kSoloWin);
#pragma unroll
        for (int q = 0; q < 4; ++q) row4[q] = z;
    }
    // this lane's bucket, coordinates relative to U (the unit's first quad)
    const uint64_t U = bucket_first<RAGGED>(D, ub0) & ~(uint64_t)3;
    const uint64_t b = ub0 + lane;
    uint32_t c0 = 0, c1 = 0;
    if (b < ub1) {
        c0 = (uint32_t)(bucket_first<RAGGED>(D, b) - U);
        c1 = (uint32_t)(bucket_first<RAGGED>(D, b + 1) - U);
    }
    const uint32_t a = c0 & ~3u;  // the row's first coordinate
    const uint32_t nwin = c1 > c0 ? (c1 - a + kSoloWin - 1) / kSoloWin : 0u;
    uint32_t maxwin = nwin;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) maxwin = max(maxwin, (uint32_t)__shfl_xor((int)maxwin, o));
    // the rows this lane stores: 16 r + lane / 4, quad lane % 4 of each window
    uint32_t ra[4], rc0[4], rc1[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int src = 16 * q + (int)(lane >> 2);
        ra[q] = (uint32_t)__shfl((int)a, src);
        rc0[q] = (uint32_t)__shfl((int)c0, src);
        rc1[q] = (uint32_t)__shfl((int)c1, src);
    }
    // the staged words and zeroed rows are read by other lanes of this wave
    wave_sync();

    const Bits<true> r{nullptr, 0u};
    const uint64_t gbit = w0 * 64 - (uint64_t)lds_address(stage) * 8;
    const uint32_t len = c1 - c0;
    uint32_t p = 0, E = 0;
    double e_b = 0.0;
    if (b < ub1) {
        p = (uint32_t)(offs[b] - gbit);
        E = (uint32_t)(offs[b + 1] - gbit);
        if (E >= p + 32u && len > 0) {
            e_b = (double)__uint_as_float(__builtin_bitreverse32((uint32_t)r.at(p)));
            p += 32u;
        } else {
            E = p;  // no records
        }
    }
    const RecordCtx<CODE> x{lut, bitlen32(len), bitlen32(D.s), D.s};
    Win W = win_at(r, p);
    uint32_t jj = ~0u;      // bucket index of the last record
    uint32_t rel = 0;       // row coordinate of the pending record
    float val = 0.0f;       // its value
    bool has = false;
    // the next record of the bucket, if any (a record that does not parse, or
    // lies past the bucket, ends it)
    auto next = [&]() {
        has = false;
        if (p < E) {
            uint32_t gap, neg, k;
            const uint32_t nq = record_at(r, x, p, gap, neg, k, W);
            if (nq) {
                jj += gap;
                if (jj < len) {
                    const float m = dequant_value(e_b, k, D.s, D.s_pow2 != 0u, D.inv_s);
                    val = neg ? -m : m;
                    rel = (c0 - a) + jj;
                    has = true;
                    p = nq;
                }
            }
        }
    };
    next();
    for (uint32_t i = 0; i < maxwin; ++i) {
        const uint32_t lo = i * kSoloWin;
        while (has && rel < lo + kSoloWin) {
            tile[solo_slot(lane, rel - lo)] = val;
            next();
        }
        wave_sync();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t row = 16u * (uint32_t)q + (lane >> 2);
            float4 *src = reinterpret_cast<float4 *>(tile + row * kSoloWin) + (((lane ^ row) & 3u));
            const float4 v = *src;
            *src = z;
            const uint32_t X = ra[q] + lo + 4u * (lane & 3u);
            if (X >= rc0[q] && X + 4u <= rc1[q])
                *reinterpret_cast<float4 *>(D.v_hat + U + X) = v;
            else  // a quad shared with a neighbouring bucket, or past the row's bucket
                QuadWriter<false>::put_part(D.v_hat + U, X, rc0[q], rc1[q], v);
        }
        // the rows are filled again for the next window
        wave_sync();
    }
}

// LDS_OUT: levels staged in LDS (D.lds_out), else each lane writes its range.
// ACC: the output accumulates the D.nstreams streams in order, per coordinate
// out = ((out + v_hat_0) + v_hat_1) + ...; the wave takes all streams of a
// group in turn, reading, adding to and writing back the group's outputs once
// per stream.
// One group of buckets [b0, b1) of every stream in turn (one stream for a plain
// decode; decode-accumulate adds each stream's values to the output before the
// next stream's): staged in the wave's LDS region, decoded, written.
template <bool RAGGED, bool LDS_OUT, bool ACC, int CODE>
__device__ __forceinline__ void decode_group_streams(const DecodeParams &D, const uint32_t *lut, uint64_t *stage,
                                                     uint8_t *lvl, double *ebs, uint64_t b0, uint64_t b1) {
    const int lane = lane_id();
    const uint64_t lbase = bucket_first<RAGGED>(D, b0) & ~(uint64_t)3;
    const uint32_t span = LDS_OUT ? (uint32_t)(bucket_first<RAGGED>(D, b1) - lbase) : 0u;
    const uint32_t nclear16 = (span + 3 + 15) >> 4;
    for (uint32_t k = 0; k < (ACC ? D.nstreams : 1u); ++k) {
        const uint64_t *in = D.in[k];
        const uint64_t *offs = D.offsets[k];
        const uint64_t total_words = (offs[D.nb] + 63) >> 6;
        const uint64_t A0 = offs[b0], E1 = offs[b1];
        const uint64_t w0 = A0 >> 6;
        uint64_t w1 = E1 > A0 ? ((E1 + 63) >> 6) : w0;
        if (w1 > total_words) w1 = total_words;
        const uint64_t nw = w1 > w0 ? w1 - w0 : 0;
        // a group whose stream does not fit the stage is staged over the
        // stage and the level buffer together (each lane then writes its
        // outputs directly), or, larger still, read from global memory
        const bool in_lds = nw <= (uint64_t)kStageWords;
        const bool in_big = !in_lds && nw <= (uint64_t)kBigStageWords;
        if (in_lds || in_big) {
            // bit-reversed words: stream bit 64 i + t of the group in bit t of word i
            for (uint64_t i = (uint64_t)lane; i < nw + kStagePad; i += 64)
                stage[i] = i < nw ? __builtin_bitreverse64(in[w0 + i]) : 0ull;
        }
        // staged words are read by other lanes of this wave
        wave_sync();
        // LDS positions are LDS bit addresses: the group's bit 0 is the first bit of stage
        Bits<true> rl{nullptr, 0u};
        const uint64_t lgbit = w0 * 64 - (uint64_t)lds_address(stage) * 8;
        Bits<false> rg{reinterpret_cast<const uint32_t *>(in + w0),
                       (uint32_t)(2 * (total_words - w0)) - 1u};
        if (in_lds)
            decode_group<RAGGED, true, LDS_OUT, ACC, CODE, true>(D, offs, lut, rl, lgbit, b0, b1, lvl, ebs,
                                                           lbase, nclear16);
        else if (in_big)
            decode_group<RAGGED, true, false, ACC, CODE, false>(D, offs, lut, rl, lgbit, b0, b1, lvl, ebs,
                                                          lbase, nclear16);
        else
            decode_group<RAGGED, false, LDS_OUT, ACC, CODE, true>(D, offs, lut, rg, w0 * 64, b0, b1, lvl,
                                                            ebs, lbase, nclear16);
        if (LDS_OUT && !in_big) {
            wave_sync();
            // the staged stream is done with: its space holds the value table
            store_group<RAGGED, ACC>(D, lvl, ebs, reinterpret_cast<float *>(stage), lbase, b0, b1);
        }
        // the LDS buffers are reused by the next stream or group of this wave
        wave_sync();
    }
}

template <bool RAGGED, bool LDS_OUT, bool ACC, int CODE>
__global__ __launch_bounds__(kDecWG) void decode_kernel(DecodeParams D) {
    extern __shared__ __align__(16) uint64_t dsmem[];
    __shared__ uint32_t next_item;  // the workgroup's next item (below)
    if (threadIdx.x == 0) next_item = 0;
    // record table after the waves' regions (a constant offset: folds into the
    // LDS instructions' offset field)
    uint32_t *lut = reinterpret_cast<uint32_t *>(reinterpret_cast<unsigned char *>(dsmem) +
                                                 (size_t)kDecWaves * kWaveLdsBytes);
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(CODE ? kRecordLutGamma.e : kRecordLut.e);
        uint4 *dst = reinterpret_cast<uint4 *>(lut);
        for (uint32_t i = threadIdx.x; i < sizeof(RecordLut) / 16; i += kDecWG) dst[i] = src[i];
    }
    __syncthreads();

    const int lane = lane_id();
    const int wv = wave_id();
    const uint32_t wofs = (uint32_t)wv * (uint32_t)kWaveLdsBytes;  // wave's bytes in dsmem
    unsigned char *wbase = reinterpret_cast<unsigned char *>(dsmem) + wofs;
    uint64_t *stage = reinterpret_cast<uint64_t *>(wbase);
    uint8_t *lvl = wbase + kStageBytes;
    double *ebs = reinterpret_cast<double *>(wbase + kStageBytes + kLevelBytes);
    const uint32_t tpw = D.tpw;
    const uint64_t ngroups = (D.nb + tpw - 1) / tpw;
    // Plain decodes with D.solo of a stream of at most kSoloAvgBits bits per
    // bucket on average go by units of kSoloBuckets buckets, a wave each: a
    // unit that qualifies is decoded a lane per bucket (solo_unit), the groups
    // of any other by the same wave in turn. For such streams the host launches
    // a wave per unit rather than the resident workgroups, so that workgroups
    // start as others finish: the memory system serves the resident waves
    // unevenly, and a fixed share of units per wave would leave the slowest
    // waves running alone at the end. Otherwise the waves take groups in turn.
    const bool solo = !ACC && LDS_OUT && D.solo != 0u &&
                      D.offsets[0][D.nb] <= D.nb * (uint64_t)kSoloAvgBits;
    const uint64_t gpu = kSoloBuckets / tpw;  // groups per unit (with solo)
    const uint64_t items = solo ? (D.nb + kSoloBuckets - 1) / kSoloBuckets : ngroups;
    // Workgroup b of G takes the consecutive items [b N / G, (b + 1) N / G) of
    // the N, so that the workgroups' shares differ by at most one. Its waves
    // take them one at a time from a counter in LDS, so waves that the SIMDs
    // serve faster (the older ones of a workgroup issue first) take more (c3:
    // with a fixed share per wave the last wave ended 37% after the median one).
    const uint64_t ibase = items * blockIdx.x / gridDim.x;
    const uint64_t ilim = items * (blockIdx.x + 1) / gridDim.x;
    while (true) {
        uint32_t k = 0;
        if (lane == 0) k = atomicAdd(&next_item, 1u);
        k = (uint32_t)__builtin_amdgcn_readfirstlane((int)k);
        const uint64_t w = ibase + k;
        if (w >= ilim) break;
        uint64_t g0 = w, g1 = w + 1;
        if (solo) {
            const uint64_t ub0 = w * kSoloBuckets;
            const uint64_t ub1 = ub0 + kSoloBuckets < D.nb ? ub0 + kSoloBuckets : D.nb;
            const uint64_t *offs = D.offsets[0];
            const uint64_t total_words = (offs[D.nb] + 63) >> 6;
            if (solo_unit_ok(offs, ub0, ub1, total_words)) {
                solo_unit<RAGGED, CODE>(D, D.in[0], offs, lut, stage, reinterpret_cast<float *>(lvl), ub0, ub1,
                                        total_words);
                continue;
            }
            g0 = w * gpu;
            g1 = g0 + gpu < ngroups ? g0 + gpu : ngroups;
        }
        for (uint64_t g = g0; g < g1; ++g) {
            const uint64_t b0 = g * tpw;
            const uint64_t b1 = b0 + tpw < D.nb ? b0 + tpw : D.nb;
            decode_group_streams<RAGGED, LDS_OUT, ACC, CODE>(D, lut, stage, lvl, ebs, b0, b1);
        }
    }
}


// ---- decode-accumulate with the streams of a group folded once ------------------
// For k <= kDecWaves streams over uniform buckets of kFoldMinD or more
// coordinates, a multiple of 4, with levels that fit a byte (the LDS level
// path). The waves of a workgroup take the k streams of P = kDecWaves / k
// consecutive groups at once, wave w stream w % k of group w / k: each decodes
// its stream's part of the group into level bytes in its own LDS region. Then,
// bucket by bucket, each such wave tabulates the 256 level bytes' values of its
// stream's bucket in its stage, and the whole workgroup adds the k values of
// every coordinate to the output in stream order, ((acc + v_0) + v_1) + ...:
// the output is read and written once per call instead of once per stream. A
// group with a stream that does not fit the stage is done by the wave of its
// first stream alone, stream by stream (decode_group_streams).
constexpr uint32_t kFoldMinD = 256;

template <int CODE>
__global__ __launch_bounds__(kDecWG) void accumulate_fold_kernel(DecodeParams D) {
    extern __shared__ __align__(16) uint64_t dsmem[];
    __shared__ uint32_t fold_slot[kDecWaves];  // group slot p of the round is folded
    unsigned char *base = reinterpret_cast<unsigned char *>(dsmem);
    uint32_t *lut = reinterpret_cast<uint32_t *>(base + (size_t)kDecWaves * kWaveLdsBytes);
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(CODE ? kRecordLutGamma.e : kRecordLut.e);
        uint4 *dst = reinterpret_cast<uint4 *>(lut);
        for (uint32_t i = threadIdx.x; i < sizeof(RecordLut) / 16; i += kDecWG) dst[i] = src[i];
    }
    __syncthreads();

    const int lane = lane_id();
    const uint32_t wv = (uint32_t)wave_id();
    unsigned char *wbase = base + (size_t)wv * kWaveLdsBytes;
    uint64_t *stage = reinterpret_cast<uint64_t *>(wbase);
    uint8_t *lvl = wbase + kStageBytes;
    double *ebs = reinterpret_cast<double *>(wbase + kStageBytes + kLevelBytes);
    const uint32_t K = D.nstreams;          // 1 .. kDecWaves
    const uint32_t P = kDecWaves / K;       // groups per round
    const uint32_t slot = wv / K, j = wv - slot * K;
    const uint32_t tpw = D.tpw, d = D.d;
    const uint32_t nqd = d >> 2;            // quads per bucket
    const uint64_t ngroups = (D.nb + tpw - 1) / tpw;
    const uint64_t rounds = (ngroups + P - 1) / P;
    // workgroup b of G takes the consecutive rounds [b R / G, (b + 1) R / G)
    const uint64_t r0 = rounds * blockIdx.x / gridDim.x, r1 = rounds * (blockIdx.x + 1) / gridDim.x;
    for (uint64_t r = r0; r < r1; ++r) {
        const uint64_t g = r * P + slot;
        const bool mine = slot < P && g < ngroups;
        const uint64_t b0 = g * tpw;
        const uint64_t b1 = b0 + tpw < D.nb ? b0 + tpw : D.nb;
        bool fold = false;
        if (mine) {
            // the group fits the stage in every stream (lane t looks at stream t)
            bool ok = true;
            if ((uint32_t)lane < K) {
                const uint64_t *offs = D.offsets[lane];
                const uint64_t total_words = (offs[D.nb] + 63) >> 6;
                const uint64_t A0 = offs[b0], E1 = offs[b1];
                const uint64_t w0 = A0 >> 6;
                uint64_t w1 = E1 > A0 ? ((E1 + 63) >> 6) : w0;
                if (w1 > total_words) w1 = total_words;
                ok = (w1 > w0 ? w1 - w0 : 0) <= (uint64_t)kStageWords;
            }
            fold = __ballot(!ok) == 0;
            if (fold) {
                const uint64_t *in = D.in[j];
                const uint64_t *offs = D.offsets[j];
                const uint64_t total_words = (offs[D.nb] + 63) >> 6;
                const uint64_t A0 = offs[b0], E1 = offs[b1];
                const uint64_t w0 = A0 >> 6;
                uint64_t w1 = E1 > A0 ? ((E1 + 63) >> 6) : w0;
                if (w1 > total_words) w1 = total_words;
                const uint64_t nw = w1 > w0 ? w1 - w0 : 0;
                for (uint64_t i = (uint64_t)lane; i < nw + kStagePad; i += 64)
                    stage[i] = i < nw ? __builtin_bitreverse64(in[w0 + i]) : 0ull;
                wave_sync();
                const Bits<true> rl{nullptr, 0u};
                const uint64_t lgbit = w0 * 64 - (uint64_t)lds_address(stage) * 8;
                const uint64_t lbase = b0 * d;
                const uint32_t nclear16 = ((uint32_t)(bucket_first<false>(D, b1) - lbase) + 3 + 15) >> 4;
                decode_group<false, true, true, false, CODE, true>(D, offs, lut, rl, lgbit, b0, b1, lvl, ebs,
                                                                   lbase, nclear16);
                wave_sync();
            } else if (j == 0) {
                decode_group_streams<false, true, true, CODE>(D, lut, stage, lvl, ebs, b0, b1);
            }
        }
        if (slot < P && j == 0 && lane == 0) fold_slot[slot] = fold ? 1u : 0u;
        __syncthreads();
        if (tpw > 1u && D.s_pow2) {
            // several buckets per group and s a power of two: each value formed
            // directly, (k * (norm / s)) rounded once (dequant_value), every
            // bucket of the round in one pass
            const uint32_t gq = tpw * nqd;  // quads per group
            for (uint32_t i = threadIdx.x; i < P * gq; i += kDecWG) {
                const uint32_t p = i / gq, gi = i - p * gq;
                const uint32_t t = 4u * gi / d;
                const uint64_t bb = (r * P + p) * tpw + t;
                if (!fold_slot[p] || bb >= D.nb) continue;
                const uint64_t a = (r * P + p) * tpw * (uint64_t)d + 4u * gi;
                if (a >= D.n) continue;
                const unsigned char *sb = base + (size_t)(p * K) * kWaveLdsBytes;
                float *o = D.v_hat + a;
                const bool whole = a + 4u <= D.n;
                float4 x;
                if (whole) {
                    x = *reinterpret_cast<const float4 *>(o);
                } else {
                    x.x = o[0];
                    x.y = a + 1u < D.n ? o[1] : 0.0f;
                    x.z = a + 2u < D.n ? o[2] : 0.0f;
                    x.w = 0.0f;
                }
                for (uint32_t jj = 0; jj < K; ++jj) {
                    const unsigned char *wb = sb + (size_t)jj * kWaveLdsBytes;
                    const uint32_t word = *reinterpret_cast<const uint32_t *>(wb + kStageBytes + 4u * gi);
                    const double e = reinterpret_cast<const double *>(wb + kStageBytes + kLevelBytes)[t];
                    float v4[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint32_t byte = (word >> (8 * u)) & 0xffu;
                        const float m = dequant_value(e, byte & 127u, D.s, true, D.inv_s);
                        v4[u] = __uint_as_float(__float_as_uint(m) | ((byte & 128u) << 24));
                    }
                    x.x = x.x + v4[0];
                    x.y = x.y + v4[1];
                    x.z = x.z + v4[2];
                    x.w = x.w + v4[3];
                }
                if (whole) {
                    *reinterpret_cast<float4 *>(o) = x;
                } else {
                    o[0] = x.x;
                    if (a + 1u < D.n) o[1] = x.y;
                    if (a + 2u < D.n) o[2] = x.z;
                }
            }
            // the level bytes are reused by the next round
            __syncthreads();
            continue;
        }
        for (uint32_t t = 0; t < tpw; ++t) {
            // this wave's stream: the values of bucket b0 + t's 256 level bytes
            if (fold && b0 + t < b1) {
                float *tbl = reinterpret_cast<float *>(stage);
                const double e = ebs[t];
#pragma unroll
                for (uint32_t v = (uint32_t)lane; v < 256u; v += 64u) {
                    const float m = dequant_value(e, v & 127u, D.s, D.s_pow2 != 0u, D.inv_s);
                    tbl[v] = __uint_as_float(__float_as_uint(m) | ((v & 128u) << 24));
                }
            }
            __syncthreads();
            // bucket t of every folded group: quad i of group slot p
            for (uint32_t i = threadIdx.x; i < P * nqd; i += kDecWG) {
                const uint32_t p = i / nqd, qi = i - p * nqd;
                const uint64_t bb = (r * P + p) * tpw + t;
                if (!fold_slot[p] || bb >= D.nb) continue;
                const uint64_t a = bb * d + 4u * qi;
                if (a >= D.n) continue;
                const uint32_t li = t * d + 4u * qi;  // the quad's level bytes in the group's buffer
                const unsigned char *sb = base + (size_t)(p * K) * kWaveLdsBytes;
                float *o = D.v_hat + a;
                const bool whole = a + 4u <= D.n;
                float4 x;
                if (whole) {
                    x = *reinterpret_cast<const float4 *>(o);
                } else {
                    x.x = o[0];
                    x.y = a + 1u < D.n ? o[1] : 0.0f;
                    x.z = a + 2u < D.n ? o[2] : 0.0f;
                    x.w = 0.0f;
                }
                for (uint32_t jj = 0; jj < K; ++jj) {
                    const unsigned char *wb = sb + (size_t)jj * kWaveLdsBytes;
                    const uint32_t word = *reinterpret_cast<const uint32_t *>(wb + kStageBytes + li);
                    const float *tb = reinterpret_cast<const float *>(wb);
                    x.x = x.x + tb[word & 0xffu];
                    x.y = x.y + tb[(word >> 8) & 0xffu];
                    x.z = x.z + tb[(word >> 16) & 0xffu];
                    x.w = x.w + tb[word >> 24];
                }
                if (whole) {
                    *reinterpret_cast<float4 *>(o) = x;
                } else {
                    o[0] = x.x;
                    if (a + 1u < D.n) o[1] = x.y;
                    if (a + 2u < D.n) o[2] = x.z;
                }
            }
            // the tables and level bytes are reused by the next bucket and round
            __syncthreads();
        }
    }
}

// ---- buckets longer than a chunk ---------------------------------------------
// A bucket whose payload is too long for one team is cut into chunks of
// kChunkBits bits, one wave each:
//   chunk_parse_kernel: the team parses its chunk as a bucket whose lane 0
//     starts on a guess (chunk 0: the exact payload start), giving the gap sum T
//     along that chain to its exit X; lane 0 then follows the true chain on from
//     X and the next chunk's lane-0 chain from that chunk's start, always
//     stepping the one behind, until they meet at y (within kChunkMerge bits):
//     y is an exact record boundary of the next chunk, with gx the gaps from X
//     to y and g0 those of the next chunk's chain before y;
//   chunk_scan_kernel: per bucket, chunk c holds the records from y_{c-1} to
//     y_c, whose gaps sum to T_c - g0_{c-1} + gx_c; a scan gives each chunk its
//     first coordinate;
//   chunk_write_kernel: each chunk decoded from its exact start y_{c-1} to y_c
//     by the same team parse (lane writers);
//   chunk_fallback_kernel: a bucket where two chains do not meet within the
//     window (or whose stream is malformed) is decoded whole by one team.
// Their records live in the library's fixed scratch.
constexpr uint32_t kChunkBits = 64u * 256u;   // 256 bits per lane
constexpr uint32_t kChunkMerge = 8192u;       // bits of the next chunk the merge search may use
constexpr uint32_t kChunkFail = 0xffffffffu;

struct ChunkRec {       // per chunk slot, written by chunk_parse_kernel
    uint32_t y;         // merge point relative to the bucket's first stream bit (kChunkFail: none)
    uint32_t g0, T, gx;
};

struct ChunkParams {
    DecodeParams D;
    const uint64_t *in;       // the stream
    const uint64_t *offs;     // its bucket offsets
    ChunkRec *rec;            // [nb * nch]
    uint32_t *vstart;         // [nb * nch] exact start of chunk c's records (relative to the bucket)
    uint32_t *vbase;          // [nb * nch] bucket index of chunk c's first coordinate
    uint32_t *bstate;         // [nb * 2]: chunks in use, failed flag
    uint32_t nch;             // chunk slots per bucket
};

// The payload bit range and chunk count of bucket b (chunk_end).
__device__ __forceinline__ void chunk_bucket(const ChunkParams &C, uint64_t b, uint64_t &A, uint64_t &E,
                                             uint64_t &nbits, uint32_t &nact) {
    A = C.offs[b];
    E = C.offs[b + 1];
    nbits = E >= A + 32 ? E - A - 32 : 0;
    nact = nbits <= kChunkBits ? (nbits ? 1u : 0u) : (uint32_t)(nbits / kChunkBits);
}

// End of chunk c of nact starting at payload bit P: whole chunks of kChunkBits
// bits, the last one taking the rest (fewer than 2 kChunkBits bits), so that a
// chain started on a guess in it has at least kChunkBits bits to meet the exact
// one before the bucket ends.
__device__ __forceinline__ uint64_t chunk_end(uint64_t P, uint32_t c, uint32_t nact, uint64_t E) {
    return c + 1 >= nact ? E : P + (uint64_t)(c + 1) * kChunkBits;
}

// Lanes and segment length of a team parse of [P0, E) (as decode_group sets them).
__device__ __forceinline__ uint32_t chunk_lane0_end(uint32_t P0, uint32_t E) {
    if (E <= P0) return E;
    uint32_t nl = (E - P0) / (uint32_t)kSyncWin;
    nl = nl < 64u ? nl : 64u;
    if (nl == 0) nl = 1;
    const uint32_t seg = ((E - P0) + nl - 1u) / nl;
    return nl == 1u ? E : P0 + seg;
}

// Stages stream words [w0, w0 + nw) of `in` (zeros at and past total words)
// bit-reversed into the wave's LDS region, with kStagePad zero words after.
__device__ __forceinline__ void chunk_stage(uint64_t *stage, const uint64_t *in, uint64_t w0, uint64_t nw,
                                            uint64_t total_words) {
    for (uint64_t i = (uint64_t)lane_id(); i < nw + kStagePad; i += 64)
        stage[i] = (i < nw && w0 + i < total_words) ? __builtin_bitreverse64(in[w0 + i]) : 0ull;
    wave_sync();
}

constexpr uint64_t kChunkStageWords = (uint64_t)kBigStageWords;
static_assert((2 * kChunkBits + kChunkMerge + 256) / 64 + 2 <= kChunkStageWords, "chunk stage");

template <int CODE>
__global__ __launch_bounds__(kDecWG) void chunk_parse_kernel(ChunkParams C) {
    extern __shared__ __align__(16) uint64_t dsmem[];
    uint32_t *lut = reinterpret_cast<uint32_t *>(reinterpret_cast<unsigned char *>(dsmem) +
                                                 (size_t)kDecWaves * kWaveLdsBytes);
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(CODE ? kRecordLutGamma.e : kRecordLut.e);
        uint4 *dst = reinterpret_cast<uint4 *>(lut);
        for (uint32_t i = threadIdx.x; i < sizeof(RecordLut) / 16; i += kDecWG) dst[i] = src[i];
    }
    __syncthreads();
    const int wv = wave_id();
    uint64_t *stage = reinterpret_cast<uint64_t *>(reinterpret_cast<unsigned char *>(dsmem) +
                                                   (size_t)wv * kWaveLdsBytes);
    const uint64_t slot = (uint64_t)blockIdx.x * kDecWaves + (uint64_t)wv;
    const uint64_t b = slot / C.nch;
    const uint32_t c = (uint32_t)(slot % C.nch);
    if (b >= C.D.nb) return;
    uint64_t A, E, nbits;
    uint32_t nact;
    chunk_bucket(C, b, A, E, nbits, nact);
    if (c >= nact || E - A >= (1ull << 31)) return;
    const uint64_t c0 = b * C.D.d;
    const uint64_t blen = (c0 + C.D.d < C.D.n ? c0 + C.D.d : C.D.n) - c0;
    const bool guess = guess_bucket(nbits, blen);
    const uint64_t total_words = (C.offs[C.D.nb] + 63) >> 6;
    // stage from the word holding the chunk's first bit through the merge window
    const uint64_t cs = A + 32 + (uint64_t)c * kChunkBits;
    const uint64_t ce = chunk_end(A + 32, c, nact, E);
    const uint64_t w0 = cs >> 6;
    const uint64_t wl = (ce + kChunkMerge + 256 + 63) >> 6;
    chunk_stage(stage, C.in, w0, wl - w0, total_words);
    Bits<true> rl{nullptr, 0u};
    const uint64_t lgbit = w0 * 64 - (uint64_t)lds_address(stage) * 8;
    const uint32_t P0r = (uint32_t)(cs - lgbit), Er = (uint32_t)(ce - lgbit);
    GroupView gv{P0r, Er, 0, 0, blen, 0.0, guess, c > 0};
    ChunkOut co{0, P0r};
    decode_group<false, true, false, false, CODE, false, 1>(C.D, nullptr, lut, rl, lgbit, 0, 0, nullptr,
                                                            nullptr, 0, 0, &gv, &co);
    ChunkRec rec{kChunkFail, 0, co.T, 0};
    if (lane_id() == 0) {
        const RecordCtx<CODE> x{lut, bitlen32((uint32_t)blen), bitlen32(C.D.s), C.D.s};
        const uint32_t Eb = (uint32_t)(E - lgbit);
        if (ce == E) {
            // the last chunk: its chain must end exactly at the bucket's end
            if (co.X == Eb) rec.y = (uint32_t)(E - A);
        } else {
            // the next chunk's lane 0 starts at ce with the same guess steps
            uint32_t pa = co.X, pb = Er, ga = 0, gb = 0;
            Win Wa = win_at(rl, pa), Wb = win_at(rl, pb);
            const uint64_t ce2 = chunk_end(A + 32, c + 1, nact, E);
            if (guess) guess_steps(rl, x, pb, chunk_lane0_end(Er, (uint32_t)(ce2 - lgbit)), gb, Wb);
            const uint32_t lim = Er + kChunkMerge;
            while (pa != pb && pa <= lim && pb <= lim && pa <= Eb && pb <= Eb) {
                if (pa < pb) chain_step(rl, x, pa, ga, Wa);
                else chain_step(rl, x, pb, gb, Wb);
            }
            if (pa == pb && pa <= lim && pa <= Eb) {
                rec.y = (uint32_t)(pa + lgbit - A);
                rec.g0 = gb;
                rec.gx = ga;
            }
        }
        C.rec[slot] = rec;
    }
}

// One workgroup per bucket: each chunk's first coordinate, or the bucket marked
// failed.
__global__ __launch_bounds__(kWG) void chunk_scan_kernel(ChunkParams C) {
    __shared__ uint64_t tot[kWG];
    __shared__ uint32_t bad;
    const uint64_t b = blockIdx.x;
    const uint32_t j = threadIdx.x;
    uint64_t A, E, nbits;
    uint32_t nact;
    chunk_bucket(C, b, A, E, nbits, nact);
    const uint64_t c0 = b * C.D.d;
    const uint64_t blen = (c0 + C.D.d < C.D.n ? c0 + C.D.d : C.D.n) - c0;
    // a bucket without payload (or shorter than its norm) is written by the
    // fallback, which writes its zeros (accumulates them: -0.0f + +0.0f)
    if (j == 0) bad = (nact == 0 || nact > C.nch || E - A >= (1ull << 31)) ? 1u : 0u;
    __syncthreads();
    const uint32_t na = bad ? 0u : nact;
    // thread j takes chunks [j * per, (j + 1) * per)
    const uint32_t per = (na + kWG - 1) / kWG;
    const ChunkRec *R = C.rec + b * C.nch;
    uint64_t sum = 0;
    uint32_t mybad = 0;
    for (uint32_t i = 0; i < per; ++i) {
        const uint32_t cc = j * per + i;
        if (cc >= na) break;
        const ChunkRec rc = R[cc];
        const uint32_t g0p = cc ? R[cc - 1].g0 : 0u;
        if (rc.y == kChunkFail || (cc && R[cc - 1].y == kChunkFail) || rc.T < g0p) mybad = 1u;
        sum += (uint64_t)rc.T - g0p + rc.gx;
    }
    tot[j] = sum;
    if (mybad) bad = 1u;
    __syncthreads();
    uint64_t base = 0, all = 0;
    for (uint32_t v = 0; v < kWG; ++v) {
        if (v < j) base += tot[v];
        all += tot[v];
    }
    if (all > blen) bad = 1u;
    __syncthreads();
    if (!bad) {
        for (uint32_t i = 0; i < per; ++i) {
            const uint32_t cc = j * per + i;
            if (cc >= na) break;
            const ChunkRec rc = R[cc];
            C.vstart[b * C.nch + cc] = cc ? R[cc - 1].y : 32u;
            C.vbase[b * C.nch + cc] = (uint32_t)base;
            base += (uint64_t)rc.T - (cc ? R[cc - 1].g0 : 0u) + rc.gx;
        }
    }
    if (j == 0) {
        C.bstate[2 * b] = na;
        C.bstate[2 * b + 1] = bad;
    }
}

// The bucket norm from the stream's 32 bits at bit A.
__device__ __forceinline__ float chunk_norm(const uint64_t *in, uint64_t A) {
    const uint64_t w = in[A >> 6];
    const uint32_t sh = (uint32_t)(A & 63u);
    uint64_t x = w << sh;
    if (sh > 32u) x |= in[(A >> 6) + 1] >> (64u - sh);
    return __uint_as_float((uint32_t)(x >> 32));
}

template <bool ACC, int CODE>
__global__ __launch_bounds__(kDecWG) void chunk_write_kernel(ChunkParams C) {
    extern __shared__ __align__(16) uint64_t dsmem[];
    uint32_t *lut = reinterpret_cast<uint32_t *>(reinterpret_cast<unsigned char *>(dsmem) +
                                                 (size_t)kDecWaves * kWaveLdsBytes);
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(CODE ? kRecordLutGamma.e : kRecordLut.e);
        uint4 *dst = reinterpret_cast<uint4 *>(lut);
        for (uint32_t i = threadIdx.x; i < sizeof(RecordLut) / 16; i += kDecWG) dst[i] = src[i];
    }
    __syncthreads();
    const int wv = wave_id();
    uint64_t *stage = reinterpret_cast<uint64_t *>(reinterpret_cast<unsigned char *>(dsmem) +
                                                   (size_t)wv * kWaveLdsBytes);
    const uint64_t slot = (uint64_t)blockIdx.x * kDecWaves + (uint64_t)wv;
    const uint64_t b = slot / C.nch;
    const uint32_t c = (uint32_t)(slot % C.nch);
    if (b >= C.D.nb) return;
    const uint32_t na = C.bstate[2 * b], bad = C.bstate[2 * b + 1];
    if (bad || c >= na) return;
    uint64_t A, E, nbits;
    uint32_t nact;
    chunk_bucket(C, b, A, E, nbits, nact);
    const uint64_t c0 = b * C.D.d;
    const uint64_t blen = (c0 + C.D.d < C.D.n ? c0 + C.D.d : C.D.n) - c0;
    const bool guess = guess_bucket(nbits, blen);
    const uint64_t vs = A + C.vstart[slot];
    const uint64_t ve = A + C.rec[slot].y;
    const uint64_t base = C.vbase[slot];
    const uint64_t vend = c + 1 < na ? C.vbase[slot + 1] : blen;
    const uint64_t total_words = (C.offs[C.D.nb] + 63) >> 6;
    const uint64_t w0 = vs >> 6;
    const uint64_t wl = (ve + 256 + 63) >> 6;
    chunk_stage(stage, C.in, w0, wl - w0, total_words);
    Bits<true> rl{nullptr, 0u};
    const uint64_t lgbit = w0 * 64 - (uint64_t)lds_address(stage) * 8;
    GroupView gv{(uint32_t)(vs - lgbit), (uint32_t)(ve - lgbit), c0 + base, vend - base, blen,
                 (double)chunk_norm(C.in, A), guess, false};
    // a plain decode's output was zeroed first (zero_fill_kernel): only values are written
    decode_group<false, true, false, ACC, CODE, false, ACC ? 2 : 3>(C.D, nullptr, lut, rl, lgbit, 0, 0,
                                                                    nullptr, nullptr, 0, 0, &gv, nullptr);
}

// +0.0f to p[0, n) (p 16-byte aligned), 16-byte stores.
__global__ __launch_bounds__(kWG) void zero_fill_kernel(float *p, uint64_t n) {
    const uint64_t nq = n >> 2;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    const uint64_t stride = (uint64_t)gridDim.x * kWG;
    for (uint64_t i = (uint64_t)blockIdx.x * kWG + threadIdx.x; i < nq; i += stride)
        reinterpret_cast<float4 *>(p)[i] = z;
    if (blockIdx.x == 0 && threadIdx.x < (n & 3u)) p[(nq << 2) + threadIdx.x] = 0.0f;
}

// One wave per bucket: a failed bucket decoded whole by one team, reading the
// stream from global memory.
template <bool ACC, int CODE>
__global__ __launch_bounds__(kDecWG) void chunk_fallback_kernel(ChunkParams C) {
    extern __shared__ __align__(16) uint64_t dsmem[];
    uint32_t *lut = reinterpret_cast<uint32_t *>(reinterpret_cast<unsigned char *>(dsmem) +
                                                 (size_t)kDecWaves * kWaveLdsBytes);
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(CODE ? kRecordLutGamma.e : kRecordLut.e);
        uint4 *dst = reinterpret_cast<uint4 *>(lut);
        for (uint32_t i = threadIdx.x; i < sizeof(RecordLut) / 16; i += kDecWG) dst[i] = src[i];
    }
    __syncthreads();
    const uint64_t b = (uint64_t)blockIdx.x * kDecWaves + (uint64_t)wave_id();
    if (b >= C.D.nb || !C.bstate[2 * b + 1]) return;
    const uint64_t total_words = (C.offs[C.D.nb] + 63) >> 6;
    const uint64_t A0 = C.offs[b];
    const uint64_t w0 = A0 >> 6;
    if (w0 >= total_words || C.offs[b + 1] - A0 >= (1ull << 31)) return;
    Bits<false> rg{reinterpret_cast<const uint32_t *>(C.in + w0), (uint32_t)(2 * (total_words - w0)) - 1u};
    decode_group<false, false, false, ACC, CODE, false>(C.D, C.offs, lut, rg, w0 * 64, b, b + 1, nullptr,
                                                        nullptr, 0, 0);
}
}  // namespace qsgd
