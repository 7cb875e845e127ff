// Decoder: parses the Elias-omega stream and dequantizes.
//
// Page "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding",
// definition paragraph: the coding is lossless, so decode inverts it exactly;
// Q_s(v)_i = ||v|| sgn(v_i) k_i / s, evaluated as RN32(k * RN64(norm / s)).
//
// Work split. A wave64 owns a group of consecutive buckets and a team of T lanes
// (T = 1..64, chosen from the bucket size) decodes each bucket. The wave first
// copies the group's stream words into LDS with coalesced loads and clears the
// group's output coordinates with coalesced 16-byte stores; values are then
// scattered on top.
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
//            restarts from lane q's true exit; pairs are repaired in order.
//   count:   each lane's index span is the sum of the gaps of its exact records
//            (phase A + B sums minus those before its sync point, re-parsed);
//            a team prefix sum gives absolute indices.
//   write:   each lane parses its exact range again and stores the values.
// Record parsing: a 64-bit MSB-aligned bit window refilled 32 bits at a time
// from LDS, and a 4096-entry table indexed by the next 12 bits that decodes a
// whole record (gap <= 16, k <= 16) at once; longer codewords take the general
// omega loop.
#pragma once

#include "qsgd_device.h"

namespace qsgd {

constexpr int kLutBits = 12;
constexpr int kSyncWin = 128;       // bits
constexpr int kStageWords = 512;    // 64-bit stream words staged per wave

struct DecodeParams {
    const uint64_t *in;
    const uint64_t *offsets;
    const uint64_t *bstart;  // ragged table or nullptr
    float *v_hat;
    uint64_t n;
    uint64_t nb;
    uint32_t s;
    uint32_t d;
    uint32_t team;           // lanes per bucket (power of two, 1..64)
};

// Record table: entry for the next 12 stream bits. bits 0-3: record length
// (0: the record is longer than 12 bits or has gap/level > 16), 4-7: gap - 1,
// 8-11: k - 1, 12: sign.
__device__ inline void build_record_lut(uint16_t *lut) {
    for (uint32_t i = threadIdx.x; i < (1u << kLutBits); i += blockDim.x) {
        int pos = 0;
        auto take = [&](int nbits) -> int {
            if (pos + nbits > kLutBits) return -1;
            const int v = (int)((i >> (kLutBits - pos - nbits)) & ((1u << nbits) - 1u));
            pos += nbits;
            return v;
        };
        auto omega = [&]() -> int {  // Elias omega, values up to 16
            int N = 1;
            while (true) {
                const int b = take(1);
                if (b < 0) return -1;
                if (b == 0) return N;
                const int v = take(N);
                if (v < 0) return -1;
                N = (1 << N) | v;
                if (N > 16) return -1;
            }
        };
        uint16_t e = 0;
        const int gap = omega();
        if (gap > 0) {
            const int sg = take(1);
            if (sg >= 0) {
                const int k = omega();
                if (k > 0) e = (uint16_t)(pos | ((gap - 1) << 4) | ((k - 1) << 8) | (sg << 12));
            }
        }
        lut[i] = e;
    }
}


// Bit positions are relative to the first stream word of the wave's bucket
// group; a group spans fewer than 2^31 bits (buckets of at most 2^24
// coordinates).
//
// MSB-first bit window over the stream. Half-word h (32 bits) is the high (h
// even) or low (h odd) half of 64-bit word h / 2, i.e. dword h ^ 1 in memory.
// LDS mode reads the group's staged words (padded with zero words, so no bound
// check is needed); global mode reads the stream and treats half-words past
// `hlast` as zero.
template <bool LDS>
struct Reader {
    const uint32_t *src;
    uint32_t hlast;
    uint64_t win;   // next bits, MSB-aligned
    uint32_t nb;    // valid bits in win (>= 32 after every step)
    uint32_t next;  // next half-word to load

    __device__ __forceinline__ uint32_t half(uint32_t h) const {
        if (LDS) return src[h ^ 1u];
        return h <= hlast ? src[h ^ 1u] : 0u;
    }
    __device__ __forceinline__ void seek(uint32_t p) {
        const uint32_t h = p >> 5, off = p & 31u;
        const uint64_t w = ((uint64_t)half(h) << 32) | (uint64_t)half(h + 1);
        win = w << off;
        nb = 64u - off;
        next = h + 2u;
    }
    __device__ __forceinline__ uint32_t pos() const { return next * 32u - nb; }
    __device__ __forceinline__ void consume(uint32_t n) {  // 1 <= n <= 32
        win <<= n;
        nb -= n;
        if (nb < 32u) {
            win |= (uint64_t)half(next) << (32u - nb);
            nb += 32u;
            ++next;
        }
    }
};

// General omega decoding (Elias 1975): N = 1; while the next bit is 1, that bit
// and the N bits after it form the new N; a 0 ends the codeword. 0 = invalid (a
// group longer than maxbits).
template <bool LDS>
__device__ __forceinline__ uint32_t read_omega(Reader<LDS> &r, uint32_t maxbits) {
    uint32_t N = 1;
    while (true) {
        if ((r.win >> 63) == 0) {
            r.consume(1);
            return N;
        }
        const uint32_t g = N + 1u;
        if (g > maxbits) return 0;
        N = (uint32_t)(r.win >> (64u - g));
        r.consume(g);
    }
}

struct RecordCtx {
    const uint16_t *lut;
    uint32_t gbits, kbits, s;
};

// One record omega(gap) | sign | omega(k). False if it does not parse. The table
// covers records of at most 12 bits with gap, k <= 16 (it does not check k <= s
// or gap <= bucket length: on the true chain those hold anyway, and a
// speculative chain only has to be a deterministic function of its start).
template <bool LDS>
__device__ __forceinline__ bool read_record(Reader<LDS> &r, const RecordCtx &x, uint32_t &gap,
                                            uint32_t &neg, uint32_t &k) {
    const uint32_t e = x.lut[(uint32_t)(r.win >> (64 - kLutBits))];
    if (e & 15u) {
        gap = ((e >> 4) & 15u) + 1u;
        k = ((e >> 8) & 15u) + 1u;
        neg = (e >> 12) & 1u;
        r.consume(e & 15u);
        return true;
    }
    gap = read_omega(r, x.gbits);
    if (gap == 0) return false;
    neg = (uint32_t)(r.win >> 63);
    r.consume(1);
    k = read_omega(r, x.kbits);
    return k != 0 && k <= x.s;
}

__device__ __forceinline__ uint32_t bitlen32(uint32_t x) { return 32u - (uint32_t)__clz(x); }

__device__ __forceinline__ bool mask_has(uint64_t m0, uint64_t m1, uint32_t rel) {
    return rel < 64u ? ((m0 >> rel) & 1u) : (rel < 128u ? ((m1 >> (rel - 64u)) & 1u) : false);
}

// Parse state of one lane over its bucket.
struct Chain {
    uint32_t x;      // first chain position >= segment end (the exit)
    uint32_t ynext;  // where the chain met the next lane's chain (or E)
    uint32_t ga;     // gap sum of records starting before the exit
    uint32_t gb;     // gap sum of records from the exit to ynext
    bool found;
};

// Phase A: follows a chain from `start` to its first position >= sn (the exit).
// With `mark`, positions in [start, start + 128) where it starts a record are
// set in own0/own1.
template <bool LDS>
__device__ __forceinline__ void follow_chain(Reader<LDS> &r, const RecordCtx &x, uint32_t start,
                                             uint32_t sn, uint32_t E, bool mark, uint64_t &own0,
                                             uint64_t &own1, Chain &c) {
    uint32_t pos = start;
    r.seek(pos);
    c.ga = 0;
    c.gb = 0;
    while (pos < sn) {
        if (mark) {
            const uint32_t rel = pos - start;
            if (rel < 64u) own0 |= 1ull << rel;
            else if (rel < 128u) own1 |= 1ull << (rel - 64u);
        }
        uint32_t gap, neg, k;
        if (read_record(r, x, gap, neg, k) && r.pos() <= E) {
            pos = r.pos();
            c.ga += gap;
        } else {
            pos = pos + 1u;
            r.seek(pos);
        }
    }
    c.x = pos;
    c.found = false;
    c.ynext = E;
}

// Phase B: continues the chain from its exit until it lands on a position noted
// by the next lane (window nxt0/nxt1 starting at sn) or on E; gives up after
// 128 bits or at an invalid record.
template <bool LDS>
__device__ __forceinline__ void extend_chain(Reader<LDS> &r, const RecordCtx &x, uint32_t sn,
                                             uint32_t E, uint64_t nxt0, uint64_t nxt1, Chain &c) {
    uint32_t pos = c.x;
    r.seek(pos);
    while (true) {
        if (pos == E) { c.found = true; c.ynext = E; return; }
        const uint32_t rel = pos - sn;
        if (rel >= (uint32_t)kSyncWin) return;
        if (mask_has(nxt0, nxt1, rel)) { c.found = true; c.ynext = pos; return; }
        uint32_t gap, neg, k;
        if (!(read_record(r, x, gap, neg, k) && r.pos() <= E)) return;
        pos = r.pos();
        c.gb += gap;
    }
}

// Writes one lane's output range [lo, hi) in index order, exactly once: values
// and the zeros between them, 16-byte stores for whole aligned quads inside the
// range, single floats for the partial quads at its ends.
struct QuadWriter {
    float *out;
    uint64_t lo, hi, q;
    float v0, v1, v2, v3;

    __device__ __forceinline__ void init(float *o, uint64_t l, uint64_t h) {
        out = o; lo = l; hi = h; q = l >> 2;
        v0 = v1 = v2 = v3 = 0.0f;
    }
    __device__ __forceinline__ void flush() const {
        const uint64_t a = q << 2;
        if (a >= lo && a + 4 <= hi) {
            *reinterpret_cast<float4 *>(out + a) = make_float4(v0, v1, v2, v3);
        } else {
            if (a >= lo && a < hi) out[a] = v0;
            if (a + 1 >= lo && a + 1 < hi) out[a + 1] = v1;
            if (a + 2 >= lo && a + 2 < hi) out[a + 2] = v2;
            if (a + 3 >= lo && a + 3 < hi) out[a + 3] = v3;
        }
    }
    // moves to quad nq > q: writes the current quad and the all-zero quads between
    __device__ __forceinline__ void advance(uint64_t nq) {
        flush();
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
        for (uint64_t t = q + 1; t < nq; ++t) *reinterpret_cast<float4 *>(out + (t << 2)) = z;
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
    if (RAGGED) return D.bstart[b];
    const uint64_t g = b * D.d;
    return g < D.n ? g : D.n;
}

// Decodes the buckets [b0, b1) of one wave group; `src` holds the group's
// stream from bit `gbit` on (LDS: staged; global: the stream itself).
template <bool RAGGED, bool LDS>
__device__ __forceinline__ void decode_group(const DecodeParams &D, const uint16_t *lut,
                                             const uint32_t *src, uint32_t hlast, uint64_t gbit,
                                             uint64_t b0, uint64_t b1) {
    const int lane = lane_id();
    const uint32_t T = D.team;
    const uint32_t q = (uint32_t)lane % T;
    const uint32_t team = (uint32_t)lane / T;

    Reader<LDS> r;
    r.src = src;
    r.hlast = hlast;

    const uint64_t b = b0 + team;
    const bool tactive = b < b1;
    uint32_t A = 0, E = 0;
    uint64_t c0 = 0, len = 0;
    double e_b = 0.0;
    uint32_t nl = 0;
    if (tactive) {
        A = (uint32_t)(D.offsets[b] - gbit);
        E = (uint32_t)(D.offsets[b + 1] - gbit);
        c0 = bucket_first<RAGGED>(D, b);
        len = bucket_first<RAGGED>(D, b + 1) - c0;
        if (E >= A + 32u && len > 0) {
            r.seek(A);
            const float norm = __uint_as_float((uint32_t)(r.win >> 32));
            e_b = (double)norm / (double)D.s;
            const uint32_t Lp = E - (A + 32u);
            if (Lp > 0) {
                const uint32_t m = Lp / (uint32_t)kSyncWin;
                nl = m < T ? m : T;
                if (nl == 0) nl = 1;
            }
        }
    }
    RecordCtx x{lut, tactive ? bitlen32((uint32_t)len) : 1u, bitlen32(D.s), D.s};
    const uint32_t P0 = A + 32u;
    const uint32_t seg = nl ? ((E - P0) + nl - 1u) / nl : 0u;
    const bool act = q < nl;
    const bool last = q + 1u >= nl;
    const uint32_t sq = act ? P0 + q * seg : E;
    const uint32_t sn = act ? (last ? E : sq + seg) : E;

    // phase A on every lane's own segment, noting its first 128 bits
    uint64_t own0 = 0, own1 = 0;
    Chain c{E, E, 0u, 0u, false};
    if (act) follow_chain(r, x, sq, sn, E, true, own0, own1, c);
    if (act && last) { c.found = true; c.ynext = E; }
    // phase B against the next lane's window
    const uint64_t nxt0 = __shfl_down(own0, 1, (int)T);
    const uint64_t nxt1 = __shfl_down(own1, 1, (int)T);
    if (act && !last) extend_chain(r, x, sn, E, nxt0, nxt1, c);

    // repair: restart, in order, every lane whose predecessor did not meet it.
    // All lanes below the lowest broken lane of a team are exact and each round
    // repairs that lane, so the loop ends after at most T rounds.
    bool repaired = false;
    uint32_t rstart = 0;
    while (true) {
        const bool pf = __shfl_up(c.found ? 1 : 0, 1, (int)T) != 0;
        const uint32_t px = __shfl_up(c.x, 1, (int)T);
        const bool broken = act && q >= 1 && !pf && !repaired;
        const uint64_t bm = __ballot(broken);
        if (bm == 0) break;
        const uint64_t team_mask = (T == 64) ? ~0ull : (((1ull << T) - 1ull) << (team * T));
        const uint64_t below = bm & team_mask & ((1ull << lane) - 1ull);
        const bool fix = broken && below == 0;
        // the predecessor of a restarted lane ends at its own exit
        const bool succ_fix = __shfl_down(fix ? 1 : 0, 1, (int)T) != 0 && !last;
        if (act && succ_fix) {
            c.ynext = c.x;
            c.gb = 0;
            c.found = true;
        }
        if (fix) {
            uint64_t d0 = 0, d1 = 0;
            follow_chain(r, x, px, sn, E, false, d0, d1, c);
            if (last) { c.found = true; c.ynext = E; }
            else extend_chain(r, x, sn, E, nxt0, nxt1, c);
            repaired = true;
            rstart = px;
        }
    }

    // exact start of each lane's records
    const uint32_t py = __shfl_up(c.ynext, 1, (int)T);
    uint32_t ystart = E;
    if (act) {
        if (q == 0) ystart = P0;
        else if (repaired) ystart = rstart;
        else ystart = py;
    }
    // gaps of the records before the sync point (same speculative chain)
    uint32_t gpre = 0;
    if (act && q >= 1 && !repaired && ystart > sq) {
        uint32_t pos = sq;
        r.seek(pos);
        while (pos < ystart) {
            uint32_t gap, neg, k;
            if (read_record(r, x, gap, neg, k) && r.pos() <= E) {
                pos = r.pos();
                gpre += gap;
            } else {
                pos = pos + 1u;
                r.seek(pos);
            }
        }
    }
    const uint32_t G = act ? c.ga + c.gb - gpre : 0u;
    // team-exclusive prefix sum of the index spans
    uint32_t incl = G;
    for (uint32_t off = 1; off < T; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off, (int)T);
        if (q >= off) incl += y;
    }
    const uint32_t basej = incl - G;

    // output: lane q owns [basej, basej + G), the last lane up to the bucket end;
    // a bucket without records is written by its team's first lane
    if (tactive && (act || (nl == 0 && q == 0))) {
        uint64_t lo = basej, hi = (last || nl == 0) ? len : (uint64_t)basej + G;
        if (lo > len) lo = len;
        if (hi > len) hi = len;
        if (hi < lo) hi = lo;
        QuadWriter w;
        w.init(D.v_hat, c0 + lo, c0 + hi);
        if (act && ystart < c.ynext) {
            r.seek(ystart);
            int64_t jj = (int64_t)basej - 1;
            while (r.pos() < c.ynext) {
                uint32_t gap, neg, k;
                if (!read_record(r, x, gap, neg, k)) break;
                jj += gap;
                if (jj >= (int64_t)hi) break;
                const float m = (float)((double)k * e_b);
                w.put(c0 + (uint64_t)jj, neg ? -m : m);
            }
        }
        w.finish();
    }
}

// Dynamic LDS: the record table, then per wave kStageWords + 2 staged words.
template <bool RAGGED>
__global__ __launch_bounds__(kWG) void decode_kernel(DecodeParams D) {
    extern __shared__ __align__(16) uint64_t dsmem[];
    uint16_t *lut = reinterpret_cast<uint16_t *>(dsmem);
    build_record_lut(lut);
    __syncthreads();

    const int lane = lane_id();
    const int wv = wave_id();
    uint64_t *stage = dsmem + (1u << kLutBits) / 4 + (size_t)wv * (kStageWords + 2);
    const uint32_t T = D.team;
    const uint32_t tpw = 64u / T;
    const uint64_t ngroups = (D.nb + tpw - 1) / tpw;
    const uint64_t total_bits = D.offsets[D.nb];
    const uint64_t total_words = (total_bits + 63) >> 6;

    for (uint64_t g = (uint64_t)blockIdx.x * kWaves + (uint64_t)wv; g < ngroups;
         g += (uint64_t)gridDim.x * kWaves) {
        const uint64_t b0 = g * tpw;
        const uint64_t b1 = b0 + tpw < D.nb ? b0 + tpw : D.nb;
        const uint64_t A0 = D.offsets[b0], E1 = D.offsets[b1];
        const uint64_t w0 = A0 >> 6;
        uint64_t w1 = E1 > A0 ? ((E1 + 63) >> 6) : w0;
        if (w1 > total_words) w1 = total_words;
        const uint64_t nw = w1 > w0 ? w1 - w0 : 0;
        if (nw <= (uint64_t)kStageWords) {
            for (uint64_t i = (uint64_t)lane; i < nw + 2; i += 64) stage[i] = i < nw ? D.in[w0 + i] : 0ull;
            // the staged words are read by other lanes of this wave
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            decode_group<RAGGED, true>(D, lut, reinterpret_cast<const uint32_t *>(stage), 0u, w0 * 64,
                                       b0, b1);
        } else {
            const uint32_t hlast = (uint32_t)(2 * (total_words - w0)) - 1u;
            decode_group<RAGGED, false>(D, lut, reinterpret_cast<const uint32_t *>(D.in + w0), hlast,
                                        w0 * 64, b0, b1);
        }
        // the stage buffer is reused by the next group of this wave
        __builtin_amdgcn_wave_barrier();
    }
}

constexpr size_t decode_lds_bytes() {
    return (size_t)(1u << kLutBits) * 2 + (size_t)kWaves * (kStageWords + 2) * 8;
}

}  // namespace qsgd
