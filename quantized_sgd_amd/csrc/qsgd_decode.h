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
constexpr int kStageWords = 1024;   // 64-bit stream words staged per wave

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

// MSB-first bit window over the stream. Half-word h (32 bits) of the stream is
// the high (h even) or low (h odd) half of 64-bit word h / 2, i.e. dword h ^ 1
// in memory. Half-words past `hlast` read as zero.
struct Reader {
    const uint32_t *lds;   // staged half-words, lds[0] = half-word hbase (even)
    const uint32_t *glb;   // the whole stream as dwords
    int64_t hbase, hlast;
    bool use_lds;
    uint64_t win;          // next bits, MSB-aligned
    int nb;                // valid bits in win (>= 32 after every step)
    int64_t next;          // next half-word to load

    __device__ __forceinline__ uint32_t half(int64_t h) const {
        if (h > hlast) return 0u;
        return use_lds ? lds[(h - hbase) ^ 1] : glb[h ^ 1];
    }
    __device__ __forceinline__ void seek(uint64_t p) {
        const int64_t h = (int64_t)(p >> 5);
        const int off = (int)(p & 31u);
        const uint64_t w = ((uint64_t)half(h) << 32) | (uint64_t)half(h + 1);
        win = w << off;
        nb = 64 - off;
        next = h + 2;
    }
    __device__ __forceinline__ uint64_t pos() const { return (uint64_t)next * 32u - (uint64_t)nb; }
    __device__ __forceinline__ void consume(int n) {  // 1 <= n <= 32
        win <<= n;
        nb -= n;
        if (nb < 32) {
            win |= (uint64_t)half(next) << (32 - nb);
            nb += 32;
            ++next;
        }
    }
};

// General omega decoding (Elias 1975): N = 1; while the next bit is 1, that bit
// and the N bits after it form the new N; a 0 ends the codeword. 0 = invalid
// (a group longer than maxbits).
__device__ __forceinline__ uint32_t read_omega(Reader &r, uint32_t maxbits) {
    uint32_t N = 1;
    while (true) {
        if ((r.win >> 63) == 0) {
            r.consume(1);
            return N;
        }
        const uint32_t g = N + 1u;
        if (g > maxbits) return 0;
        N = (uint32_t)(r.win >> (64u - g));
        r.consume((int)g);
    }
}

// One record omega(gap) | sign | omega(k). False if it does not parse.
__device__ __forceinline__ bool read_record(Reader &r, const uint16_t *lut, uint32_t gbits,
                                            uint32_t kbits, uint32_t s, uint32_t &gap,
                                            uint32_t &neg, uint32_t &k) {
    const uint32_t e = lut[(uint32_t)(r.win >> (64 - kLutBits))];
    if (e & 15u) {
        gap = ((e >> 4) & 15u) + 1u;
        k = ((e >> 8) & 15u) + 1u;
        neg = (e >> 12) & 1u;
        r.consume((int)(e & 15u));
        return true;
    }
    gap = read_omega(r, gbits);
    if (gap == 0) return false;
    neg = (uint32_t)(r.win >> 63);
    r.consume(1);
    k = read_omega(r, kbits);
    return k != 0 && k <= s;
}

__device__ __forceinline__ uint32_t bitlen32(uint32_t x) { return 32u - (uint32_t)__clz(x); }

__device__ __forceinline__ bool mask_has(uint64_t m0, uint64_t m1, uint64_t rel) {
    return rel < 64 ? ((m0 >> rel) & 1u) : (rel < 128 ? ((m1 >> (rel - 64)) & 1u) : false);
}

// Parse-state of one lane over its bucket.
struct Chain {
    uint64_t x;      // first chain position >= segment end (the exit)
    uint64_t ynext;  // where the chain met the next lane's chain (or E)
    uint32_t ga;     // gap sum of records starting before the exit
    uint32_t gb;     // gap sum of records from the exit to ynext
    bool found;
};

// Phase A: follows a chain from `start` to its first position >= sn (the exit).
// Positions in [mark0, mark0 + 128) where it starts a record are recorded in
// own0/own1 when `mark` is set.
__device__ __forceinline__ void follow_chain(Reader &r, const uint16_t *lut, uint32_t gbits,
                                             uint32_t kbits, uint32_t s, uint64_t start, uint64_t sn,
                                             uint64_t E, bool /*last*/, bool mark, uint64_t mark0,
                                             uint64_t &own0, uint64_t &own1, Chain &c) {
    uint64_t pos = start;
    r.seek(pos);
    c.ga = 0;
    c.gb = 0;
    while (pos < sn) {
        if (mark) {
            const uint64_t rel = pos - mark0;
            if (rel < 64) own0 |= 1ull << rel;
            else if (rel < 128) own1 |= 1ull << (rel - 64);
        }
        uint32_t gap, neg, k;
        if (read_record(r, lut, gbits, kbits, s, gap, neg, k) && r.pos() <= E) {
            pos = r.pos();
            c.ga += gap;
        } else {
            pos = pos + 1;
            r.seek(pos);
        }
    }
    c.x = pos;
    c.found = false;
    c.ynext = E;
}

// Phase B: continues the chain from its exit until it lands on a position noted
// by the next lane (window nxt0/nxt1 starting at sn) or on E; gives up after
// 128 bits.
__device__ __forceinline__ void extend_chain(Reader &r, const uint16_t *lut, uint32_t gbits,
                                             uint32_t kbits, uint32_t s, uint64_t sn, uint64_t E,
                                             uint64_t nxt0, uint64_t nxt1, Chain &c) {
    uint64_t pos = c.x;
    r.seek(pos);
    while (true) {
        if (pos == E) { c.found = true; c.ynext = E; return; }
        const uint64_t rel = pos - sn;
        if (rel >= (uint64_t)kSyncWin) return;
        if (mask_has(nxt0, nxt1, rel)) { c.found = true; c.ynext = pos; return; }
        uint32_t gap, neg, k;
        if (!(read_record(r, lut, gbits, kbits, s, gap, neg, k) && r.pos() <= E)) return;
        pos = r.pos();
        c.gb += gap;
    }
}

template <bool RAGGED>
__device__ __forceinline__ uint64_t bucket_first(const DecodeParams &D, uint64_t b) {
    if (RAGGED) return D.bstart[b];
    const uint64_t g = b * D.d;
    return g < D.n ? g : D.n;
}

// Clears v_hat[c0, c1) with 16-byte stores where aligned (one wave).
__device__ __forceinline__ void zero_fill(float *v, uint64_t c0, uint64_t c1, int lane) {
    if (c1 <= c0) return;
    uint64_t a = (c0 + 3) & ~(uint64_t)3;
    if (a > c1) a = c1;
    const uint64_t z = c1 & ~(uint64_t)3;
    for (uint64_t i = c0 + (uint64_t)lane; i < a; i += 64) v[i] = 0.0f;
    if (z > a) {
        float4 *p = reinterpret_cast<float4 *>(v + a);
        const uint64_t nq = (z - a) >> 2;
        const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
        for (uint64_t i = (uint64_t)lane; i < nq; i += 64) p[i] = zero;
    }
    for (uint64_t i = (z > a ? z : a) + (uint64_t)lane; i < c1; i += 64) v[i] = 0.0f;
}

template <bool RAGGED>
__global__ __launch_bounds__(kWG) void decode_kernel(DecodeParams D) {
    __shared__ uint16_t lut[1 << kLutBits];
    __shared__ uint64_t stage[kWaves][kStageWords];
    build_record_lut(lut);
    __syncthreads();

    const int lane = lane_id();
    const int wv = wave_id();
    const uint32_t T = D.team;
    const uint32_t tpw = 64u / T;            // buckets per wave group
    const uint32_t q = (uint32_t)lane % T;   // lane within its team
    const uint32_t team = (uint32_t)lane / T;
    const uint64_t ngroups = (D.nb + tpw - 1) / tpw;
    const uint64_t total_bits = D.offsets[D.nb];
    const int64_t hlast_all = (int64_t)((total_bits + 31) >> 5) - 1;
    const uint32_t kbits = bitlen32(D.s);
    const uint32_t *glb = reinterpret_cast<const uint32_t *>(D.in);
    const uint32_t *lds = reinterpret_cast<const uint32_t *>(stage[wv]);

    for (uint64_t g = (uint64_t)blockIdx.x * kWaves + (uint64_t)wv; g < ngroups;
         g += (uint64_t)gridDim.x * kWaves) {
        const uint64_t b0 = g * tpw;
        const uint64_t b1 = b0 + tpw < D.nb ? b0 + tpw : D.nb;
        const uint64_t A0 = D.offsets[b0], E1 = D.offsets[b1];
        // stage the group's stream words
        const uint64_t w0 = A0 >> 6;
        const uint64_t w1 = E1 > A0 ? ((E1 + 63) >> 6) : w0;
        const bool use_lds = (w1 - w0) <= (uint64_t)kStageWords && E1 >= A0;
        if (use_lds) {
            uint32_t *st32 = reinterpret_cast<uint32_t *>(stage[wv]);
            const uint32_t *src = reinterpret_cast<const uint32_t *>(D.in + w0);
            for (uint64_t i = (uint64_t)lane; i < 2 * (w1 - w0); i += 64) st32[i] = src[i];
        }
        // the staged words are read by other lanes of this wave
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // clear the group's coordinates
        zero_fill(D.v_hat, bucket_first<RAGGED>(D, b0), bucket_first<RAGGED>(D, b1), lane);

        Reader r;
        r.lds = lds;
        r.glb = glb;
        r.use_lds = use_lds;
        r.hbase = (int64_t)(w0 * 2);
        r.hlast = use_lds ? (int64_t)(w1 * 2) - 1 : hlast_all;
        if (r.hlast > hlast_all) r.hlast = hlast_all;

        const uint64_t b = b0 + team;
        const bool tactive = b < b1;
        uint64_t A = 0, E = 0, c0 = 0, len = 0;
        double e_b = 0.0;
        uint32_t nl = 0;
        if (tactive) {
            A = D.offsets[b];
            E = D.offsets[b + 1];
            c0 = bucket_first<RAGGED>(D, b);
            len = bucket_first<RAGGED>(D, b + 1) - c0;
            if (E >= A + 32 && len > 0) {
                r.seek(A);
                const float norm = __uint_as_float((uint32_t)(r.win >> 32));
                e_b = (double)norm / (double)D.s;
                const uint64_t Lp = E - (A + 32);
                if (Lp > 0) {
                    const uint64_t m = Lp / kSyncWin;
                    nl = (uint32_t)(m < T ? m : T);
                    if (nl == 0) nl = 1;
                }
            }
        }
        const uint32_t gbits = tactive ? bitlen32((uint32_t)len) : 1u;
        const uint64_t P0 = A + 32;
        const uint64_t seg = nl ? ((E - P0) + nl - 1) / nl : 0;
        const bool act = q < nl;
        const bool last = q + 1 >= nl;
        const uint64_t sq = act ? P0 + (uint64_t)q * seg : E;
        const uint64_t sn = act ? (last ? E : sq + seg) : E;

        // phase A on every lane's own segment, noting its first 128 bits
        uint64_t own0 = 0, own1 = 0;
        Chain c{E, E, 0, 0, false};
        if (act)
            follow_chain(r, lut, gbits, kbits, D.s, sq, sn, E, last, true, sq, own0, own1, c);
        if (act && last) { c.found = true; c.ynext = E; }
        // phase B against the next lane's window
        uint64_t nxt0 = __shfl_down(own0, 1, (int)T);
        uint64_t nxt1 = __shfl_down(own1, 1, (int)T);
        if (act && !last) extend_chain(r, lut, gbits, kbits, D.s, sn, E, nxt0, nxt1, c);

        // repair: restart, in order, every lane whose predecessor did not meet it;
        // all lanes below the lowest broken lane of a team are exact, and each
        // round repairs that lane, so the loop ends after at most T rounds
        bool repaired = false;
        uint64_t rstart = 0;
        while (true) {
            const bool pf = __shfl_up(c.found ? 1 : 0, 1, (int)T) != 0;
            const uint64_t px = __shfl_up(c.x, 1, (int)T);
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
                follow_chain(r, lut, gbits, kbits, D.s, px, sn, E, last, false, 0, d0, d1, c);
                if (last) { c.found = true; c.ynext = E; }
                else extend_chain(r, lut, gbits, kbits, D.s, sn, E, nxt0, nxt1, c);
                repaired = true;
                rstart = px;
            }
        }

        // exact start of each lane's records
        const uint64_t py = __shfl_up(c.ynext, 1, (int)T);
        uint64_t ystart = E;
        if (act) {
            if (q == 0) ystart = P0;
            else if (repaired) ystart = rstart;
            else ystart = py;
        }
        // gaps before the sync point (re-parse of the speculative prefix)
        uint32_t gpre = 0;
        if (act && q >= 1 && !repaired && ystart > sq) {
            uint64_t pos = sq;
            r.seek(pos);
            while (pos < ystart) {
                uint32_t gap, neg, k;
                if (read_record(r, lut, gbits, kbits, D.s, gap, neg, k) && r.pos() <= E) {
                    pos = r.pos();
                    gpre += gap;
                } else {
                    pos = pos + 1;
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

        // the cleared coordinates must be in memory before values land on them
        __builtin_amdgcn_s_waitcnt(0);
        if (act && ystart < c.ynext) {
            float *out = D.v_hat + c0;
            r.seek(ystart);
            int64_t jj = (int64_t)basej - 1;
            while (r.pos() < c.ynext) {
                uint32_t gap, neg, k;
                if (!read_record(r, lut, gbits, kbits, D.s, gap, neg, k)) break;
                jj += gap;
                if (jj >= (int64_t)len) break;
                const float m = (float)((double)k * e_b);
                out[jj] = neg ? -m : m;
            }
        }
    }
}

}  // namespace qsgd
