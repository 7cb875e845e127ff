// Decoder: parses the Elias-omega stream and dequantizes.
//
// Page "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding",
// definition paragraph: the coding is lossless, so decode inverts it exactly;
// Q_s(v)_i = ||v|| sgn(v_i) k_i / s, evaluated as RN32(k * RN64(norm / s)).
//
// One wave64 decodes one bucket at a time. A bucket's records form a chain that
// can only be followed serially, so the wave splits the bucket's payload into
// equal bit segments and every lane parses its segment speculatively from the
// segment start (a guess at a record boundary):
//   pass 1: lane q follows a chain from its start s_q to s_{q+1} + 64 and records
//           the record boundaries it visits in the 64-bit windows after s_q
//           ("own") and after s_{q+1} ("ext"). A chain that hits an invalid code
//           restarts one bit later. Lane 0 starts at a true boundary.
//   sync:   two chains that meet at one position coincide from there on. If lane
//           q is on the true chain by s_{q+1}, the first common position of its
//           ext window and lane q+1's own window is the first true boundary lane
//           q+1 visits; from there lane q+1 is on the true chain. Segments of at
//           least 64 bits keep every sync point inside its lane's segment.
//   pass 2: each lane re-parses its exact record range, counting the index
//           distance it covers; a wave prefix sum gives absolute indices.
//   pass 3: each lane parses the range again and stores the values.
// If some pair of neighbours never meets inside the window, lane 0 decodes the
// whole bucket serially. The bucket's coordinates are first cleared to +0.0f
// with coalesced stores.
#pragma once

#include "qsgd_device.h"

namespace qsgd {

struct DecodeParams {
    const uint64_t *in;
    const uint64_t *offsets;
    const uint64_t *bstart;  // ragged table or nullptr
    float *v_hat;
    uint64_t n;
    uint64_t nb;
    uint32_t s;
    uint32_t d;
};

// Reads bits MSB-first from the stream; words past `last_word` read as zero.
struct BitReader {
    const uint64_t *in;
    int64_t last_word;
    uint64_t w0, w1;
    uint64_t widx;
    uint32_t boff;

    __device__ __forceinline__ uint64_t load(uint64_t i) const {
        return (int64_t)i <= last_word ? in[i] : 0ull;
    }
    __device__ __forceinline__ void seek(uint64_t pos) {
        widx = pos >> 6;
        boff = (uint32_t)(pos & 63u);
        w0 = load(widx);
        w1 = load(widx + 1);
    }
    __device__ __forceinline__ uint64_t pos() const { return widx * 64u + boff; }
    __device__ __forceinline__ uint64_t peek() const {
        return boff ? (w0 << boff) | (w1 >> (64u - boff)) : w0;
    }
    __device__ __forceinline__ void skip(uint32_t nbits) {  // nbits <= 64
        uint32_t b = boff + nbits;
        if (b >= 64u) {
            w0 = w1;
            ++widx;
            w1 = load(widx + 1);
            b -= 64u;
        }
        boff = b;
    }
};

// Omega decoding (Elias 1975): N = 1; while the next bit is 1, that bit and the N
// bits after it form the new N; a 0 ends the codeword. Returns 0 for a codeword
// whose groups exceed `maxbits` bits (no valid value that large).
__device__ __forceinline__ uint32_t read_omega(BitReader &br, uint32_t maxbits) {
    uint32_t N = 1;
    while (true) {
        const uint64_t w = br.peek();
        if ((w >> 63) == 0) {
            br.skip(1);
            return N;
        }
        const uint32_t g = N + 1u;
        if (g > maxbits) return 0;
        N = (uint32_t)(w >> (64u - g));
        br.skip(g);
    }
}

// One record: omega(gap) | sign | omega(k). False if it is not a valid record
// ending at or before `end`.
__device__ __forceinline__ bool read_record(BitReader &br, uint64_t end, uint32_t gbits,
                                            uint32_t kbits, uint32_t s, uint32_t &gap,
                                            uint32_t &neg, uint32_t &k) {
    gap = read_omega(br, gbits);
    if (gap == 0) return false;
    neg = (uint32_t)(br.peek() >> 63);
    br.skip(1);
    k = read_omega(br, kbits);
    if (k == 0 || k > s) return false;
    return br.pos() <= end;
}

__device__ __forceinline__ uint32_t bitlen32(uint32_t x) { return 32u - (uint32_t)__clz(x); }

template <bool RAGGED>
__device__ void decode_bucket(const DecodeParams &D, uint64_t b, int64_t last_word) {
    const int lane = lane_id();
    const uint64_t A = D.offsets[b], E = D.offsets[b + 1];
    uint64_t g0, len;
    if (RAGGED) {
        g0 = D.bstart[b];
        len = D.bstart[b + 1] - g0;
    } else {
        g0 = b * D.d;
        len = D.n - g0 < D.d ? D.n - g0 : D.d;
    }
    float *out = D.v_hat + g0;
    for (uint64_t i = (uint64_t)lane; i < len; i += 64) out[i] = 0.0f;
    if (E < A + 32 || len == 0) return;  // malformed: leave zeros

    BitReader br{D.in, last_word, 0, 0, 0, 0};
    br.seek(A);
    const uint32_t nbits_norm = (uint32_t)(br.peek() >> 32);
    const float norm = __uint_as_float(nbits_norm);
    const double e_b = (double)norm / (double)D.s;
    const uint64_t P0 = A + 32, Lp = E - P0;
    const uint32_t gbits = bitlen32((uint32_t)len);
    const uint32_t kbits = bitlen32(D.s);

    // order the zero stores before the value stores of other lanes
    __builtin_amdgcn_s_waitcnt(0);

    const uint32_t nl = (uint32_t)(Lp / 64u < 64u ? Lp / 64u : 64u);
    bool serial = nl <= 1;
    uint64_t ystart = P0, yend = E;
    if (!serial) {
        const uint64_t seg = (Lp + nl - 1) / nl;
        const uint32_t q = (uint32_t)lane;
        const bool act = q < nl;
        const uint64_t sq = P0 + (uint64_t)q * seg;
        const uint64_t sn = (q + 1 < nl) ? sq + seg : E;
        uint64_t own = 0, ext = 0;
        if (act) {
            const uint64_t limit = (q + 1 < nl) ? (sn + 64 < E ? sn + 64 : E) : E;
            uint64_t pos = sq;
            br.seek(pos);
            while (pos < limit) {
                if (pos - sq < 64) own |= 1ull << (pos - sq);
                if (pos >= sn) ext |= 1ull << (pos - sn);
                uint32_t gap, neg, k;
                if (read_record(br, E, gbits, kbits, D.s, gap, neg, k)) {
                    pos = br.pos();
                } else {
                    pos = pos + 1;
                    br.seek(pos);
                }
            }
            if (pos == E) {
                if (E - sq < 64) own |= 1ull << (E - sq);
                if (E >= sn && E - sn < 64) ext |= 1ull << (E - sn);
            }
        }
        const uint64_t own_next = __shfl_down(own, 1, 64);
        const uint64_t common = (act && q + 1 < nl) ? (ext & own_next) : 0ull;
        const bool ok = !(act && q + 1 < nl) || common != 0;
        serial = !__all(ok);
        if (!serial) {
            const uint64_t ynext = (act && q + 1 < nl) ? sn + (uint64_t)__builtin_ctzll(common) : E;
            const uint64_t yprev = __shfl_up(ynext, 1, 64);
            ystart = (q == 0) ? P0 : yprev;
            yend = ynext;
            // pass 2: index distance covered by this lane's records
            uint32_t G = 0;
            if (act && ystart < yend) {
                br.seek(ystart);
                while (br.pos() < yend) {
                    uint32_t gap, neg, k;
                    if (!read_record(br, yend, gbits, kbits, D.s, gap, neg, k)) break;
                    G += gap;
                }
            }
            const uint32_t incl = wave_incl_scan(G, [](uint32_t a, uint32_t c) { return a + c; });
            const uint32_t basej = incl - G;
            // pass 3: store
            if (act && ystart < yend) {
                br.seek(ystart);
                int64_t jj = (int64_t)basej - 1;
                while (br.pos() < yend) {
                    uint32_t gap, neg, k;
                    if (!read_record(br, yend, gbits, kbits, D.s, gap, neg, k)) break;
                    jj += gap;
                    if (jj >= (int64_t)len) break;
                    const float m = (float)((double)k * e_b);
                    out[jj] = neg ? -m : m;
                }
            }
            return;
        }
    }
    // serial decode of the whole bucket by lane 0
    if (lane == 0) {
        br.seek(P0);
        int64_t jj = -1;
        while (br.pos() < E) {
            uint32_t gap, neg, k;
            if (!read_record(br, E, gbits, kbits, D.s, gap, neg, k)) break;
            jj += gap;
            if (jj >= (int64_t)len) break;
            const float m = (float)((double)k * e_b);
            out[jj] = neg ? -m : m;
        }
    }
}

template <bool RAGGED>
__global__ __launch_bounds__(kWG) void decode_kernel(DecodeParams D) {
    const uint64_t total_bits = D.offsets[D.nb];
    const int64_t last_word = (int64_t)((total_bits + 63) >> 6) - 1;
    const uint64_t wv = (uint64_t)blockIdx.x * kWaves + (uint64_t)wave_id();
    const uint64_t nwaves = (uint64_t)gridDim.x * kWaves;
    for (uint64_t b = wv; b < D.nb; b += nwaves) decode_bucket<RAGGED>(D, b, last_word);
}

}  // namespace qsgd
