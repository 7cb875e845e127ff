/*
 * QSGD oracle implementation. TEST INFRASTRUCTURE ONLY (see qsgd_oracle.h): a
 * plain, slow, single-threaded statement of what the compressor computes, used
 * to check the GPU library. Compiled with -ffp-contract=off so that every
 * floating-point expression below is evaluated as written, one IEEE operation
 * at a time (round to nearest even).
 *
 * Parity status of each function (what pins it; the pins live in tests/):
 *  - or_philox4x32_10 / or_random_word: pinned to PyTorch's independent host
 *    Philox engine (ATen/core/PhiloxRNGEngine.h) on many (seed, index) pairs.
 *  - or_omega_length / or_omega_codeword: pinned to textbook codewords of the
 *    Elias omega code (tests/golden/elias_omega_codewords.txt), Kraft sum and
 *    prefix-freeness.
 *  - or_quantize / or_quantize_u24 / or_dequantize: pinned by exhaustive
 *    enumeration of all 2^n rounding outcomes (unbiasedness and the variance
 *    identity of Lemma 3.1), the support bound, the d = 1 identity, and
 *    hand-derived special cases.
 *  - or_encode / or_decode: pinned by hand-derived streams
 *    (tests/golden/special_streams.json), exact expected bit counts against
 *    Monte Carlo, and the round-trip identity.
 */
#include "qsgd_oracle.h"

#include <math.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11, Section 3): a 10-round bijection of a
 * 128-bit counter under a 64-bit key. Each round multiplies counter words 0
 * and 2 by the two round multipliers, and mixes the high halves of the products
 * with the other two words and the round key. The round key starts as the key
 * and is bumped by the two Weyl constants after every round. */
#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void or_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t prod0 = (uint64_t)PHILOX_M0 * (uint64_t)x0;
        uint64_t prod1 = (uint64_t)PHILOX_M1 * (uint64_t)x2;
        uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
        uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
        uint32_t y0 = hi1 ^ x1 ^ k0;
        uint32_t y1 = lo1;
        uint32_t y2 = hi0 ^ x3 ^ k1;
        uint32_t y3 = lo0;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
        k0 += PHILOX_W0;
        k1 += PHILOX_W1;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

uint32_t or_random_word(uint64_t seed, uint64_t i) {
    uint64_t block = i >> 2;
    uint32_t ctr[4] = {(uint32_t)block, (uint32_t)(block >> 32), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    or_philox4x32_10(ctr, key, out);
    return out[i & 3];
}

void or_random_words(uint64_t seed, uint64_t first, uint64_t count, uint32_t *out) {
    for (uint64_t t = 0; t < count; ++t) out[t] = or_random_word(seed, first + t);
}

/* ------------------------------------------------------------------------ */
/* Elias omega code, from its recursive definition: start from the single bit
 * "0"; while N > 1, put the binary representation of N in front and continue
 * with N = (number of bits of that representation) - 1. */
static unsigned bit_count(uint64_t x) { /* number of binary digits, x >= 1 */
    unsigned c = 0;
    while (x) { ++c; x >>= 1; }
    return c;
}

unsigned or_omega_codeword(uint64_t N, char *out) {
    char rev[160]; /* built from the end backwards */
    unsigned len = 0;
    rev[len++] = '0';
    while (N > 1) {
        unsigned nb = bit_count(N);
        for (unsigned b = 0; b < nb; ++b) /* least significant bit first */
            rev[len++] = (char)('0' + ((N >> b) & 1u));
        N = nb - 1;
    }
    for (unsigned t = 0; t < len; ++t) out[t] = rev[len - 1 - t];
    out[len] = '\0';
    return len;
}

unsigned or_omega_length(uint64_t N) {
    unsigned len = 1;
    while (N > 1) {
        unsigned nb = bit_count(N);
        len += nb;
        N = nb - 1;
    }
    return len;
}

/* Elias gamma code (same paper as omega): floor(log2 N) zeros, then the binary
 * form of N, most significant bit first. The page names "Elias recursive
 * gamma/omega" coding for the gaps and levels. */
unsigned or_gamma_codeword(uint64_t N, char *out) {
    unsigned nb = bit_count(N), len = 0;
    for (unsigned z = 1; z < nb; ++z) out[len++] = '0';
    for (unsigned b = nb; b-- > 0;) out[len++] = (char)('0' + ((N >> b) & 1u));
    out[len] = '\0';
    return len;
}

unsigned or_gamma_length(uint64_t N) { return 2 * bit_count(N) - 1; }

/* ------------------------------------------------------------------------ */
/* Buckets: Section 3.3 of the paper (per the claims on the curated page) applies
 * the quantizer independently to blocks of d consecutive coordinates; the last
 * block of a vector (or of each tensor in a ragged batch) may be shorter. */
uint64_t or_uniform_buckets(uint64_t n, uint64_t d, uint64_t *bstart) {
    if (d == 0) return 0;
    uint64_t nb = 0, pos = 0;
    while (pos < n) {
        if (bstart) bstart[nb] = pos;
        ++nb;
        pos = (n - pos > d) ? pos + d : n;
    }
    if (bstart) bstart[nb] = n;
    return nb;
}

uint64_t or_ragged_buckets(const uint64_t *seg_len, uint64_t nseg, uint64_t d,
                           uint64_t *bstart) {
    if (d == 0) return 0;
    uint64_t nb = 0, base = 0;
    for (uint64_t t = 0; t < nseg; ++t) {
        uint64_t end = base + seg_len[t], pos = base;
        while (pos < end) {
            if (bstart) bstart[nb] = pos;
            ++nb;
            pos = (end - pos > d) ? pos + d : end;
        }
        base = end;
    }
    if (bstart) bstart[nb] = base;
    return nb;
}

/* ------------------------------------------------------------------------ */
/* ||v||_2 of one bucket: fp32 squares are exact in fp64; they are summed in
 * index order in fp64, the square root is taken in fp64 and rounded once to the
 * 32-bit float that the stream carries (F = 32). */
static float bucket_norm(const float *v, uint64_t lo, uint64_t hi) {
    double acc = 0.0;
    for (uint64_t i = lo; i < hi; ++i) {
        double x = (double)v[i];
        acc = acc + x * x;
    }
    return (float)sqrt(acc);
}

void or_bucket_norms(const float *v, const uint64_t *bstart, uint64_t nb, float *norms) {
    for (uint64_t b = 0; b < nb; ++b) norms[b] = bucket_norm(v, bstart[b], bstart[b + 1]);
}

/* max_i |v_i| of each bucket: the scale of the reading of the heuristic
 * variant that page "NUQSGD: Provably Communication-efficient Data-parallel SGD
 * via Nonuniform Quantization" (abstract) names QSGDinf -- the infinity norm in
 * place of ||v||_2. Exact (a value of the input). Quantizing with these norms
 * given (or_quantize's given_norms) is that variant. */
void or_bucket_max_norms(const float *v, const uint64_t *bstart, uint64_t nb, float *norms) {
    for (uint64_t b = 0; b < nb; ++b) {
        float m = 0.0f;
        for (uint64_t i = bstart[b]; i < bstart[b + 1]; ++i) {
            float a = fabsf(v[i]);
            if (a > m) m = a;
        }
        norms[b] = m;
    }
}

/* Q_s on one coordinate, in the page's order: l = floor(s|v|/||v||),
 * p = s|v|/||v|| - l, round up to l + 1 with probability p. The ratio is the
 * binary32 value nearest to the exact quotient s|v|/||v|| (ties to even): s|v| is
 * exact in fp64 (at most 24 + 24 significant bits), the fp64 quotient is
 * correctly rounded, and rounding that to fp32 gives the correctly rounded
 * fp32 quotient, because an fp32 rounding boundary is either hit exactly (then
 * the fp64 quotient is exact too) or lies more than 2^-49 relative away. The
 * uniform is u = u24 * 2^-24 and the coordinate rounds up iff u < p. Returns k. */
static uint32_t level_of(float v, float norm, uint32_t s, uint32_t u24) {
    float a = fabsf(v);
    float r = (float)(((double)s * (double)a) / (double)norm);
    float l = floorf(r);
    float p = r - l; /* exact: l <= r < l + 1 */
    float u = (float)u24 * 0x1p-24f;
    uint32_t k = (uint32_t)l;
    if (u < p) k += 1u;
    return k;
}

static int quantize_impl(const float *v, const uint64_t *bstart, uint64_t nb, uint32_t s,
                         uint64_t seed, const uint32_t *u24, const float *given_norms,
                         int32_t *levels, float *norms_out) {
    if (s == 0 || s > (1u << 24)) return OR_ERR_ARG;
    for (uint64_t b = 0; b < nb; ++b) {
        uint64_t lo = bstart[b], hi = bstart[b + 1];
        for (uint64_t i = lo; i < hi; ++i)
            if (!isfinite(v[i])) return OR_ERR_ARG;
        float norm = given_norms ? given_norms[b] : bucket_norm(v, lo, hi);
        if (!isfinite(norm) || norm < 0.0f) return OR_ERR_ARG;
        if (norms_out) norms_out[b] = norm;
        if (norm == 0.0f) { /* all-zero bucket: every level is 0 */
            for (uint64_t i = lo; i < hi; ++i) levels[i] = 0;
            continue;
        }
        for (uint64_t i = lo; i < hi; ++i) {
            uint32_t w24 = u24 ? u24[i] : (or_random_word(seed, i) >> 8);
            uint32_t k = level_of(v[i], norm, s, w24);
            if (k > s) return OR_ERR_ARG; /* only with a norm below max |v_i| */
            levels[i] = signbit(v[i]) ? -(int32_t)k : (int32_t)k;
        }
    }
    return OR_OK;
}

int or_quantize(const float *v, const uint64_t *bstart, uint64_t nb, uint32_t s,
                uint64_t seed, const float *given_norms, int32_t *levels,
                float *norms_out) {
    return quantize_impl(v, bstart, nb, s, seed, NULL, given_norms, levels, norms_out);
}

int or_quantize_u24(const float *v, const uint64_t *bstart, uint64_t nb, uint32_t s,
                    const uint32_t *u24, const float *given_norms, int32_t *levels,
                    float *norms_out) {
    return quantize_impl(v, bstart, nb, s, 0, u24, given_norms, levels, norms_out);
}

/* Q_s(v)_i = ||v|| * sgn(v_i) * k_i / s: the magnitude is the binary32 value
 * nearest to the exact ||v|| k / s (ties to even). norm * k is exact in fp64 (at
 * most 24 + 24 significant bits); the fp64 quotient and its rounding to fp32
 * give the correctly rounded result, as for the ratio in level_of. */
static float dequant_magnitude(float norm, uint32_t s, uint32_t k) {
    return (float)(((double)norm * (double)k) / (double)s);
}

void or_dequantize(const int32_t *levels, const float *norms, const uint64_t *bstart,
                   uint64_t nb, uint32_t s, float *out) {
    for (uint64_t b = 0; b < nb; ++b) {
        for (uint64_t i = bstart[b]; i < bstart[b + 1]; ++i) {
            int32_t q = levels[i];
            if (q == 0) { out[i] = 0.0f; continue; }
            uint32_t k = (uint32_t)(q < 0 ? -q : q);
            float m = dequant_magnitude(norms[b], s, k);
            out[i] = q < 0 ? -m : m;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Bit writer / reader: stream bit t is bit 63 - (t mod 64) of word t / 64. */
typedef struct { uint64_t *w; uint64_t cap_bits; uint64_t pos; int overflow; } bitwriter;

static void put_bit(bitwriter *bw, unsigned bit) {
    if (bw->pos >= bw->cap_bits) { bw->overflow = 1; return; }
    if (bit) bw->w[bw->pos >> 6] |= (uint64_t)1 << (63 - (bw->pos & 63));
    bw->pos++;
}

/* The integer code of a record field: omega (code 0) or gamma (code 1). */
static void put_code(bitwriter *bw, uint64_t N, int code) {
    char cw[160];
    unsigned len = code ? or_gamma_codeword(N, cw) : or_omega_codeword(N, cw);
    for (unsigned t = 0; t < len; ++t) put_bit(bw, cw[t] == '1');
}

int or_encode(const int32_t *levels, const float *norms, const uint64_t *bstart,
              uint64_t nb, uint32_t s, uint64_t *words, uint64_t cap_words,
              uint64_t *offsets, uint64_t *out_bits) {
    return or_encode_code(levels, norms, bstart, nb, s, 0, words, cap_words, offsets, out_bits);
}

int or_encode_code(const int32_t *levels, const float *norms, const uint64_t *bstart,
                   uint64_t nb, uint32_t s, int code, uint64_t *words, uint64_t cap_words,
                   uint64_t *offsets, uint64_t *out_bits) {
    if (s == 0 || code < 0 || code > 1) return OR_ERR_ARG;
    bitwriter bw = {words, cap_words * 64, 0, 0};
    memset(words, 0, cap_words * sizeof(uint64_t));
    for (uint64_t b = 0; b < nb; ++b) {
        offsets[b] = bw.pos;
        /* the norm as its 32-bit binary32 pattern, most significant bit first */
        uint32_t nbits;
        memcpy(&nbits, &norms[b], sizeof nbits);
        for (int t = 31; t >= 0; --t) put_bit(&bw, (nbits >> t) & 1u);
        /* each non-zero: code(gap), sign, code(k); gaps are 1-based */
        int64_t prev = -1;
        for (uint64_t i = bstart[b]; i < bstart[b + 1]; ++i) {
            int32_t q = levels[i];
            if (q == 0) continue;
            int64_t j = (int64_t)(i - bstart[b]);
            uint32_t k = (uint32_t)(q < 0 ? -q : q);
            if (k > s) return OR_ERR_ARG;
            put_code(&bw, (uint64_t)(j - prev), code);
            put_bit(&bw, q < 0 ? 1u : 0u);
            put_code(&bw, k, code);
            prev = j;
        }
    }
    offsets[nb] = bw.pos;
    *out_bits = bw.pos;
    return bw.overflow ? OR_ERR_CAPACITY : OR_OK;
}

typedef struct { const uint64_t *w; uint64_t end; uint64_t pos; int bad; } bitreader;

static unsigned get_bit(bitreader *br) {
    if (br->pos >= br->end) { br->bad = 1; return 0; }
    unsigned bit = (unsigned)((br->w[br->pos >> 6] >> (63 - (br->pos & 63))) & 1u);
    br->pos++;
    return bit;
}

/* Omega decoding: N = 1; while the next bit is 1, that bit and the N bits after
 * it are the binary representation of the new N; a 0 bit ends the codeword. */
static uint64_t get_omega(bitreader *br) {
    uint64_t N = 1;
    while (!br->bad && get_bit(br)) {
        if (N > 63) { br->bad = 1; return 0; }
        uint64_t val = 1;
        for (uint64_t t = 0; t < N; ++t) val = (val << 1) | get_bit(br);
        N = val;
    }
    return N;
}

/* Gamma decoding: count the 0 bits before the first 1; that 1 and the same
 * number of bits after it are the binary form of N. */
static uint64_t get_gamma(bitreader *br) {
    unsigned z = 0;
    while (!br->bad && !get_bit(br)) {
        if (++z > 63) { br->bad = 1; return 0; }
    }
    uint64_t N = 1;
    for (unsigned t = 0; t < z; ++t) N = (N << 1) | get_bit(br);
    return N;
}

int or_decode(const uint64_t *words, uint64_t nwords, const uint64_t *offsets,
              const uint64_t *bstart, uint64_t nb, uint32_t s, float *out) {
    return or_decode_code(words, nwords, offsets, bstart, nb, s, 0, out);
}

int or_decode_code(const uint64_t *words, uint64_t nwords, const uint64_t *offsets,
                   const uint64_t *bstart, uint64_t nb, uint32_t s, int code, float *out) {
    if (s == 0 || code < 0 || code > 1) return OR_ERR_ARG;
    if (offsets[nb] > nwords * 64) return OR_ERR_MALFORMED;
    for (uint64_t b = 0; b < nb; ++b)
        if (offsets[b + 1] < offsets[b]) return OR_ERR_MALFORMED;
    for (uint64_t b = 0; b < nb; ++b) {
        uint64_t lo = bstart[b], len = bstart[b + 1] - bstart[b];
        for (uint64_t i = 0; i < len; ++i) out[lo + i] = 0.0f;
        bitreader br = {words, offsets[b + 1], offsets[b], 0};
        uint32_t nbits = 0;
        for (int t = 0; t < 32; ++t) nbits = (nbits << 1) | get_bit(&br);
        if (br.bad) return OR_ERR_MALFORMED;
        float norm;
        memcpy(&norm, &nbits, sizeof norm);
        int64_t j = -1;
        while (br.pos < br.end) {
            uint64_t gap = code ? get_gamma(&br) : get_omega(&br);
            unsigned neg = get_bit(&br);
            uint64_t k = code ? get_gamma(&br) : get_omega(&br);
            if (br.bad) return OR_ERR_MALFORMED;
            j += (int64_t)gap;
            if (j >= (int64_t)len || k < 1 || k > s) return OR_ERR_MALFORMED;
            float m = dequant_magnitude(norm, s, (uint32_t)k);
            out[lo + (uint64_t)j] = neg ? -m : m;
        }
    }
    return OR_OK;
}

/* Receiving side of a gradient exchange: each node sums the quantized gradients
 * it receives (page "QSGD: Communication-Efficient SGD via Gradient Quantization
 * and Encoding", abstract: nodes communicate quantized gradient updates). The
 * pages do not say how the sum is formed; reading: decode stream j, then add it
 * to acc coordinate by coordinate in fp32, for j = 0, 1, ..., k-1 in turn. */
int or_decode_accumulate(const uint64_t *const *words, const uint64_t *nwords,
                         const uint64_t *const *offsets, uint64_t k, const uint64_t *bstart,
                         uint64_t nb, uint32_t s, float *acc, float *scratch) {
    return or_decode_accumulate_code(words, nwords, offsets, k, bstart, nb, s, 0, acc, scratch);
}

/* The same with the record code of the streams (omega 0, gamma 1). */
int or_decode_accumulate_code(const uint64_t *const *words, const uint64_t *nwords,
                              const uint64_t *const *offsets, uint64_t k, const uint64_t *bstart,
                              uint64_t nb, uint32_t s, int code, float *acc, float *scratch) {
    const uint64_t n = bstart[nb];
    for (uint64_t j = 0; j < k; ++j) {
        int rc = or_decode_code(words[j], nwords[j], offsets[j], bstart, nb, s, code, scratch);
        if (rc != OR_OK) return rc;
        for (uint64_t i = 0; i < n; ++i) acc[i] = acc[i] + scratch[i];
    }
    return OR_OK;
}
