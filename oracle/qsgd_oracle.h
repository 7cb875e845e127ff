/*
 * QSGD oracle: plain, slow, single-threaded CPU implementation of the QSGD
 * compressor. TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only users. The GPU library never links,
 * includes or calls anything in this directory, and this code shares nothing with
 * it.
 *
 * Sources (cited by page title and the part of the page):
 *  - "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding" (AIMech
 *    curated page), definition paragraph: the operator Q_s(v)_i =
 *    ||v||_2 * sgn(v_i) * xi_i(v,s), with l_i = floor(s|v_i|/||v||_2),
 *    p_i = s|v_i|/||v||_2 - l_i, xi_i = (l_i+1)/s with probability p_i and l_i/s
 *    otherwise; the encoded tuple (norm, signs, non-zero run-length gaps, levels
 *    k_i = s*xi_i) written with Elias recursive (omega) integer codes.
 *  - same page, claim "elias coding communication complexity tradeoff": the norm is
 *    sent as an F = 32 bit float; gaps and levels k_i in {1..s} use Elias codes.
 *  - same page, claim "QSVRG, non-convex and multi-GPU bucketed training"
 *    (Section 3.3 of the paper): Q_s is applied independently per bucket of d
 *    consecutive coordinates.
 *
 * The pages give real-valued mathematics only. Every step they leave open is
 * fixed as follows (each a reading, see the comments at the definitions):
 *  - norm:     RN32(sqrt(sum (double)v_i^2)), summed in index order in fp64.
 *  - ratio:    r_i = RN32(s |v_i| / norm_b), the fp32 value nearest to the exact
 *              quotient (ties to even).
 *  - rounding: l = floor(r), p = r - l, u = (w >> 8) * 2^-24 with w the
 *              Philox4x32-10 word (i & 3) of counter (i >> 2, key = seed),
 *              k = l + [u < p].
 *  - stream:   per bucket, the 32 bits of norm_b, then for each non-zero level in
 *              index order omega(gap) | sign (1 = negative) | omega(k); gap is the
 *              bucket-local 1-based distance to the previous non-zero; buckets
 *              are concatenated with no padding; stream bit t is bit 63 - (t mod 64)
 *              of 64-bit word t / 64; bucket b starts at offsets[b].
 *  - dequantization: m = RN32(norm_b k / s), the fp32 value nearest to the
 *              exact quotient (ties to even); value +-m, +0.0f where k = 0.
 */
#ifndef QSGD_ORACLE_H
#define QSGD_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { OR_OK = 0, OR_ERR_ARG = 1, OR_ERR_MALFORMED = 2, OR_ERR_CAPACITY = 3 };

/* Philox4x32-10 block function (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11). */
void or_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* The random 32-bit word that coordinate i draws: word (i & 3) of
 * Philox4x32-10 with key (lo32(seed), hi32(seed)) and counter
 * (lo32(i >> 2), hi32(i >> 2), 0, 0). */
uint32_t or_random_word(uint64_t seed, uint64_t i);
/* or_random_word for i = first .. first + count - 1. */
void or_random_words(uint64_t seed, uint64_t first, uint64_t count, uint32_t *out);

/* Elias omega code (P. Elias, "Universal codeword sets and representations of
 * the integers", IEEE Trans. Inf. Theory 21(2), 1975). N >= 1. */
unsigned or_omega_length(uint64_t N);
/* Writes the codeword of N as a NUL-terminated string of '0'/'1' into out (at
 * least 130 bytes); returns its length. */
unsigned or_omega_codeword(uint64_t N, char *out);

/* Elias gamma code (same paper): floor(log2 N) zeros, then N in binary, most
 * significant bit first; length 2 floor(log2 N) + 1. */
unsigned or_gamma_length(uint64_t N);
unsigned or_gamma_codeword(uint64_t N, char *out);

/* Bucket tables: bstart has nb + 1 entries; bucket b covers coordinates
 * [bstart[b], bstart[b+1]). Return nb. A NULL bstart only counts. */
uint64_t or_uniform_buckets(uint64_t n, uint64_t d, uint64_t *bstart);
uint64_t or_ragged_buckets(const uint64_t *seg_len, uint64_t nseg, uint64_t d,
                           uint64_t *bstart);

/* Bucket norms in fp64, index order. */
void or_bucket_norms(const float *v, const uint64_t *bstart, uint64_t nb, float *norms);
/* Bucket max-norms max|v_i| (the reading of the named variant QSGDinf; pass them
 * as given_norms to or_quantize). */
void or_bucket_max_norms(const float *v, const uint64_t *bstart, uint64_t nb, float *norms);

/* Stochastic quantization. If given_norms is non-NULL those norms are used in
 * place of the computed ones (to condition on another implementation's norms).
 * levels[i] = sgn(v_i) * k_i. norms_out (nb entries) receives the norms used. */
int or_quantize(const float *v, const uint64_t *bstart, uint64_t nb, uint32_t s,
                uint64_t seed, const float *given_norms, int32_t *levels,
                float *norms_out);

/* Same, with the 24-bit uniform integers u24[i] (u = u24 * 2^-24) supplied
 * instead of drawn from Philox. */
int or_quantize_u24(const float *v, const uint64_t *bstart, uint64_t nb, uint32_t s,
                    const uint32_t *u24, const float *given_norms, int32_t *levels,
                    float *norms_out);

/* Q_s(v) from levels and norms. */
void or_dequantize(const int32_t *levels, const float *norms, const uint64_t *bstart,
                   uint64_t nb, uint32_t s, float *out);

/* Encoding of the quantized tuple into one bitstream. offsets has nb + 1
 * entries. Fails with OR_ERR_CAPACITY if cap_words is too small. */
int or_encode(const int32_t *levels, const float *norms, const uint64_t *bstart,
              uint64_t nb, uint32_t s, uint64_t *words, uint64_t cap_words,
              uint64_t *offsets, uint64_t *out_bits);

/* or_encode with the integer code chosen: 0 = Elias omega, 1 = Elias gamma (the
 * page names "Elias recursive gamma/omega" coding). The stream layout is the
 * same; only the codewords of gaps and levels change. */
int or_encode_code(const int32_t *levels, const float *norms, const uint64_t *bstart,
                   uint64_t nb, uint32_t s, int code, uint64_t *words, uint64_t cap_words,
                   uint64_t *offsets, uint64_t *out_bits);

/* Decoding and dequantization. Returns OR_ERR_MALFORMED for a stream that does
 * not parse (gap past the bucket, level outside 1..s, record past the bucket's
 * end, offsets not monotone); out is then partially written. */
int or_decode(const uint64_t *words, uint64_t nwords, const uint64_t *offsets,
              const uint64_t *bstart, uint64_t nb, uint32_t s, float *out);
/* or_decode with the integer code chosen as in or_encode_code. */
int or_decode_code(const uint64_t *words, uint64_t nwords, const uint64_t *offsets,
                   const uint64_t *bstart, uint64_t nb, uint32_t s, int code, float *out);

/* Decode-accumulate of k streams: for j = 0..k-1 in turn, decode stream j
 * (words[j], nwords[j] words, offsets[j]) into scratch [bstart[nb]] and set
 * acc[i] = acc[i] + scratch[i] (one fp32 addition) for every coordinate.
 * Returns the first decode error (acc then holds the streams before it). */
int or_decode_accumulate(const uint64_t *const *words, const uint64_t *nwords,
                         const uint64_t *const *offsets, uint64_t k, const uint64_t *bstart,
                         uint64_t nb, uint32_t s, float *acc, float *scratch);
/* or_decode_accumulate for streams of the given record code (0 omega, 1 gamma). */
int or_decode_accumulate_code(const uint64_t *const *words, const uint64_t *nwords,
                              const uint64_t *const *offsets, uint64_t k, const uint64_t *bstart,
                              uint64_t nb, uint32_t s, int code, float *acc, float *scratch);

#ifdef __cplusplus
}
#endif
#endif
