/* Drives the oracle through quantize, encode, decode, decode-accumulate and the
 * code helpers on seeded inputs, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py). Exits non-zero on a
 * failed check; the sanitizers abort on any memory or undefined-behaviour error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qsgd_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform01(void) { /* xorshift64*: input generation only */
    rng_state ^= rng_state >> 12; rng_state ^= rng_state << 25; rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) * 0x1p-53;
}

static int run_case(uint64_t n, uint64_t d, uint32_t s, int code, int maxnorm) {
    float *v = malloc(n * sizeof(float));
    for (uint64_t i = 0; i < n; ++i) {
        double u = uniform01();
        v[i] = u < 0.2 ? 0.0f : (float)((uniform01() - 0.5) * pow(10.0, 6.0 * u - 3.0));
    }
    uint64_t nb = or_uniform_buckets(n, d, NULL);
    uint64_t *bst = malloc((nb + 1) * sizeof(uint64_t));
    or_uniform_buckets(n, d, bst);
    float *norms = malloc((nb ? nb : 1) * sizeof(float));
    if (maxnorm) or_bucket_max_norms(v, bst, nb, norms); else or_bucket_norms(v, bst, nb, norms);
    int32_t *lev = malloc((n ? n : 1) * sizeof(int32_t));
    if (or_quantize(v, bst, nb, s, 7, norms, lev, NULL) != OR_OK) return 1;
    uint64_t cap = 64 + (nb * 32 + n * 80) / 64;
    uint64_t *words = malloc(cap * sizeof(uint64_t));
    uint64_t *offs = malloc((nb + 1) * sizeof(uint64_t));
    uint64_t bits = 0;
    if (or_encode_code(lev, norms, bst, nb, s, code, words, cap, offs, &bits) != OR_OK) return 2;
    float *out = malloc((n ? n : 1) * sizeof(float)), *want = malloc((n ? n : 1) * sizeof(float));
    if (or_decode_code(words, (bits + 63) / 64, offs, bst, nb, s, code, out) != OR_OK) return 3;
    or_dequantize(lev, norms, bst, nb, s, want);
    if (n && memcmp(out, want, n * sizeof(float)) != 0) return 4;
    float *acc = calloc(n ? n : 1, sizeof(float)), *scratch = malloc((n ? n : 1) * sizeof(float));
    const uint64_t *wl[2] = {words, words};
    const uint64_t nw[2] = {(bits + 63) / 64, (bits + 63) / 64};
    const uint64_t *ol[2] = {offs, offs};
    if (or_decode_accumulate_code(wl, nw, ol, 2, bst, nb, s, code, acc, scratch) != OR_OK) return 5;
    /* a truncated stream is reported, never read past its end */
    if (nb && bits > 40) {
        offs[nb] = bits + 64 * 4;
        if (or_decode_code(words, (bits + 63) / 64, offs, bst, nb, s, code, out) != OR_ERR_MALFORMED) return 6;
    }
    char cw[160];
    for (uint64_t N = 1; N < 5000; N += 37) {
        if (or_omega_codeword(N, cw) != or_omega_length(N)) return 7;
        if (or_gamma_codeword(N, cw) != or_gamma_length(N)) return 8;
    }
    free(v); free(bst); free(norms); free(lev); free(words); free(offs); free(out); free(want);
    free(acc); free(scratch);
    return 0;
}

int main(void) {
    const struct { uint64_t n, d; uint32_t s; int code, maxnorm; } cases[] = {
        {0, 4, 4, 0, 0}, {1, 1, 1, 0, 0}, {4096, 4096, 64, 0, 0}, {10007, 37, 3, 1, 0},
        {20000, 512, 16, 0, 1}, {5000, 1, 1u << 24, 1, 0}, {3000, 5000, 100, 0, 0}};
    for (unsigned i = 0; i < sizeof cases / sizeof cases[0]; ++i) {
        int rc = run_case(cases[i].n, cases[i].d, cases[i].s, cases[i].code, cases[i].maxnorm);
        if (rc) { printf("case %u failed: %d\n", i, rc); return 1; }
    }
    uint64_t seg[5] = {5, 0, 3, 8, 9}, bst[16];
    if (or_ragged_buckets(seg, 5, 4, bst) != 8) return 1;
    printf("oracle sanitizer driver ok\n");
    return 0;
}
