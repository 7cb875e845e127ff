/*
 * qsgd.h -- C ABI of the MI355X (gfx950) QSGD compressor library (libqsgd.so).
 *
 * The method (page "QSGD (Quantized Stochastic Gradient Descent) with Elias
 * Coding", definition paragraph): each bucket of d consecutive coordinates of an
 * fp32 gradient v is stochastically quantized to
 *     Q_s(v)_i = ||v||_2 * sgn(v_i) * k_i / s,   k_i in {0..s},
 * where l_i = floor(s|v_i|/||v||_2), p_i = s|v_i|/||v||_2 - l_i and k_i = l_i + 1
 * with probability p_i, else l_i. The tuple (norm, signs, gaps between non-zero
 * coordinates, levels k_i) is written losslessly with Elias omega codes (same
 * page, claim on Elias coding: F = 32 bit norm; bucketing per the claim on
 * bucketed training, paper Section 3.3).
 *
 * Exact semantics (the pages give real-valued math only; these are the readings
 * this library implements, bit for bit):
 *   norm_b   = RN32(sqrt(sum_{i in b} (double)v_i^2)) with an fp64 sum in a fixed
 *              (deterministic) order.
 *   r_i      = RN32(s |v_i| / norm_b), the binary32 value nearest to the exact
 *              quotient (ties to even);  l = floor(r);  p = r - l.
 *   uniform  = (w >> 8) * 2^-24 where w is word (i & 3) of Philox4x32-10
 *              (Salmon et al., SC'11) with key (lo32(seed), hi32(seed)) and
 *              counter (lo32(i >> 2), hi32(i >> 2), 0, 0); i is the flat index
 *              of the coordinate in v. k = l + [uniform < p].
 *   stream   = for each bucket: the 32-bit pattern of norm_b, then for each
 *              non-zero level in index order: omega(gap), 1 sign bit (1 =
 *              negative), omega(k). gap = j - j_prev with j_prev = -1 at the
 *              bucket start (bucket-local indices). Buckets are concatenated with
 *              no padding. Stream bit t is bit 63 - (t mod 64) of 64-bit word
 *              t / 64; unused bits of the last word are 0.
 *   decode   = v_hat_i = +-RN32(norm_b k / s), the binary32 value nearest to the
 *              exact quotient (minus for sign bit 1), +0.0f elsewhere.
 *   An all-zero bucket has norm 0 and no records.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers, allocated and owned by the caller,
 *     except the arguments documented as HOST arrays. The library allocates no
 *     device memory during a call and keeps no device state between calls; its
 *     one fixed scratch array (64 MiB per device, held from the library's first
 *     use on a device until the process ends) serves qsgd_encode_noalloc and the
 *     decode of uniform buckets longer than 16384 coordinates only.
 *   - Calls only enqueue work on `stream` (0 = the null stream) and return
 *     without synchronizing; results are valid once the stream reaches them.
 *   - Argument errors are detected on the host before anything is enqueued and
 *     reported as QSGD_ERR_INVALID_ARG; a failed kernel launch is
 *     QSGD_ERR_LAUNCH. Data-dependent problems (non-finite v, a malformed stream
 *     passed to decode) are not reported: the output is then unspecified, but no
 *     kernel reads or writes outside the buffers described here.
 *   - v must be 16-byte aligned. Outputs must not overlap inputs.
 *   - Calls on different streams may run concurrently as long as their buffers
 *     are disjoint.
 *   - Preconditions: 1 <= s <= 2^24, d >= 1, every v_i finite, every bucket norm
 *     finite in fp32.
 */
#ifndef QSGD_H
#define QSGD_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QSGD_OK = 0,
    QSGD_ERR_INVALID_ARG = 1,
    QSGD_ERR_LAUNCH = 2,
    QSGD_ERR_UNSUPPORTED = 3,
    QSGD_ERR_SCRATCH = 4      /* the call's records exceed the library's fixed scratch */
} qsgd_status;

/* Integer code of the record fields (gaps and levels). The page names "Elias
 * recursive gamma/omega" coding; omega is the default of every call without a
 * code argument. Elias gamma writes N as floor(log2 N) zero bits followed by N
 * in binary (2 floor(log2 N) + 1 bits); the stream layout is otherwise the same. */
typedef enum { QSGD_CODE_OMEGA = 0, QSGD_CODE_GAMMA = 1 } qsgd_code;

/* Scale of a bucket. QSGD_NORM_L2 is the page's ||v||_2 (the default of every
 * call without a norm argument). QSGD_NORM_MAX scales by max_i |v_i| instead:
 * the pages name a practical heuristic variant "QSGDinf" (page "NUQSGD: Provably
 * Communication-efficient Data-parallel SGD via Nonuniform Quantization",
 * abstract) without defining it; this library reads the name as the infinity
 * norm. The norm field of the stream then holds max|v_i| (exact), r_i =
 * RN32(s |v_i| / max|v|) and everything else is unchanged, so decode
 * needs no norm argument. The coordinates of largest magnitude get k = s. */
typedef enum { QSGD_NORM_L2 = 0, QSGD_NORM_MAX = 1 } qsgd_norm;

/* Human-readable name of a status code (static string). */
const char *qsgd_status_string(qsgd_status status);

/* ceil(n / d): the number of buckets of a single vector (0 if d == 0). */
uint64_t qsgd_num_buckets(uint64_t n, uint32_t d);

/* Largest bucket length of a ragged batch (4081 in this build: a tile of 4096
 * coordinates holds whole buckets starting anywhere); longer ragged buckets
 * return QSGD_ERR_UNSUPPORTED. Uniform buckets may have any length up to the
 * whole vector (d >= n is the single bucket of n coordinates). */
uint32_t qsgd_max_bucket(void);

/* Number of uint64 words the `out` buffer of qsgd_encode must hold for (n, s, d):
 * a worst-case stream bound, 32 nb + n (2.5 + |omega(s)|) bits (|omega(g)| <=
 * 1.5 g bounds the gap codes of a bucket by 1.5 times its length), followed by
 * the encoder's workspace: one slot per tile of at most 4096 coordinates, sized
 * by the same bound for the tile, and the tiles' bit counts (about as large
 * again as the stream bound). */
uint64_t qsgd_encode_capacity_words(uint64_t n, uint32_t s, uint32_t d);

/*
 * qsgd_quantize: Q_s per bucket (page "QSGD ... with Elias Coding", definition
 * paragraph), without encoding.
 *   v       [n] fp32 input.
 *   levels  [n] int32 output: sgn(v_i) * k_i (0 where k_i = 0).
 *   norms   [ceil(n/d)] fp32 output: norm_b.
 * n == 0 enqueues nothing.
 */
qsgd_status qsgd_quantize(const float *v, uint64_t n, uint32_t s, uint32_t d, uint64_t seed,
                          int32_t *levels, float *norms, hipStream_t stream);

/*
 * qsgd_encode: quantize and Elias-omega encode v into one bitstream (same page,
 * definition paragraph and claim on Elias coding), reading v once.
 *   out                 [qsgd_encode_capacity_words(n, s, d)] uint64 output,
 *                       16-byte aligned: the stream in words [0, ceil(out_bits/64));
 *                       the words after it are workspace and hold unspecified
 *                       values afterwards.
 *   out_bits            [1] uint64 output: stream length in bits.
 *   bucket_bit_offsets  [ceil(n/d) + 1] uint64 output: start bit of each bucket;
 *                       the last entry equals out_bits.
 * n == 0 writes out_bits = 0 and bucket_bit_offsets[0] = 0.
 */
qsgd_status qsgd_encode(const float *v, uint64_t n, uint32_t s, uint32_t d, uint64_t seed,
                        uint64_t *out, uint64_t *out_bits, uint64_t *bucket_bit_offsets,
                        hipStream_t stream);

/*
 * qsgd_decode: parse the stream and dequantize (the coding is lossless: same
 * page, definition paragraph).
 *   in                  stream words written by qsgd_encode (read-only).
 *   bucket_bit_offsets  [ceil(n/d) + 1] the offsets written by qsgd_encode.
 *   v_hat               [n] fp32 output, 16-byte aligned; every element is written
 *                       exactly once.
 * n, s, d must be those of the encode call. Uniform buckets of any length are
 * decoded; those longer than 16384 coordinates are cut into chunks of 16384
 * stream bits, one wave each, and need the library's fixed scratch (see
 * qsgd_encode_noalloc): such calls must not overlap in time on one device with
 * each other or with qsgd_encode_noalloc, and return QSGD_ERR_SCRATCH when
 * their chunk records exceed it (about 2 M chunks). A bucket's stream must be
 * shorter than 2^31 bits (checked against the bound of qsgd_encode_capacity_words;
 * QSGD_ERR_UNSUPPORTED otherwise). Buckets of a ragged table are decoded up to
 * 2^24 coordinates.
 */
qsgd_status qsgd_decode(const uint64_t *in, const uint64_t *bucket_bit_offsets, uint64_t n,
                        uint32_t s, uint32_t d, float *v_hat, hipStream_t stream);

/* ---- choice of code and norm (and of uniform or ragged buckets) in one call --
 * bucket_start is the DEVICE bucket table of a ragged batch, or NULL for
 * uniform buckets of d coordinates (then nb must be ceil(n/d)). Other arguments
 * as in qsgd_quantize / qsgd_encode / qsgd_decode; a stream must be decoded with
 * the code it was encoded with. An unknown code or norm is QSGD_ERR_INVALID_ARG. */

/* Capacity of `out` for qsgd_encode_ex (a bound for uniform and ragged layouts
 * alike); 0 for invalid arguments. */
uint64_t qsgd_encode_capacity_words_ex(uint64_t n, uint64_t nb, uint32_t s, uint32_t d,
                                       qsgd_code code);
qsgd_status qsgd_quantize_ex(const float *v, uint64_t n, const uint64_t *bucket_start, uint64_t nb,
                             uint32_t s, uint32_t d, uint64_t seed, qsgd_norm norm, int32_t *levels,
                             float *norms, hipStream_t stream);
qsgd_status qsgd_encode_ex(const float *v, uint64_t n, const uint64_t *bucket_start, uint64_t nb,
                           uint32_t s, uint32_t d, uint64_t seed, qsgd_code code, qsgd_norm norm,
                           uint64_t *out, uint64_t *out_bits, uint64_t *bucket_bit_offsets,
                           hipStream_t stream);
qsgd_status qsgd_decode_ex(const uint64_t *in, const uint64_t *bucket_bit_offsets, uint64_t n,
                           const uint64_t *bucket_start, uint64_t nb, uint32_t s, uint32_t d,
                           qsgd_code code, float *v_hat, hipStream_t stream);

/* ---- decode-accumulate: the receiving side of a gradient exchange ----------
 * In data-parallel SGD every node sends its quantized gradient and each
 * receiver sums the gradients it gets (page "QSGD: Communication-Efficient SGD
 * via Gradient Quantization and Encoding", abstract: nodes communicate
 * quantized gradient updates; page "QSGD (Quantized Stochastic Gradient Descent)
 * with Elias Coding", claim on multi-GPU bucketed training). The pages do not
 * fix how the sum is formed; this library's reading: for every coordinate i,
 *     acc_i <- (((acc_i + v_hat_0,i) + v_hat_1,i) + ... + v_hat_{k-1},i)
 * in fp32 (round to nearest even, one rounding per addition), in stream order,
 * where v_hat_j is what qsgd_decode returns for stream j (its +0.0f zeros
 * included, so an acc_i of -0.0f becomes +0.0f). Zero acc first for the plain sum.
 */

/* Largest number of streams one decode-accumulate call takes (32). */
uint32_t qsgd_max_streams(void);

/*
 * qsgd_decode_accumulate: adds the decodes of k streams to acc in one launch;
 * the decoded values never go to memory. For k <= 8 streams over uniform
 * buckets of 256 or more coordinates (a multiple of 4) with s <= 127, the waves
 * of a workgroup decode the k streams of a group side by side and add them to
 * acc together, reading and writing acc once per call; otherwise each wave
 * decodes the k streams of a group in turn and adds each to the group's part
 * of acc (acc read and written once per stream). The result is the same.
 *   in                  HOST array of k DEVICE pointers: stream words of each
 *                       stream, written by qsgd_encode with the same n, s, d.
 *   bucket_bit_offsets  HOST array of k DEVICE pointers: each stream's
 *                       [ceil(n/d) + 1] bucket offsets.
 *   k                   number of streams, 0..qsgd_max_streams() (0: nothing is
 *                       enqueued); more is QSGD_ERR_INVALID_ARG, as is a NULL
 *                       array or entry.
 *   acc                 [n] fp32 input and output, 16-byte aligned; must not
 *                       overlap any stream or offset table.
 * The pointer arrays are read during the call only.
 */
qsgd_status qsgd_decode_accumulate(const uint64_t *const *in, const uint64_t *const *bucket_bit_offsets,
                                   uint32_t k, uint64_t n, uint32_t s, uint32_t d, float *acc,
                                   hipStream_t stream);

/* qsgd_decode_accumulate for streams of either record code (all k streams of
 * the same code) and uniform (bucket_start NULL, nb = ceil(n/d)) or ragged
 * buckets; arguments otherwise as above and as in qsgd_decode_ex. */
qsgd_status qsgd_decode_accumulate_ex(const uint64_t *const *in, const uint64_t *const *bucket_bit_offsets,
                                      uint32_t k, uint64_t n, const uint64_t *bucket_start, uint64_t nb,
                                      uint32_t s, uint32_t d, qsgd_code code, float *acc, hipStream_t stream);

/* ---- ragged batches: several tensors in one flat buffer --------------------
 * Buckets restart at every tensor boundary (per-tensor quantization); the
 * Philox index of a coordinate is its flat index in the concatenation. The
 * bucket layout is a table bucket_start[nb + 1] (bucket b covers flat
 * coordinates [bucket_start[b], bucket_start[b+1]), every bucket at most d long),
 * built on the host by qsgd_ragged_bucket_table and copied to the device by the
 * caller. */

/* Number of buckets for host seg_len[nseg] (tensor lengths; zero-length tensors
 * have no buckets). */
uint64_t qsgd_num_buckets_ragged(const uint64_t *seg_len, uint32_t nseg, uint32_t d);

/* Fills the HOST array bucket_start[nb + 1] from HOST seg_len[nseg]; nb must be
 * qsgd_num_buckets_ragged(seg_len, nseg, d). */
qsgd_status qsgd_ragged_bucket_table(const uint64_t *seg_len, uint32_t nseg, uint32_t d,
                                     uint64_t *bucket_start, uint64_t nb);

/* Capacity of `out` for qsgd_encode_ragged with n coordinates and nb buckets. */
uint64_t qsgd_encode_capacity_words_ragged(uint64_t n, uint64_t nb, uint32_t s, uint32_t d);

/* Ragged variants of the three calls: bucket_start is the DEVICE copy of the
 * table; n = bucket_start[nb] (passed by value). Other arguments as above. */
qsgd_status qsgd_quantize_ragged(const float *v, uint64_t n, const uint64_t *bucket_start,
                                 uint64_t nb, uint32_t s, uint32_t d, uint64_t seed,
                                 int32_t *levels, float *norms, hipStream_t stream);
qsgd_status qsgd_encode_ragged(const float *v, uint64_t n, const uint64_t *bucket_start,
                               uint64_t nb, uint32_t s, uint32_t d, uint64_t seed,
                               uint64_t *out, uint64_t *out_bits,
                               uint64_t *bucket_bit_offsets, hipStream_t stream);
qsgd_status qsgd_decode_ragged(const uint64_t *in, const uint64_t *bucket_bit_offsets,
                               uint64_t n, const uint64_t *bucket_start, uint64_t nb,
                               uint32_t s, uint32_t d, float *v_hat, hipStream_t stream);
qsgd_status qsgd_decode_accumulate_ragged(const uint64_t *const *in,
                                          const uint64_t *const *bucket_bit_offsets, uint32_t k,
                                          uint64_t n, const uint64_t *bucket_start, uint64_t nb,
                                          uint32_t s, uint32_t d, float *acc, hipStream_t stream);

/* ---- ragged batches given by HOST tensor lengths ---------------------------
 * The same three calls with the layout given as HOST seg_len[nseg] (tensor
 * lengths, buckets of at most d restarting at every tensor, n = the sum of the
 * lengths, nb = qsgd_num_buckets_ragged(seg_len, nseg, d)) instead of a device
 * bucket table: the lengths travel in the kernel arguments, so these take at
 * most 160 tensors (more returns QSGD_ERR_UNSUPPORTED before anything is
 * enqueued; the table form has no such limit). Results are those of the table
 * form for the same layout; out needs qsgd_encode_capacity_words_ragged(n, nb, s,
 * d) words; seg_len is read during the call only. */
qsgd_status qsgd_quantize_seglen(const float *v, const uint64_t *seg_len, uint32_t nseg, uint32_t s,
                                 uint32_t d, uint64_t seed, int32_t *levels, float *norms, hipStream_t stream);
qsgd_status qsgd_encode_seglen(const float *v, const uint64_t *seg_len, uint32_t nseg, uint32_t s, uint32_t d,
                               uint64_t seed, uint64_t *out, uint64_t *out_bits, uint64_t *bucket_bit_offsets,
                               hipStream_t stream);
qsgd_status qsgd_decode_seglen(const uint64_t *in, const uint64_t *bucket_bit_offsets, const uint64_t *seg_len,
                               uint32_t nseg, uint32_t s, uint32_t d, float *v_hat, hipStream_t stream);

/* ---- encode without allocation ----------------------------------------------
 * For callers that cannot allocate device memory during the call (code under
 * HIP graph capture, tight loops, harnesses that forbid allocation): the same
 * computation as qsgd_encode, with the encoder's workspace (one bit-string slot
 * per tile of at most 4096 coordinates, the tiles' lengths and the pass-1 run
 * totals) in a fixed scratch array of 64 MiB inside the library instead of the
 * tail of `out`. Every device the library runs on holds its own copy of that
 * array until the process ends; its address is looked up on the first call on
 * a device. The call allocates nothing (no hipMalloc, no library allocation).
 * Nothing in the scratch needs clearing between calls: each call writes every
 * workspace word it reads. Calls that overlap in time on one device share the
 * scratch and race: serialize them (for instance on one stream). Decodes of
 * uniform buckets longer than 16384 coordinates use the same array.
 *
 * qsgd_encode_noalloc_capacity_words: the words `out` must hold, the stream
 * bound of qsgd_encode_capacity_words without the workspace; 0 when the
 * workspace of (n, s, d) exceeds the scratch or the arguments are invalid.
 * About 8 KB of scratch per tile at s = 64 (under 2 KB at s = 1): up to about
 * 34 M coordinates at s = 64, d = 4096, 39 M at s = 16, d = 512, and 149 M at
 * s = 1, d = 512.
 *
 * qsgd_encode_noalloc: arguments as qsgd_encode, with `out` holding
 * qsgd_encode_noalloc_capacity_words(n, s, d) words. Returns QSGD_ERR_SCRATCH,
 * enqueueing nothing, when the workspace exceeds the scratch; its results are
 * bit-identical to qsgd_encode's.
 */
uint64_t qsgd_encode_noalloc_capacity_words(uint64_t n, uint32_t s, uint32_t d);
qsgd_status qsgd_encode_noalloc(const float *v, uint64_t n, uint32_t s, uint32_t d, uint64_t seed,
                                uint64_t *out, uint64_t *out_bits, uint64_t *bucket_bit_offsets,
                                hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* QSGD_H */
