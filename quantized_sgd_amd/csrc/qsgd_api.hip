// Host side of libqsgd.so: the C ABI declared in include/qsgd.h. Validates
// arguments, derives the tiling, and enqueues the gfx950 kernels on the caller's
// stream. No device memory is allocated here; the encoder's workspace lives in
// the tail of the caller's `out` buffer.
#include "qsgd.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <cstdint>

#include "qsgd_decode.h"
#include "qsgd_encode.h"

using namespace qsgd;

namespace {

constexpr uint32_t kMaxRuns = 4096;    // pass-1 workgroups at most (run totals in the workspace)
constexpr uint32_t kFinishChunk = 8;   // tiles per pass-2 workgroup

uint32_t host_omega_len(uint64_t N) {  // Elias omega codeword length
    uint32_t L = 1;
    while (N > 1) {
        uint32_t b = 0;
        for (uint64_t x = N; x; x >>= 1) ++b;
        L += b;
        N = b - 1;
    }
    return L;
}

uint32_t host_code_len(uint32_t code, uint64_t N) {  // codeword length of a record field
    if (code == QSGD_CODE_GAMMA) {
        uint32_t b = 0;
        for (uint64_t x = N; x; x >>= 1) ++b;
        return 2 * b - 1;
    }
    return host_omega_len(N);
}

// Buckets per tile: whole buckets whose coordinates fit 4096 slots after the
// tile start is rounded down to a multiple of 16 (no rounding when every bucket
// start is a multiple of 16).
uint32_t buckets_per_tile(uint32_t d, bool aligned_starts) {
    if (d == 0) return 0;
    const uint32_t room = aligned_starts ? (uint32_t)kTC : (uint32_t)(kTC - 15);
    return std::min<uint32_t>((uint32_t)kKMax, room / d);
}

struct EncodePlan {
    uint32_t K = 0;
    uint64_t ntiles = 0;
    uint64_t stream_words = 0;  // capacity reserved for the stream
    uint64_t ws_words = 0;      // workspace words after the stream
    uint32_t obuf_words = 0;    // words of a tile's bit string bound, + 1 (also its slot size)
    uint64_t slot_region_words = 0;
    bool table = false;         // record codes from the LDS table (s <= kTabS)
    size_t lds_bytes = 0;
};

EncodePlan make_plan(uint64_t n, uint64_t nb, uint32_t s, uint32_t d, bool aligned_starts,
                     uint32_t code = QSGD_CODE_OMEGA) {
    EncodePlan p;
    p.K = buckets_per_tile(d, aligned_starts);
    if (p.K == 0) return p;
    p.ntiles = (nb + p.K - 1) / p.K;
    const uint64_t Ls = host_code_len(code, s);
    // stream bound: 32 nb + n (2.5 + Ls) bits (both codes spend at most 1.5 g
    // bits on a gap g, so a bucket's gap codes take at most 1.5 times its
    // length), rounded up to words, plus one
    const uint64_t twice_bits = 64 * nb + n * (5 + 2 * Ls);
    p.stream_words = (twice_bits + 127) / 128 + 1;
    p.stream_words = (p.stream_words + 31) & ~(uint64_t)31;
    // a tile's bit string: the same bound for its K buckets and at most 4096
    // coordinates, plus one spare word (a two-word read at the string's end)
    const uint64_t tile_twice_bits = 64ull * p.K + (uint64_t)kTC * (5 + 2 * Ls);
    p.obuf_words = (uint32_t)((tile_twice_bits + 127) / 128 + 1);
    // workspace: one slot per tile, then the tiles' lengths (uint32, 16-byte
    // aligned when out is)
    p.slot_region_words = (p.ntiles * p.obuf_words + 1) & ~(uint64_t)1;
    p.ws_words = p.slot_region_words + (p.ntiles + 1) / 2 + kMaxRuns;
    p.table = s <= kTabS;
    p.lds_bytes = EncodeLayout(p.obuf_words, p.K).total;
    return p;
}

size_t quantize_lds_bytes(const EncodePlan &p) { return EncodeLayout(0, p.K).total; }

// Workgroups of a kernel that fit on the current device at once (cached per
// kernel, LDS size and device; safe to call from several host threads).
template <typename K>
uint32_t resident_blocks(K kernel, size_t lds, int block = kWG) {
    struct Entry { const void *k; size_t lds; int block; int dev; uint32_t blocks; };
    static std::mutex mu;
    static Entry cache[32];
    static int used = 0;
    int dev = 0;
    (void)hipGetDevice(&dev);
    {
        std::lock_guard<std::mutex> g(mu);
        for (int i = 0; i < used; ++i)
            if (cache[i].k == (const void *)kernel && cache[i].lds == lds && cache[i].block == block &&
                cache[i].dev == dev)
                return cache[i].blocks;
    }
    int cus = 0, per_cu = 0;
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, lds);
    const uint32_t blocks = (uint32_t)std::max(1, cus) * (uint32_t)std::max(1, per_cu);
    std::lock_guard<std::mutex> g(mu);
    if (used < 32) cache[used++] = Entry{(const void *)kernel, lds, block, dev, blocks};
    return blocks;
}

constexpr size_t kMaxLds = 64 * 1024;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

qsgd_status launch_status() {
    return hipGetLastError() == hipSuccess ? QSGD_OK : QSGD_ERR_LAUNCH;
}

qsgd_status check_common(const float *v, uint32_t s, uint32_t d) {
    if (s == 0 || s > (1u << 24) || d == 0) return QSGD_ERR_INVALID_ARG;
    if (v && !aligned16(v)) return QSGD_ERR_INVALID_ARG;
    return QSGD_OK;
}

// The fast path serves single vectors whose buckets are 2^m coordinates with
// 16 <= d <= 4096 and s within the record table; quantize and encode take the
// same path for the same arguments, so their norms agree bit for bit.
bool use_aligned(const uint64_t *bstart, uint32_t s, uint32_t d) {
    return bstart == nullptr && d >= 16 && d <= (uint32_t)kTC && (d & (d - 1)) == 0 && s <= kTabS;
}

uint32_t log2u(uint32_t d) { return 31u - (uint32_t)__builtin_clz(d); }

qsgd_status quantize_impl(const float *v, uint64_t n, const uint64_t *bstart, uint64_t nb,
                          uint32_t s, uint32_t d, uint64_t seed, int32_t *levels, float *norms,
                          hipStream_t stream, uint32_t norm = QSGD_NORM_L2) {
    qsgd_status st = check_common(v, s, d);
    if (st != QSGD_OK) return st;
    if (norm > QSGD_NORM_MAX) return QSGD_ERR_INVALID_ARG;
    if (n == 0) return QSGD_OK;
    if (!v || !levels || !norms || !aligned16(levels)) return QSGD_ERR_INVALID_ARG;
    const bool ragged = bstart != nullptr;
    EncodePlan p = make_plan(n, nb, s, d, !ragged && (d % 16 == 0));
    if (p.K == 0) return QSGD_ERR_UNSUPPORTED;
    QsgdParams P{};
    P.v = v; P.n = n; P.nb = nb; P.bstart = bstart; P.seed = seed; P.s = s; P.d = d;
    P.K = p.K; P.ntiles = (uint32_t)p.ntiles; P.levels = levels; P.norms = norms;
    P.obuf_words = 0;
    P.maxnorm = norm;
    if (use_aligned(bstart, s, d)) {
        hipLaunchKernelGGL(quantize_aligned_kernel, dim3((uint32_t)p.ntiles), dim3(kWG), 0, stream, P,
                           log2u(d));
        return launch_status();
    }
    const size_t lds = quantize_lds_bytes(p);
    if (ragged)
        hipLaunchKernelGGL(quantize_kernel<true>, dim3((uint32_t)p.ntiles), dim3(kWG), lds, stream, P);
    else
        hipLaunchKernelGGL(quantize_kernel<false>, dim3((uint32_t)p.ntiles), dim3(kWG), lds, stream, P);
    return launch_status();
}

qsgd_status encode_impl(const float *v, uint64_t n, const uint64_t *bstart, uint64_t nb, uint32_t s,
                        uint32_t d, uint64_t seed, uint64_t *out, uint64_t *out_bits,
                        uint64_t *offsets, hipStream_t stream, uint32_t code = QSGD_CODE_OMEGA,
                        uint32_t norm = QSGD_NORM_L2) {
    qsgd_status st = check_common(v, s, d);
    if (st != QSGD_OK) return st;
    if (code > QSGD_CODE_GAMMA || norm > QSGD_NORM_MAX) return QSGD_ERR_INVALID_ARG;
    if (!out_bits || !offsets) return QSGD_ERR_INVALID_ARG;
    if (n == 0 || nb == 0) {
        hipLaunchKernelGGL(encode_empty_kernel, dim3(1), dim3(64), 0, stream, out_bits, offsets);
        return launch_status();
    }
    if (!v || !out || !aligned16(out)) return QSGD_ERR_INVALID_ARG;
    const bool ragged = bstart != nullptr;
    EncodePlan p = make_plan(n, nb, s, d, !ragged && (d % 16 == 0), code);
    if (p.K == 0) return QSGD_ERR_UNSUPPORTED;
    if (p.lds_bytes > kMaxLds || p.ntiles >= (1ull << 32)) return QSGD_ERR_UNSUPPORTED;
    QsgdParams P{};
    P.v = v; P.n = n; P.nb = nb; P.bstart = bstart; P.seed = seed; P.s = s; P.d = d;
    P.K = p.K; P.ntiles = (uint32_t)p.ntiles;
    P.offsets = offsets;
    P.slots = out + p.stream_words;
    P.tile_bits = reinterpret_cast<uint32_t *>(P.slots + p.slot_region_words);
    P.run_bits = P.slots + p.slot_region_words + (p.ntiles + 1) / 2;
    P.obuf_words = p.obuf_words;
    P.code = code;
    P.maxnorm = norm;
    // pass 1 grid: at most the given number of workgroups (and kMaxRuns), each
    // taking a run of consecutive tiles
    auto runs_for = [&](uint32_t resident) {
        const uint64_t g = std::min<uint64_t>(std::min<uint64_t>(p.ntiles, resident), kMaxRuns);
        P.run = (uint32_t)(p.ntiles / g);
        P.rem = (uint32_t)(p.ntiles - (uint64_t)P.run * g);
        return (uint32_t)g;
    };
    // pass 1: every tile into its slot
    if (use_aligned(bstart, s, d)) {
        const size_t lds = aligned_encode_lds_bytes(p.obuf_words);
        // records packed per quarter of a thread when levels are large: mean level
        // about 0.8 s / sqrt(d) under the L2 norm, 0.8 s / max|z| (about s / 4)
        // under the max-norm; past about 2 a half's 8 records pass 64 bits
        const bool quarters = norm == QSGD_NORM_MAX ? s >= 8 : (uint64_t)s * s >= 6ull * d;
        // twice the resident workgroups: the second half starts as workgroups of
        // the first finish, which evens out the end of the pass (per encode, c3:
        // 115.7 -> 109.2 us, c2: 54.9 -> 54.0, c4: 455 -> 442; on c3 1.5 times is
        // slower than once, 2.5 and 4 times a little slower than twice)
        auto launch = [&](auto kernel) {
            const uint32_t blocks = runs_for(2 * resident_blocks(kernel, lds));
            hipLaunchKernelGGL(kernel, dim3(blocks), dim3(kWG), lds, stream, P, log2u(d));
        };
        if (quarters) launch(encode_aligned_kernel<true>);
        else launch(encode_aligned_kernel<false>);
    } else {
        // twice the resident workgroups too (c5: 221 -> 211 us per encode)
        auto launch = [&](auto kernel) {
            const uint32_t blocks = runs_for(2 * resident_blocks(kernel, p.lds_bytes));
            hipLaunchKernelGGL(kernel, dim3(blocks), dim3(kWG), p.lds_bytes, stream, P);
        };
        if (ragged) {
            if (p.table) launch(encode_kernel<true, true>); else launch(encode_kernel<true, false>);
        } else {
            if (p.table) launch(encode_kernel<false, true>); else launch(encode_kernel<false, false>);
        }
    }
    if (hipGetLastError() != hipSuccess) return QSGD_ERR_LAUNCH;
    // pass 2: tile offsets, the stream words, absolute bucket offsets
    FinishParams F{};
    F.out = out; F.slots = P.slots; F.tile_bits = P.tile_bits; F.offsets = offsets;
    F.run_bits = P.run_bits; F.run = P.run; F.rem = P.rem;
    F.out_bits = out_bits; F.nb = nb; F.ntiles = (uint32_t)p.ntiles; F.slot_words = p.obuf_words;
    F.K = p.K;
    F.chunk = kFinishChunk;
    const uint32_t fgrid = (uint32_t)((p.ntiles + F.chunk - 1) / F.chunk);
    hipLaunchKernelGGL(encode_finish_kernel, dim3(fgrid), dim3(kWG), 0, stream, F);
    return launch_status();
}

// Decodes one stream into v_hat, or (acc) adds the decodes of the nstreams
// streams in[k] / offsets[k] to v_hat in stream order.
qsgd_status decode_impl(const uint64_t *const *in, const uint64_t *const *offsets, uint32_t nstreams,
                        bool acc, uint64_t n, const uint64_t *bstart, uint64_t nb, uint32_t s,
                        uint32_t d, float *v_hat, hipStream_t stream, uint32_t code = QSGD_CODE_OMEGA) {
    qsgd_status st = check_common(nullptr, s, d);
    if (st != QSGD_OK) return st;
    if (code > QSGD_CODE_GAMMA) return QSGD_ERR_INVALID_ARG;
    if (nstreams > kMaxStreams || (nstreams && (!in || !offsets))) return QSGD_ERR_INVALID_ARG;
    if (n == 0 || nb == 0 || nstreams == 0) return QSGD_OK;
    for (uint32_t k = 0; k < nstreams; ++k)
        if (!in[k] || !offsets[k]) return QSGD_ERR_INVALID_ARG;
    if (!v_hat || !aligned16(v_hat)) return QSGD_ERR_INVALID_ARG;
    if (d > (1u << 24)) return QSGD_ERR_UNSUPPORTED;
    DecodeParams D{};
    for (uint32_t k = 0; k < nstreams; ++k) {
        D.in[k] = in[k];
        D.offsets[k] = offsets[k];
    }
    D.nstreams = nstreams;
    D.bstart = bstart; D.v_hat = v_hat;
    D.n = n; D.nb = nb; D.s = s; D.d = d;
    // LDS-staged output: whole groups of buckets of at most kGroupCoords
    // coordinates, levels fit int8. Team size: a power of two, about one lane per
    // 64 coordinates of a bucket, teams * buckets per group <= 64.
    const bool lds_out = s <= 127 && d <= (uint32_t)kGroupCoords;
    uint32_t tpw, team = 1;
    if (lds_out) {
        tpw = std::max<uint32_t>(1, std::min<uint32_t>(64, (uint32_t)kGroupCoords / d));
        while (team * 2 * tpw <= 64) team *= 2;
    } else {
        while (team < 64 && (uint64_t)team * 2 * 64 <= d) team *= 2;
        tpw = 64 / team;
    }
    D.team = team;
    D.tpw = tpw;
    D.lds_out = lds_out ? 1u : 0u;
    const uint64_t groups = (nb + tpw - 1) / tpw;
    const uint64_t want = (groups + kDecWaves - 1) / kDecWaves;
    const size_t lds = decode_lds_bytes();
    // the resident workgroups (twice as many: c3 119 -> 118.6 us, but c2 61.6 ->
    // 64.9 us, where that gives every group a workgroup of its own)
    auto launch = [&](auto kernel) {
        const uint32_t blocks = (uint32_t)std::min<uint64_t>(want, resident_blocks(kernel, lds, kDecWG));
        hipLaunchKernelGGL(kernel, dim3(blocks), dim3(kDecWG), lds, stream, D);
    };
    // accumulation is served for omega streams; the code is a kernel parameter so
    // that each kernel holds one record decoder
    if (acc) {
        if (code != QSGD_CODE_OMEGA) return QSGD_ERR_UNSUPPORTED;
        if (bstart) lds_out ? launch(decode_kernel<true, true, true, 0>) : launch(decode_kernel<true, false, true, 0>);
        else lds_out ? launch(decode_kernel<false, true, true, 0>) : launch(decode_kernel<false, false, true, 0>);
    } else if (code == QSGD_CODE_GAMMA) {
        if (bstart) lds_out ? launch(decode_kernel<true, true, false, 1>) : launch(decode_kernel<true, false, false, 1>);
        else lds_out ? launch(decode_kernel<false, true, false, 1>) : launch(decode_kernel<false, false, false, 1>);
    } else {
        if (bstart) lds_out ? launch(decode_kernel<true, true, false, 0>) : launch(decode_kernel<true, false, false, 0>);
        else lds_out ? launch(decode_kernel<false, true, false, 0>) : launch(decode_kernel<false, false, false, 0>);
    }
    return launch_status();
}

uint64_t ragged_count(const uint64_t *seg_len, uint32_t nseg, uint32_t d, uint64_t *table) {
    uint64_t nb = 0, base = 0;
    for (uint32_t t = 0; t < nseg; ++t) {
        const uint64_t end = base + seg_len[t];
        for (uint64_t pos = base; pos < end; pos = (end - pos > d) ? pos + d : end) {
            if (table) table[nb] = pos;
            ++nb;
        }
        base = end;
    }
    if (table) table[nb] = base;
    return nb;
}

}  // namespace

extern "C" {

const char *qsgd_status_string(qsgd_status status) {
    switch (status) {
        case QSGD_OK: return "QSGD_OK";
        case QSGD_ERR_INVALID_ARG: return "QSGD_ERR_INVALID_ARG";
        case QSGD_ERR_LAUNCH: return "QSGD_ERR_LAUNCH";
        case QSGD_ERR_UNSUPPORTED: return "QSGD_ERR_UNSUPPORTED";
    }
    return "QSGD_UNKNOWN_STATUS";
}

uint64_t qsgd_num_buckets(uint64_t n, uint32_t d) { return d ? (n + d - 1) / d : 0; }

uint32_t qsgd_max_bucket(void) { return (uint32_t)kTC; }

uint64_t qsgd_encode_capacity_words(uint64_t n, uint32_t s, uint32_t d) {
    if (d == 0 || s == 0) return 0;
    const uint64_t nb = qsgd_num_buckets(n, d);
    if (nb == 0) return 1;
    EncodePlan p = make_plan(n, nb, s, d, d % 16 == 0);
    if (p.K == 0) return 0;
    return p.stream_words + p.ws_words;
}

uint64_t qsgd_encode_capacity_words_ragged(uint64_t n, uint64_t nb, uint32_t s, uint32_t d) {
    if (d == 0 || s == 0) return 0;
    if (nb == 0) return 1;
    EncodePlan p = make_plan(n, nb, s, d, false);
    if (p.K == 0) return 0;
    return p.stream_words + p.ws_words;
}

qsgd_status qsgd_quantize(const float *v, uint64_t n, uint32_t s, uint32_t d, uint64_t seed,
                          int32_t *levels, float *norms, hipStream_t stream) {
    return quantize_impl(v, n, nullptr, qsgd_num_buckets(n, d), s, d, seed, levels, norms, stream);
}

qsgd_status qsgd_encode(const float *v, uint64_t n, uint32_t s, uint32_t d, uint64_t seed,
                        uint64_t *out, uint64_t *out_bits, uint64_t *bucket_bit_offsets,
                        hipStream_t stream) {
    return encode_impl(v, n, nullptr, qsgd_num_buckets(n, d), s, d, seed, out, out_bits,
                       bucket_bit_offsets, stream);
}

qsgd_status qsgd_decode(const uint64_t *in, const uint64_t *bucket_bit_offsets, uint64_t n,
                        uint32_t s, uint32_t d, float *v_hat, hipStream_t stream) {
    return decode_impl(&in, &bucket_bit_offsets, 1, false, n, nullptr, qsgd_num_buckets(n, d), s, d,
                       v_hat, stream);
}

uint32_t qsgd_max_streams(void) { return kMaxStreams; }

uint64_t qsgd_encode_capacity_words_ex(uint64_t n, uint64_t nb, uint32_t s, uint32_t d, qsgd_code code) {
    if (d == 0 || s == 0 || (uint32_t)code > QSGD_CODE_GAMMA) return 0;
    if (nb == 0) return 1;
    // the larger of the two tilings (bucket starts on multiples of 16 or not;
    // buckets of more than 4081 coordinates only tile with aligned starts)
    EncodePlan a = make_plan(n, nb, s, d, true, code), b = make_plan(n, nb, s, d, false, code);
    const uint64_t ca = a.K ? a.stream_words + a.ws_words : 0, cb = b.K ? b.stream_words + b.ws_words : 0;
    return std::max(ca, cb);
}

qsgd_status qsgd_quantize_ex(const float *v, uint64_t n, const uint64_t *bucket_start, uint64_t nb,
                             uint32_t s, uint32_t d, uint64_t seed, qsgd_norm norm, int32_t *levels,
                             float *norms, hipStream_t stream) {
    if (!bucket_start && nb != qsgd_num_buckets(n, d)) return QSGD_ERR_INVALID_ARG;
    if (bucket_start && nb == 0 && n != 0) return QSGD_ERR_INVALID_ARG;
    return quantize_impl(v, n, bucket_start, nb, s, d, seed, levels, norms, stream, (uint32_t)norm);
}

qsgd_status qsgd_encode_ex(const float *v, uint64_t n, const uint64_t *bucket_start, uint64_t nb,
                           uint32_t s, uint32_t d, uint64_t seed, qsgd_code code, qsgd_norm norm,
                           uint64_t *out, uint64_t *out_bits, uint64_t *bucket_bit_offsets,
                           hipStream_t stream) {
    if (!bucket_start && nb != qsgd_num_buckets(n, d)) return QSGD_ERR_INVALID_ARG;
    if (bucket_start && nb == 0 && n != 0) return QSGD_ERR_INVALID_ARG;
    return encode_impl(v, n, bucket_start, nb, s, d, seed, out, out_bits, bucket_bit_offsets, stream,
                       (uint32_t)code, (uint32_t)norm);
}

qsgd_status qsgd_decode_ex(const uint64_t *in, const uint64_t *bucket_bit_offsets, uint64_t n,
                           const uint64_t *bucket_start, uint64_t nb, uint32_t s, uint32_t d,
                           qsgd_code code, float *v_hat, hipStream_t stream) {
    if (!bucket_start && nb != qsgd_num_buckets(n, d)) return QSGD_ERR_INVALID_ARG;
    return decode_impl(&in, &bucket_bit_offsets, 1, false, n, bucket_start, nb, s, d, v_hat, stream,
                       (uint32_t)code);
}

qsgd_status qsgd_decode_accumulate(const uint64_t *const *in, const uint64_t *const *bucket_bit_offsets,
                                   uint32_t k, uint64_t n, uint32_t s, uint32_t d, float *acc,
                                   hipStream_t stream) {
    return decode_impl(in, bucket_bit_offsets, k, true, n, nullptr, qsgd_num_buckets(n, d), s, d, acc,
                       stream);
}

uint64_t qsgd_num_buckets_ragged(const uint64_t *seg_len, uint32_t nseg, uint32_t d) {
    if (d == 0 || (!seg_len && nseg)) return 0;
    return ragged_count(seg_len, nseg, d, nullptr);
}

qsgd_status qsgd_ragged_bucket_table(const uint64_t *seg_len, uint32_t nseg, uint32_t d,
                                     uint64_t *bucket_start, uint64_t nb) {
    if (d == 0 || (!seg_len && nseg) || !bucket_start) return QSGD_ERR_INVALID_ARG;
    if (ragged_count(seg_len, nseg, d, nullptr) != nb) return QSGD_ERR_INVALID_ARG;
    ragged_count(seg_len, nseg, d, bucket_start);
    return QSGD_OK;
}

qsgd_status qsgd_quantize_ragged(const float *v, uint64_t n, const uint64_t *bucket_start,
                                 uint64_t nb, uint32_t s, uint32_t d, uint64_t seed,
                                 int32_t *levels, float *norms, hipStream_t stream) {
    if (!bucket_start && nb) return QSGD_ERR_INVALID_ARG;
    if (nb == 0) return n == 0 ? QSGD_OK : QSGD_ERR_INVALID_ARG;
    return quantize_impl(v, n, bucket_start, nb, s, d, seed, levels, norms, stream);
}

qsgd_status qsgd_encode_ragged(const float *v, uint64_t n, const uint64_t *bucket_start,
                               uint64_t nb, uint32_t s, uint32_t d, uint64_t seed,
                               uint64_t *out, uint64_t *out_bits, uint64_t *bucket_bit_offsets,
                               hipStream_t stream) {
    if (!bucket_start && nb) return QSGD_ERR_INVALID_ARG;
    return encode_impl(v, n, bucket_start, nb, s, d, seed, out, out_bits, bucket_bit_offsets, stream);
}

qsgd_status qsgd_decode_ragged(const uint64_t *in, const uint64_t *bucket_bit_offsets, uint64_t n,
                               const uint64_t *bucket_start, uint64_t nb, uint32_t s, uint32_t d,
                               float *v_hat, hipStream_t stream) {
    if (!bucket_start && nb) return QSGD_ERR_INVALID_ARG;
    return decode_impl(&in, &bucket_bit_offsets, 1, false, n, bucket_start, nb, s, d, v_hat, stream);
}

qsgd_status qsgd_decode_accumulate_ragged(const uint64_t *const *in,
                                          const uint64_t *const *bucket_bit_offsets, uint32_t k,
                                          uint64_t n, const uint64_t *bucket_start, uint64_t nb,
                                          uint32_t s, uint32_t d, float *acc, hipStream_t stream) {
    if (!bucket_start && nb) return QSGD_ERR_INVALID_ARG;
    return decode_impl(in, bucket_bit_offsets, k, true, n, bucket_start, nb, s, d, acc, stream);
}

}  // extern "C"
