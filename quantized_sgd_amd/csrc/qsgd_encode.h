// Quantize kernel and the two-pass encode.
//
// Page "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding":
// definition paragraph (Q_s and the Elias-coded tuple of norm, signs, non-zero
// gaps and levels) and the claim on Elias coding (F = 32 bit norm).
//
// Encode pass 1, per tile (a run of whole buckets, <= 4096 coordinates, one
// workgroup; workgroup b takes the tiles [b run, (b + 1) run) in order, so no
// workgroup ever waits for another, and publishes their total length):
//   1. load v once from HBM, per-bucket norms, Philox rounding (qsgd_front.h);
//   2. each thread looks up the code of every coordinate's record -- the 32-bit
//      norm at a bucket start, and c(gap) | sign | c(k) per non-zero, c the
//      Elias omega code or (the page names "gamma/omega") the gamma code --
//      in a table of all records with gap <= 16 and k <= s (gaps inside one
//      thread's 16 coordinates never exceed 16) and sums their lengths. The gap
//      of a thread's first non-zero, when its origin lies in an earlier thread,
//      is resolved after an exclusive max-scan of "last marker" positions;
//   3. an exclusive sum-scan of per-thread bit counts gives each thread's offset
//      in the tile and the tile's length T;
//   4. every record is OR-ed into the tile's 64-bit words in LDS at its offset
//      from the tile's first bit; the words go to the tile's slot in the
//      workspace, T to tile_bits, and the bucket offsets (tile-relative) to the
//      offsets array.
// Encode pass 2 (encode_finish_kernel): tile offsets by prefix sums of the run
// totals and tile lengths, each stream word gathered from the slots of the
// tiles it covers (every word written once), bucket offsets made absolute.
#pragma once

#include "qsgd_front.h"

namespace qsgd {

// Record code table for s <= kTabS: entry (code << 5) | length of
// c(g) | sign | c(k) (c: the record fields' code; at most 23 bits) for g in
// [0, 16] (g = 0: no gap code) and k in [0, s] (k = 0: no record, entry 0).
// Index ((k * 17 + g) << 1) | sign.
constexpr uint32_t kTabS = 64;
constexpr uint32_t kTabG = 17;

__host__ __device__ constexpr uint32_t code_table_entries(uint32_t s) { return kTabG * (s + 1) * 2; }

__device__ __forceinline__ uint32_t code_index(uint32_t g, uint32_t k, uint32_t neg) {
    return ((((k << 4) + k) + g) << 1) | neg;
}

// The table for s = kTabS, computed at compile time for each code (the entries
// of k <= s serve any s <= kTabS); the encoders read it from constant memory
// through the vector L1 cache.
constexpr uint32_t ct_bitlen(uint32_t m) {
    uint32_t b = 0;
    while (m) {
        ++b;
        m >>= 1;
    }
    return b;
}

// Elias omega (CODE 0) or gamma (CODE 1) codeword of N >= 1, right-aligned.
template <int CODE>
constexpr uint64_t ct_field_code(uint32_t N, uint32_t &L) {
    if (CODE) {
        L = 2u * ct_bitlen(N) - 1u;
        return N;
    }
    uint64_t code = 0;
    L = 1;
    uint32_t m = N;
    while (m > 1u) {
        const uint32_t b = ct_bitlen(m);
        code |= (uint64_t)m << L;
        L += b;
        m = b - 1u;
    }
    return code;
}

struct alignas(16) CodeTable {
    uint32_t e[code_table_entries(kTabS)];
};

template <int CODE>
constexpr CodeTable make_code_table() {
    CodeTable t{};
    for (uint32_t i = 0; i < code_table_entries(kTabS); ++i) {
        const uint32_t neg = i & 1u;
        const uint32_t g = (i >> 1) % kTabG;
        const uint32_t k = (i >> 1) / kTabG;
        uint32_t e = 0;
        if (k) {
            uint32_t Lk = 0;
            const uint64_t kc = ct_field_code<CODE>(k, Lk);
            uint64_t code = ((uint64_t)neg << Lk) | kc;
            uint32_t len = Lk + 1;
            if (g) {
                uint32_t Lg = 0;
                const uint64_t gc = ct_field_code<CODE>(g, Lg);
                code |= gc << len;
                len += Lg;
            }
            e = ((uint32_t)code << 5) | len;
        }
        t.e[i] = e;
    }
    return t;
}

__constant__ CodeTable kCodeTableOmega = make_code_table<0>();
__constant__ CodeTable kCodeTableGamma = make_code_table<1>();

// OR a left-aligned bit string (len <= 64 bits at the top of `word`) into the
// LDS word window at bit position pos.
__device__ __forceinline__ void or_bits(uint64_t *buf, uint32_t pos, uint64_t word, uint32_t len) {
    const uint32_t idx = pos >> 6, sh = pos & 63u;
    atomicOr(reinterpret_cast<unsigned long long *>(buf + idx), (unsigned long long)(word >> sh));
    if (sh + len > 64u)
        atomicOr(reinterpret_cast<unsigned long long *>(buf + idx + 1),
                 (unsigned long long)(word << (64u - sh)));
}

struct EncodeLds {
    FrontLds f;
    uint64_t *obuf;
};

__host__ __device__ constexpr size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Dynamic LDS layout shared by host and device: [obuf][cb][segv][bs][nrm][segf].
struct EncodeLayout {
    size_t obuf, cb, segv, bs, nrm, segf, total;
    __host__ __device__ EncodeLayout(uint32_t obuf_words, uint32_t K) {
        size_t off = 0;
        obuf = off; off = align16(off + (size_t)obuf_words * 8);
        cb = off;   off = align16(off + (size_t)K * 8);
        segv = off; off = align16(off + kWaves * 8);
        bs = off;   off = align16(off + (size_t)(K + 1) * 4);
        nrm = off;  off = align16(off + (size_t)K * 4);
        segf = off; off = align16(off + kWaves * 4);
        total = off;
    }
};

__device__ __forceinline__ EncodeLds carve_encode_lds(unsigned char *smem, const QsgdParams &P) {
    const EncodeLayout lay(P.obuf_words, P.K);
    EncodeLds L;
    L.obuf = reinterpret_cast<uint64_t *>(smem + lay.obuf);
    L.f.cb = reinterpret_cast<double *>(smem + lay.cb);
    L.f.segv = reinterpret_cast<double *>(smem + lay.segv);
    L.f.bs = reinterpret_cast<int32_t *>(smem + lay.bs);
    L.f.nrm = reinterpret_cast<float *>(smem + lay.nrm);
    L.f.segf = reinterpret_cast<int *>(smem + lay.segf);
    return L;
}

template <bool RAGGED>
__global__ __launch_bounds__(kWG) void quantize_kernel(QsgdParams P) {
    extern __shared__ __align__(16) unsigned char smem[];
    EncodeLds L = carve_encode_lds(smem, P);
    const uint32_t tile = blockIdx.x;
    const Tile t = tile_geometry<RAGGED>(P, tile);
    fill_bucket_starts<RAGGED>(P, t, L.f);
    ThreadCoords c;
    load_coords(P, t, c);
    __syncthreads();
    if (P.maxnorm) bucket_norms<RAGGED, true>(P, t, L.f, c);
    else bucket_norms<RAGGED, false>(P, t, L.f, c);
    ThreadLevels lv;
    quantize_coords(P, t, L.f, c, lv);
    const int j = (int)threadIdx.x;
    const uint64_t g0 = t.A + (uint64_t)j * kCPT;
    if (c.vx0 == j * kCPT && c.vx1 == j * kCPT + kCPT) {
        int4 *dst = reinterpret_cast<int4 *>(P.levels + g0);
#pragma unroll
        for (int q = 0; q < kCPT / 4; ++q) {
            int4 o;
            o.x = (lv.neg >> (4 * q + 0)) & 1 ? -(int)lv.k[4 * q + 0] : (int)lv.k[4 * q + 0];
            o.y = (lv.neg >> (4 * q + 1)) & 1 ? -(int)lv.k[4 * q + 1] : (int)lv.k[4 * q + 1];
            o.z = (lv.neg >> (4 * q + 2)) & 1 ? -(int)lv.k[4 * q + 2] : (int)lv.k[4 * q + 2];
            o.w = (lv.neg >> (4 * q + 3)) & 1 ? -(int)lv.k[4 * q + 3] : (int)lv.k[4 * q + 3];
            dst[q] = o;
        }
    } else {
#pragma unroll
        for (int q = 0; q < kCPT; ++q) {
            const int x = j * kCPT + q;
            if (x >= c.vx0 && x < c.vx1)
                P.levels[g0 + q] = (lv.neg >> q) & 1 ? -(int)lv.k[q] : (int)lv.k[q];
        }
        // keeps the compiler from merging the last of these stores with the last
        // 16-byte store above (which it would split into 12- and 4-byte stores)
        asm volatile("" ::: "memory");
    }
    for (uint32_t b = threadIdx.x; b < t.K; b += kWG) P.norms[t.b0 + b] = L.f.nrm[b];
}

__global__ void encode_empty_kernel(uint64_t *out_bits, uint64_t *offsets) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        *out_bits = 0;
        offsets[0] = 0;
    }
}

// Code and length of one record, table path (g <= 16, k <= s <= kTabS) or
// arithmetic path. g = 0 means "no gap code" (resolved later).
template <bool TABLE>
__device__ __forceinline__ uint32_t record_entry(const uint32_t *rt, uint32_t g, uint32_t k,
                                                 uint32_t neg, uint64_t &code, uint32_t fcode) {
    if (TABLE) {
        const uint32_t e = rt[code_index(g, k, neg)];
        code = e >> 5;
        return e & 31u;
    }
    if (k == 0) { code = 0; return 0; }
    uint32_t Lk;
    const uint64_t kc = field_code(fcode, k, Lk);
    code = ((uint64_t)neg << Lk) | kc;
    uint32_t len = Lk + 1;
    if (g) {
        uint32_t Lg;
        const uint64_t gc = field_code(fcode, g, Lg);
        code |= gc << len;
        len += Lg;
    }
    return len;  // omega: <= 11 + 1 + 36 = 48 bits; gamma: <= 9 + 1 + 49 = 59
}

template <bool RAGGED, bool TABLE>
__global__ __launch_bounds__(kWG) void encode_kernel(QsgdParams P) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int sh_mx[kWaves];
    __shared__ uint32_t sh_bits[kWaves];

    EncodeLds L = carve_encode_lds(smem, P);
    const uint32_t *rt = P.code ? kCodeTableGamma.e : kCodeTableOmega.e;
    const int j = (int)threadIdx.x;
    const int lane = lane_id();
    // the wave index as a scalar, so that branches on it are uniform to the compiler
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());

    const uint32_t tend = run_first(blockIdx.x + 1, P.run, P.rem);
    uint64_t run_total = 0;
    for (uint32_t tile = run_first(blockIdx.x, P.run, P.rem); tile < tend; ++tile) {
        __syncthreads();  // separates this tile's LDS use from the previous one
        const Tile t = tile_geometry<RAGGED>(P, tile);
        fill_bucket_starts<RAGGED>(P, t, L.f);
        ThreadCoords c;
        load_coords(P, t, c);
        __syncthreads();
        if (P.maxnorm) bucket_norms<RAGGED, true>(P, t, L.f, c);
        else bucket_norms<RAGGED, false>(P, t, L.f, c);
        ThreadLevels lv;
        quantize_coords(P, t, L.f, c, lv);

        // ---- phase 1: record codes, bit count, last marker; with the table, the
        // norms of buckets starting here and the records are also packed
        // right-aligned into two 64-bit registers (coordinates 0-7 and 8-15) ----
        uint32_t ec[kCPT];
        uint64_t ecx[TABLE ? 1 : kCPT];
        uint64_t racc[2] = {0, 0};
        uint32_t rlen[2] = {0, 0};
        uint32_t r = 0;
        int prev = 0;
        int have = 0;
        int pendx = -1;
        // the tile-local bucket before the thread's first bucket start
        int kb0 = c.kf;
        if (c.vx0 < c.vx1 && ((lv.bst >> (c.vx0 - j * kCPT)) & 1u)) kb0 -= 1;
        int kbp = kb0;
#pragma unroll
        for (int q = 0; q < kCPT; ++q) {
            const int x = j * kCPT + q;
            if ((lv.bst >> q) & 1u) {
                r += 32u;
                prev = x - 1;
                have = 1;
                if (TABLE) {
                    ++kbp;
                    racc[q >> 3] = (racc[q >> 3] << 32) | (uint64_t)__float_as_uint(L.f.nrm[kbp]);
                    rlen[q >> 3] += 32u;
                }
            }
            const uint32_t k = lv.k[q];
            const uint32_t g = have ? (uint32_t)(x - prev) : 0u;
            uint64_t code;
            const uint32_t len = record_entry<TABLE>(rt, g, k, (lv.neg >> q) & 1u, code, P.code);
            if (TABLE) ec[q] = ((uint32_t)code << 5) | len;
            else { ec[q] = len; ecx[TABLE ? 0 : q] = code; }
            if (TABLE) {
                racc[q >> 3] = (racc[q >> 3] << len) | code;
                rlen[q >> 3] += len;
            }
            r += len;
            if (k) {
                if (!have) pendx = x;
                prev = x;
                have = 1;
            }
            // markers formed four coordinates at a time (as in the aligned
            // kernel: SGPR spills 73 -> 35, c5 encode 220 -> 208 us)
            if ((q & 3) == 3) asm volatile("" : "+v"(pendx), "+v"(prev), "+v"(have));
        }
        const int marker = have ? prev : INT_MIN;

        // ---- exclusive max-scan of markers: origin of the pending first gap ----
        int mi = wave_incl_max_i32(marker);
        if (lane == 63) sh_mx[wave] = mi;
        __syncthreads();
        int mpre = INT_MIN;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            if (w < wave) mpre = mpre > sh_mx[w] ? mpre : sh_mx[w];
        int mex = wave_shr1_i32(INT_MIN, mi);
        mex = mex > mpre ? mex : mpre;
        uint32_t Lp = 0;
        uint64_t pc = 0;
        if (pendx >= 0) pc = field_code(P.code, (uint32_t)(pendx - mex), Lp);
        const uint32_t bits = r + Lp;

        // ---- tile scan of bit counts ----
        const uint32_t bi = wave_incl_add_u32(bits);
        if (lane == 63) sh_bits[wave] = bi;
        __syncthreads();
        uint32_t bpre = 0, T = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            if (w < wave) bpre += sh_bits[w];
            T += sh_bits[w];
        }
        uint32_t off = (uint32_t)wave_shr1_i32(0, (int)bi);
        off += bpre;

        const uint32_t W = (T + 63u) >> 6;
        for (uint32_t w = threadIdx.x; w <= W; w += kWG) L.obuf[w] = 0;
        __syncthreads();

        // ---- phase 2: OR every record into the tile's words at its offset ----
        uint32_t p = off;
        if (Lp) or_bits(L.obuf, p, pc << (64u - Lp), Lp);
        p += Lp;
        int kb = kb0;
        if (TABLE && rlen[0] <= 64u && rlen[1] <= 64u) {
            // the two packed registers; the bucket offsets from the record lengths
            if (lv.bst) {
                uint32_t pp = p;
#pragma unroll
                for (int q = 0; q < kCPT; ++q) {
                    if ((lv.bst >> q) & 1u) {
                        ++kb;
                        P.offsets[t.b0 + kb] = pp;
                        pp += 32u;
                    }
                    pp += ec[q] & 31u;
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (rlen[h]) or_bits(L.obuf, p, racc[h] << (64u - rlen[h]), rlen[h]);
                p += rlen[h];
            }
        } else {
#pragma unroll
        for (int q = 0; q < kCPT; ++q) {
            if ((lv.bst >> q) & 1u) {
                ++kb;
                P.offsets[t.b0 + kb] = p;
                or_bits(L.obuf, p, (uint64_t)__float_as_uint(L.f.nrm[kb]) << 32, 32u);
                p += 32u;
            }
            const uint32_t len = TABLE ? (ec[q] & 31u) : ec[q];
            if (len) {
                const uint64_t code = TABLE ? (uint64_t)(ec[q] >> 5) : ecx[TABLE ? 0 : q];
                or_bits(L.obuf, p, code << (64u - len), len);
            }
            p += len;
        }
        }
        __syncthreads();

        // ---- the tile's words to its slot ----
        uint64_t *slot = P.slots + (uint64_t)tile * P.obuf_words;
        for (uint32_t w = threadIdx.x; w < W; w += kWG) slot[w] = L.obuf[w];
        if (j == 0) P.tile_bits[tile] = T;
        run_total += T;
    }
    if (threadIdx.x == 0) P.run_bits[blockIdx.x] = run_total;
}

// Aligned fast path, front half. aligned_load: the thread's 16 coordinates
// from g0 (0 past n). aligned_norm: the bucket norm RN32(sqrt(sum of squares))
// of the thread's bucket (MAXN: its max-norm max|x_i|, exact in any order). The sum: fp64 fma per thread in index order, an xor
// butterfly over the bucket's lanes (both operands of every addition are the
// same pair on each lane, so all lanes get the same bits), and for G > 64 the
// bucket's waves added in wave order through red[kWaves] (ends with a barrier
// in that case; G is uniform).
__device__ __forceinline__ void aligned_load(const QsgdParams &P, uint64_t g0, float (&x)[kCPT]) {
    if (g0 + kCPT <= P.n) {
        const float4 *src = reinterpret_cast<const float4 *>(P.v + g0);
#pragma unroll
        for (int q = 0; q < kCPT / 4; ++q) {
            const float4 f = src[q];
            x[4 * q + 0] = f.x;
            x[4 * q + 1] = f.y;
            x[4 * q + 2] = f.z;
            x[4 * q + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < kCPT; ++q) x[q] = g0 + q < P.n ? P.v[g0 + q] : 0.0f;
    }
}

template <bool MAXN = false>
__device__ __forceinline__ float aligned_norm(const float (&x)[kCPT], uint32_t G, double *red) {
    auto op = [](double a, double b) { return MAXN ? (a > b ? a : b) : a + b; };
    double acc = 0.0;
#pragma unroll
    for (int q = 0; q < kCPT; ++q) {
        const double y = (double)x[q];
        acc = MAXN ? op(acc, fabs(y)) : fma(y, y, acc);
    }
    const uint32_t gw = G < 64u ? G : 64u;
    if (gw == 64u) acc = wave_total_f64<MAXN>(acc);
    else if (gw == 32u) acc = half_wave_total_f64<MAXN>(acc);
    else
        for (uint32_t o = 1; o < gw; o <<= 1) acc = op(acc, __shfl_xor(acc, (int)o, 64));
    if (G > 64u) {
        const int wave = __builtin_amdgcn_readfirstlane(wave_id());
        if (lane_id() == 0) red[wave] = acc;
        __syncthreads();
        const uint32_t nwb = G >> 6;
        const uint32_t w0 = (uint32_t)wave & ~(nwb - 1u);
        double tsum = red[w0];
        for (uint32_t w = 1; w < nwb; ++w) tsum = op(tsum, red[w0 + w]);
        acc = tsum;
    }
    return MAXN ? (float)acc : (float)sqrt(acc);
}

// Quantize, aligned fast path (the encode fast path's front half): one
// workgroup per 4096-coordinate tile; writes sgn * k and the bucket norms.
__global__ __launch_bounds__(kWG) void quantize_aligned_kernel(QsgdParams P, uint32_t log2d) {
    __shared__ double sh_red[kWaves];
    const int j = (int)threadIdx.x;
    const uint32_t G = 1u << (log2d - 4);
    const uint32_t tile = blockIdx.x;
    const uint64_t g0 = (uint64_t)tile * kTC + (uint64_t)(j * kCPT);
    float x[kCPT];
    aligned_load(P, g0, x);
    const float norm = P.maxnorm ? aligned_norm<true>(x, G, sh_red) : aligned_norm<false>(x, G, sh_red);
    if ((j & (G - 1)) == 0 && g0 < P.n) P.norms[g0 >> log2d] = norm;
    // ratios (ratio_of) per block of four, just before their levels
    const double cb = ratio_scale(norm, P.s);
    const bool tie = ratio_may_tie(norm, P.sigma);
    const uint32_t key0 = (uint32_t)P.seed, key1 = (uint32_t)(P.seed >> 32);
    int32_t lv[kCPT];
#pragma unroll
    for (int g = 0; g < kCPT / 4; ++g) {
        uint32_t w[4];
        const uint64_t blk = (g0 >> 2) + (uint64_t)g;
        philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), key0, key1, w);
        float rq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) rq[e] = ratio_fast(x[4 * g + e], cb);
        if (tie) {
#pragma unroll
            for (int e = 0; e < 4; ++e) rq[e] = ratio_tiefix(x[4 * g + e], rq[e], norm, P.s);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int q = 4 * g + e;
            const int k = (int)level_of_ratio(rq[e], w[e]);
            lv[q] = (__float_as_uint(rq[e]) >> 31) ? -k : k;
        }
    }
    if (g0 + kCPT <= P.n) {
        int4 *dst = reinterpret_cast<int4 *>(P.levels + g0);
#pragma unroll
        for (int q = 0; q < kCPT / 4; ++q)
            dst[q] = make_int4(lv[4 * q], lv[4 * q + 1], lv[4 * q + 2], lv[4 * q + 3]);
    } else {
#pragma unroll
        for (int q = 0; q < kCPT; ++q)
            if (g0 + q < P.n) P.levels[g0 + q] = lv[q];
    }
}

// Encode pass 1, fast path for buckets of d = 2^m coordinates, 16 <= d <= 4096,
// one vector, s <= kTabS. Tile t is the 4096 coordinates from 4096 t (4096 / d
// whole buckets); the G = d / 16 threads of a bucket are consecutive, so each
// thread's 16 coordinates lie in one bucket and thread j starts a bucket iff
// j mod G = 0. Coordinates past n read as 0, which quantize to level 0 and add
// nothing to a norm. Per tile:
//   - the workgroup's next tile (tile + gridDim.x) is copied into LDS with
//     direct global-to-LDS loads while this one is processed;
//   - bucket norms (aligned_norm), levels and record codes as in the general
//     kernel; each thread packs its records into two 64-bit registers
//     (coordinates 0-7 and 8-15) while it codes them;
//   - exclusive max-scan of markers (origin of each thread's pending first gap)
//     and sum-scan of bit counts;
//   - each thread ORs its bit string (norm or pending first gap, then its two
//     record registers) into the tile's LDS words at its offset, and the words
//     go to the tile's slot.
__host__ __device__ constexpr size_t aligned_encode_lds_bytes(uint32_t obuf_words) {
    return align16((size_t)obuf_words * 8) + (size_t)kTC * 4;
}

// Starts copying the 4096 coordinates of a whole tile from v[g] into LDS
// pbuf[0, 4096) with direct global-to-LDS loads: wave w copies the 4 KB its own
// threads use (thread j's 16 coordinates land at pbuf[16 j]), so a wave only
// has to wait for its own loads (vmcnt) before reading them.
__device__ __forceinline__ void tile_prefetch_lds(const float *v, uint64_t g, float *pbuf, int wave,
                                                  int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t o = (uint32_t)wave * 1024u + (uint32_t)i * 256u;
        __builtin_amdgcn_global_load_lds(v + g + o + 4u * (uint32_t)lane,
                                         (__attribute__((address_space(3))) void *)(pbuf + o), 16, 0, 0);
    }
}

// A tile's results (aligned path): its words to its slot, each thread clearing
// the LDS words it copied; its length; its tile-relative bucket offsets.
__device__ __forceinline__ void store_tile_slot(const QsgdParams &P, uint64_t *obuf, uint32_t tile,
                                                uint32_t T, bool bstart, uint32_t off, uint32_t log2d) {
    const uint32_t W = (T + 63u) >> 6;
    uint64_t *slot = P.slots + (uint64_t)tile * P.obuf_words;
    for (uint32_t w = threadIdx.x; w < W; w += kWG) {
        slot[w] = obuf[w];
        obuf[w] = 0;
    }
    if (threadIdx.x == 0) P.tile_bits[tile] = T;
    if (bstart) P.offsets[((uint64_t)tile << (12 - log2d)) + (threadIdx.x >> (log2d - 4))] = off;
}

// QUARTERS: records packed per quarter of the thread (4 coordinates) in four
// 64-bit registers, for large levels, whose records would often pass 64 bits in
// a half; otherwise per half (8 coordinates) in two. A part whose records pass
// 64 bits draws its levels again from v and Philox and writes its records one
// at a time.
template <bool QUARTERS>
__global__ __launch_bounds__(kWG) void encode_aligned_kernel(QsgdParams P, uint32_t log2d) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int sh_mx[kWaves];
    __shared__ uint32_t sh_bits[kWaves];
    __shared__ double sh_red[kWaves];

    // dynamic LDS: [obuf][pbuf] (aligned_encode_lds_bytes); the record code
    // table is read from constant memory
    uint64_t *obuf = reinterpret_cast<uint64_t *>(smem);
    float *pbuf = reinterpret_cast<float *>(smem + align16((size_t)P.obuf_words * 8));
    const uint32_t *rt = P.code ? kCodeTableGamma.e : kCodeTableOmega.e;
    const int j = (int)threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());
    const uint32_t G = 1u << (log2d - 4);      // threads per bucket
    const uint32_t key0 = (uint32_t)P.seed, key1 = (uint32_t)(P.seed >> 32);
    const int x0 = j * kCPT;
    const bool first_of_bucket = (j & (G - 1)) == 0;
    // the previous tile's results go out after the next tile's first barrier,
    // before that tile's prefetch is issued, so the wait for the prefetch never
    // waits for these stores
    uint32_t prev_tile = 0xffffffffu, prev_T = 0, prev_off = 0;
    bool prev_bstart = false;

    // whole tiles are prefetched into pbuf; a partial tile is loaded directly
    const uint32_t tend = run_first(blockIdx.x + 1, P.run, P.rem);
    uint64_t run_total = 0;
    uint32_t cur = run_first(blockIdx.x, P.run, P.rem);
    bool pref = cur < tend && (uint64_t)cur * kTC + kTC <= P.n;
    if (pref) tile_prefetch_lds(P.v, (uint64_t)cur * kTC, pbuf, wave, lane);

    for (; cur < tend; ++cur) {
        const uint32_t tile = cur;
        const uint64_t g0 = (uint64_t)tile * kTC + (uint64_t)x0;
        float x[kCPT];
        if (pref) {
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's prefetch has landed
            const float4 *src = reinterpret_cast<const float4 *>(pbuf + x0);
#pragma unroll
            for (int q = 0; q < kCPT / 4; ++q) {
                const float4 f = src[q];
                x[4 * q + 0] = f.x;
                x[4 * q + 1] = f.y;
                x[4 * q + 2] = f.z;
                x[4 * q + 3] = f.w;
            }
        } else {
            aligned_load(P, g0, x);
        }
        const float norm = P.maxnorm ? aligned_norm<true>(x, G, sh_red) : aligned_norm<false>(x, G, sh_red);
        const bool bstart = first_of_bucket && g0 < P.n;
        // ratios (ratio_of) per block of four, just before their levels; the
        // coordinates are converted to fp64 again there, so that the norm's fp64
        // copies do not stay live through the loop (91 VGPRs instead of 117, five
        // waves per SIMD instead of four)
        const double cb = ratio_scale(norm, P.s);
        const bool tie = ratio_may_tie(norm, P.sigma);
#pragma unroll
        for (int q = 0; q < kCPT; ++q) asm volatile("" : "+v"(x[q]));

        // ---- levels and record codes; records packed right-aligned into two
        // 64-bit registers (coordinates 0-7 and 8-15) ----
        constexpr int NA = QUARTERS ? 4 : 2;          // packing registers
        constexpr int QS = QUARTERS ? 2 : 3;          // coordinate q goes to register q >> QS
        uint64_t racc[NA] = {};
        uint32_t rlen[NA] = {};
        int prev = x0 - 1;
        bool have = bstart;
        int pendx = -1;
        const uint64_t blk0 = g0 >> 2;
#pragma unroll
        for (int g = 0; g < kCPT / 4; ++g) {
            uint32_t w[4];
            const uint64_t blk = blk0 + (uint64_t)g;
            // fresh scalar copies of the key per call: keeps the round keys out
            // of the registers that live across the persistent loop
            uint32_t k0 = key0, k1 = key1;
            asm volatile("" : "+s"(k0), "+s"(k1));
            philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), k0, k1, w);
            float rq[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) rq[e] = ratio_fast(x[4 * g + e], cb);
            if (tie) {
#pragma unroll
                for (int e = 0; e < 4; ++e) rq[e] = ratio_tiefix(x[4 * g + e], rq[e], norm, P.s);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int q = 4 * g + e;
                const int xi = x0 + q;
                const uint32_t k = level_of_ratio(rq[e], w[e]);
                const uint32_t neg = __float_as_uint(rq[e]) >> 31;
                const uint32_t gg = have ? (uint32_t)(xi - prev) : 0u;
                const uint32_t ent = rt[code_index(gg, k, neg)];
                const uint32_t len = ent & 31u;
                racc[q >> QS] = (racc[q >> QS] << len) | (uint64_t)(ent >> 5);
                rlen[q >> QS] += len;
                const bool nz = k != 0u;
                pendx = (nz && !have) ? xi : pendx;
                prev = nz ? xi : prev;
                have = have || nz;
            }
            // the markers are formed block by block: left to the compiler, the
            // selects sank below the loop and kept 16 lane masks live in SGPRs
            // (58 spilled to VGPR lanes, 5 now; c3 encode 127.9 -> 126.0 us)
            asm volatile("" : "+v"(pendx), "+v"(prev));
        }
        uint32_t r = bstart ? 32u : 0u;
#pragma unroll
        for (int h = 0; h < NA; ++h) r += rlen[h];
        const int marker = have ? prev : INT_MIN;

        // ---- exclusive max-scan of markers: origin of the pending first gap ----
        const int mi = wave_incl_max_i32(marker);
        if (lane == 63) sh_mx[wave] = mi;
        __syncthreads();
        // the previous tile's words to its slot (each thread clears the words it
        // copied), then start loading the next tile (this wave has read its
        // part of pbuf)
        if (prev_tile != 0xffffffffu) {
            store_tile_slot(P, obuf, prev_tile, prev_T, prev_bstart, prev_off, log2d);
        } else {
            for (uint32_t w = threadIdx.x; w < P.obuf_words; w += kWG) obuf[w] = 0;
        }
        const uint32_t nxt = cur + 1;
        const bool pref_next = nxt < tend && (uint64_t)nxt * kTC + kTC <= P.n;
        if (pref_next) tile_prefetch_lds(P.v, (uint64_t)nxt * kTC, pbuf, wave, lane);
        int mpre = INT_MIN;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            if (w < wave) mpre = mpre > sh_mx[w] ? mpre : sh_mx[w];
        int mex = wave_shr1_i32(INT_MIN, mi);
        mex = mex > mpre ? mex : mpre;
        uint32_t Lp = 0;
        uint64_t pc = 0;
        if (pendx >= 0) pc = field_code(P.code, (uint32_t)(pendx - mex), Lp);
        const uint32_t bits = r + Lp;

        // ---- tile scan of bit counts ----
        const uint32_t bi = wave_incl_add_u32(bits);
        if (lane == 63) sh_bits[wave] = bi;
        __syncthreads();
        uint32_t bpre = 0, T = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            if (w < wave) bpre += sh_bits[w];
            T += sh_bits[w];
        }
        uint32_t off = (uint32_t)wave_shr1_i32(0, (int)bi);
        off += bpre;

        // ---- OR the thread's pieces into the tile's words ----
        uint32_t p = off;
        if (bstart) {
            or_bits(obuf, p, (uint64_t)__float_as_uint(norm) << 32, 32u);
            p += 32u;
        } else if (Lp) {
            or_bits(obuf, p, pc << (64u - Lp), Lp);
            p += Lp;
        }
#pragma unroll
        for (int h = 0; h < NA; ++h) {
            if (rlen[h] <= 64u) {
                if (rlen[h]) or_bits(obuf, p, racc[h] << (64u - rlen[h]), rlen[h]);
                p += rlen[h];
            } else {
                // more than 64 bits in this part: its records one at a time,
                // the gaps followed from the thread's first coordinate, the
                // levels drawn again from v
                constexpr int QW = kCPT / NA;
                int pv = x0 - 1;
                bool hv = bstart;
#pragma unroll 1
                for (int q = 0; q < QW * h + QW; ++q) {
                    const uint64_t gi = g0 + (uint64_t)q;
                    uint32_t w[4];
                    uint32_t k0 = key0, k1 = key1;
                    asm volatile("" : "+s"(k0), "+s"(k1));
                    philox4x32_10((uint32_t)(gi >> 2), (uint32_t)(gi >> 34), k0, k1, w);
                    const float xv = gi < P.n ? P.v[gi] : 0.0f;
                    const uint32_t k = qlevel(xv, cb, tie, norm, P.s, w[q & 3]);
                    const uint32_t neg = __float_as_uint(xv) >> 31;
                    if (q >= QW * h) {
                        const uint32_t gg = hv ? (uint32_t)(x0 + q - pv) : 0u;
                        const uint32_t ent = rt[code_index(gg, k, neg)];
                        const uint32_t len = ent & 31u;
                        if (len) or_bits(obuf, p, (uint64_t)(ent >> 5) << (64u - len), len);
                        p += len;
                    }
                    pv = k ? x0 + q : pv;
                    hv = hv || k != 0u;
                }
            }
        }
        prev_tile = tile;
        prev_T = T;
        run_total += T;
        prev_off = off;
        prev_bstart = bstart;
        pref = pref_next;
    }
    if (prev_tile != 0xffffffffu) {
        __syncthreads();
        store_tile_slot(P, obuf, prev_tile, prev_T, prev_bstart, prev_off, log2d);
    }
    if (threadIdx.x == 0) P.run_bits[blockIdx.x] = run_total;
}

// Encode pass 2. Workgroup w takes tiles [t0, t1) (a contiguous share): the
// stream offset of t0 is the sum of all earlier tiles' lengths, then a block
// scan gives its tiles' offsets. Stream word i (bits [64 i, 64 i + 64)) is
// written by the workgroup of the tile holding bit 64 i, gathered from that
// tile's slot and, past its end, from the next tiles' slots. The tiles' bucket
// offsets get the tile offset added; the last tile also writes offsets[nb] and
// out_bits.
struct FinishParams {
    uint64_t *out;
    const uint64_t *slots;
    const uint32_t *tile_bits;
    const uint64_t *run_bits;  // pass 1's run totals
    uint32_t run, rem;         // pass 1's runs (run_first)
    uint64_t *offsets;
    uint64_t *out_bits;
    uint64_t nb;
    uint32_t ntiles;
    uint32_t slot_words;
    uint32_t K;        // buckets per tile
    uint32_t chunk;    // tiles per workgroup
};

constexpr int kFinishTiles = 256;  // tiles per finish workgroup at most

// The `take` (1..64) bits of tile tt's string from bit rel on, at the top of
// the result.
__device__ __forceinline__ uint64_t slot_bits(const FinishParams &F, uint32_t tt, uint32_t rel,
                                              uint32_t take) {
    const uint64_t *s = F.slots + (uint64_t)tt * F.slot_words;
    const uint32_t wi = rel >> 6, sh = rel & 63u;
    uint64_t x = s[wi] << sh;
    if (sh) x |= s[wi + 1] >> (64u - sh);
    return take >= 64u ? x : (x & ~(~0ull >> take));
}

__global__ __launch_bounds__(kWG) void encode_finish_kernel(FinishParams F) {
    __shared__ uint64_t sh_base[kFinishTiles + 1];
    __shared__ uint64_t sh_red[kWaves];
    __shared__ uint64_t sh_scan[kWaves];
    const uint32_t t0 = blockIdx.x * F.chunk;
    const uint32_t t1 = t0 + F.chunk < F.ntiles ? t0 + F.chunk : F.ntiles;
    if (t0 >= t1) return;
    const int j = (int)threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());

    // stream offset of t0: the totals of the pass-1 runs before t0's run, then
    // the lengths of the tiles of that run before t0
    const uint32_t r0 = run_of(t0, F.run, F.rem);
    const uint32_t m = t1 - t0;  // this share's tiles (chunk <= kFinishTiles <= kWG)
    const uint64_t mine = (uint32_t)j < m ? (uint64_t)F.tile_bits[t0 + j] : 0ull;
    // (eight loads in flight per thread: a sum over a strided loop would wait
    // for each load before issuing the next)
    uint64_t acc = 0;
    for (uint32_t i = (uint32_t)j; i < r0; i += 8u * kWG) {
        uint64_t rb[8];
#pragma unroll
        for (uint32_t u = 0; u < 8u; ++u) rb[u] = i + u * kWG < r0 ? F.run_bits[i + u * kWG] : 0ull;
#pragma unroll
        for (uint32_t u = 0; u < 8u; ++u) acc += rb[u];
    }
    for (uint32_t t = run_first(r0, F.run, F.rem) + (uint32_t)j; t < t0; t += kWG) acc += F.tile_bits[t];
    acc = wave_incl_add_u64(acc);
    if (lane == 63) sh_red[wave] = acc;
    if (m <= 64u) {
        // the share's tiles are wave 0's lanes: their offsets need no second
        // block-wide step
        const uint64_t incl = wave_incl_add_u64(mine);
        __syncthreads();
        uint64_t pre = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) pre += sh_red[w];
        if ((uint32_t)j < m) sh_base[j] = pre + incl - mine;
        if ((uint32_t)j + 1u == m) sh_base[m] = pre + incl;  // end of the share
    } else {
        __syncthreads();
        uint64_t pre = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) pre += sh_red[w];
        uint64_t total = 0;
        const uint64_t ex = block_excl_add_u64(mine, sh_scan, total);
        if ((uint32_t)j < m) sh_base[j] = pre + ex;
        if (j == 0) sh_base[m] = pre + total;  // end of the share
    }
    __syncthreads();

    // every stream word whose first bit lies in this share's tiles, four per
    // thread at a time with their slot loads issued together; a thread's words
    // increase, so its tile index only moves forward
    const uint64_t wbeg = (sh_base[0] + 63) >> 6, wend = (sh_base[m] + 63) >> 6;
    uint32_t i = 0;
    for (uint64_t wb = wbeg; wb < wend; wb += 4 * kWG) {
        uint32_t tt[4], rel[4], Tt[4];
        uint64_t a[4], b[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint64_t w = wb + (uint64_t)j + (uint64_t)k * kWG;
            const uint64_t g = (w < wend ? w : wend - 1) << 6;
            while (sh_base[i + 1] <= g) ++i;
            tt[k] = t0 + i;
            rel[k] = (uint32_t)(g - sh_base[i]);
            Tt[k] = (uint32_t)(sh_base[i + 1] - sh_base[i]);
            const uint64_t *s = F.slots + (uint64_t)tt[k] * F.slot_words + (rel[k] >> 6);
            a[k] = s[0];
            b[k] = s[1];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint64_t w = wb + (uint64_t)j + (uint64_t)k * kWG;
            if (w >= wend) break;
            const uint32_t sh = rel[k] & 63u;
            uint64_t v = a[k] << sh;
            if (sh) v |= b[k] >> (64u - sh);
            if (Tt[k] - rel[k] < 64u) {
                // the word runs past its tile: the rest from the next tiles
                uint32_t have = Tt[k] - rel[k];
                v &= ~(~0ull >> have);
                uint32_t t2 = tt[k];
                while (have < 64u && ++t2 < F.ntiles) {
                    const uint32_t T2 = t2 < t1 ? (uint32_t)(sh_base[t2 - t0 + 1] - sh_base[t2 - t0])
                                                : F.tile_bits[t2];
                    const uint32_t take = 64u - have < T2 ? 64u - have : T2;
                    v |= slot_bits(F, t2, 0u, take) >> have;
                    have += take;
                }
            }
            F.out[w] = v;
        }
    }
    // bucket offsets of this share's tiles
    const uint64_t bb0 = (uint64_t)t0 * F.K;
    const uint64_t bb1 = (uint64_t)t1 * F.K < F.nb ? (uint64_t)t1 * F.K : F.nb;
    for (uint64_t b = bb0 + (uint64_t)j; b < bb1; b += kWG) F.offsets[b] += sh_base[(b - bb0) / F.K];
    if (t1 == F.ntiles && j == 0) {
        F.offsets[F.nb] = sh_base[m];
        *F.out_bits = sh_base[m];
    }
}

}  // namespace qsgd
