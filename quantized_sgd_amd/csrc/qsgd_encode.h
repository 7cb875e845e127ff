// Quantize kernel and the fused single-pass encode kernel.
//
// Page "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding":
// definition paragraph (Q_s and the Elias-coded tuple of norm, signs, non-zero
// gaps and levels) and the claim on Elias coding (F = 32 bit norm).
//
// Encode, per tile (a run of whole buckets, <= 4096 coordinates, one workgroup;
// workgroups are persistent and take tiles in order from a work counter):
//   1. load v once from HBM, per-bucket norms, Philox rounding (qsgd_front.h);
//   2. each thread looks up the code of every coordinate's record -- the 32-bit
//      norm at a bucket start, and omega(gap) | sign | omega(k) per non-zero --
//      in a table of all records with gap <= 16 and k <= s (gaps inside one
//      thread's 16 coordinates never exceed 16) and sums their lengths. The gap
//      of a thread's first non-zero, when its origin lies in an earlier thread,
//      is resolved after an exclusive max-scan of "last marker" positions;
//   3. an exclusive sum-scan of per-thread bit counts gives each thread's offset
//      in the tile and the tile's size T;
//   4. decoupled lookback over earlier tiles' status words (agent-scope atomics,
//      flag and value packed in one 64-bit word) gives the tile's stream offset;
//   5. every record is OR-ed into the tile's 64-bit words in LDS at its final
//      bit position, and the words are stored with coalesced 8-byte stores. The
//      word shared with the previous tile is completed with that tile's
//      published "carry" (its partial last word); the tile's own partial last
//      word is published the same way for the next tile.
// Every output word is written by exactly one tile; v is read once.
#pragma once

#include "qsgd_front.h"

namespace qsgd {

// Record code table for s <= kTabS: entry (code << 5) | length of
// omega(g) | sign | omega(k) for g in [0, 16] (g = 0: no gap code) and k in
// [0, s] (k = 0: no record, entry 0). Index ((k * 17 + g) << 1) | sign, which
// needs no integer multiply (k * 17 = (k << 4) + k).
constexpr uint32_t kTabS = 64;
constexpr uint32_t kTabG = 17;

__host__ __device__ constexpr uint32_t code_table_entries(uint32_t s) { return kTabG * (s + 1) * 2; }

__device__ __forceinline__ uint32_t code_index(uint32_t g, uint32_t k, uint32_t neg) {
    return ((((k << 4) + k) + g) << 1) | neg;
}

__device__ inline void build_code_table(uint32_t *rt, uint32_t s) {
    const uint32_t n = code_table_entries(s);
    for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
        const uint32_t neg = i & 1u;
        const uint32_t g = (i >> 1) % kTabG;
        const uint32_t k = (i >> 1) / kTabG;
        uint32_t e = 0;
        if (k) {
            uint32_t Lk;
            const uint64_t kc = omega_code(k, Lk);
            uint64_t code = ((uint64_t)neg << Lk) | kc;
            uint32_t len = Lk + 1;
            if (g) {
                uint32_t Lg;
                const uint64_t gc = omega_code(g, Lg);
                code |= gc << len;
                len += Lg;
            }
            e = ((uint32_t)code << 5) | len;
        }
        rt[i] = e;
    }
}

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
    uint32_t *rt;   // record code table (table path)
};

__host__ __device__ constexpr size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Dynamic LDS layout shared by host and device: [obuf][rt][cb][segv][bs][nrm][segf].
struct EncodeLayout {
    size_t obuf, rt, cb, segv, bs, nrm, segf, total;
    __host__ __device__ EncodeLayout(uint32_t obuf_words, uint32_t rt_entries, uint32_t K) {
        size_t off = 0;
        obuf = off; off = align16(off + (size_t)obuf_words * 8);
        rt = off;   off = align16(off + (size_t)rt_entries * 4);
        cb = off;   off = align16(off + (size_t)K * 8);
        segv = off; off = align16(off + kWaves * 8);
        bs = off;   off = align16(off + (size_t)(K + 1) * 4);
        nrm = off;  off = align16(off + (size_t)K * 4);
        segf = off; off = align16(off + kWaves * 4);
        total = off;
    }
};

__device__ __forceinline__ EncodeLds carve_encode_lds(unsigned char *smem, const QsgdParams &P,
                                                      uint32_t rt_entries) {
    const EncodeLayout lay(P.obuf_words, rt_entries, P.K);
    EncodeLds L;
    L.obuf = reinterpret_cast<uint64_t *>(smem + lay.obuf);
    L.rt = reinterpret_cast<uint32_t *>(smem + lay.rt);
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
    EncodeLds L = carve_encode_lds(smem, P, 0);
    const uint32_t tile = blockIdx.x;
    const Tile t = tile_geometry<RAGGED>(P, tile);
    fill_bucket_starts<RAGGED>(P, t, L.f);
    ThreadCoords c;
    load_coords(P, t, c);
    __syncthreads();
    bucket_norms<RAGGED>(P, t, L.f, c);
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
    }
    for (uint32_t b = threadIdx.x; b < t.K; b += kWG) P.norms[t.b0 + b] = L.f.nrm[b];
}

__global__ void encode_init_kernel(uint64_t *status, uint64_t *carry, uint32_t *ticket, uint32_t ntiles) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t stride = gridDim.x * blockDim.x;
    for (uint32_t t = i; t < ntiles; t += stride) {
        status[t] = 0;
        carry[t] = 0;
    }
    if (i == 0) *ticket = 0;
}

__global__ void encode_empty_kernel(uint64_t *out_bits, uint64_t *offsets) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        *out_bits = 0;
        offsets[0] = 0;
    }
}

constexpr uint64_t kFlagAgg = 1ull << 62;
constexpr uint64_t kFlagIncl = 2ull << 62;
constexpr uint64_t kValMask = (1ull << 62) - 1;

// Decoupled lookback (Merrill and Garland, single-pass prefix scan), run by wave
// 0 of the tile's workgroup: publishes the tile's bit count T as an aggregate,
// sums the predecessors' values back to the nearest inclusive one (lane l
// inspects tile - 1 - l, 64 tiles per step) and publishes the inclusive value.
// Returns the tile's exclusive stream offset, uniform across the wave. Waits
// only in wave-uniform control flow.
__device__ __forceinline__ uint64_t tile_lookback(const QsgdParams &P, uint32_t tile, uint32_t T) {
    const int lane = lane_id();
    if (lane == 0) st_agent(&P.status[tile], (tile == 0 ? kFlagIncl : kFlagAgg) | (uint64_t)T);
    uint64_t excl = 0;
    int64_t i = (int64_t)tile - 1;
    while (i >= 0) {
        const int64_t idx = i - lane;
        const uint64_t w = idx >= 0 ? ld_agent(&P.status[idx]) : kFlagIncl;
        const uint64_t f = w & ~kValMask;
        const uint64_t incl = __ballot(f == kFlagIncl);
        const uint64_t zero = __ballot(f == 0);
        // lanes up to (and including) the nearest inclusive one, if all ready
        const int pfx = incl ? __builtin_ctzll(incl) : 63;
        const uint64_t need = (pfx == 63) ? ~0ull : ((2ull << pfx) - 1ull);
        if ((zero & need) != 0) {
            __builtin_amdgcn_s_sleep(1);
            continue;
        }
        uint64_t v = (lane <= pfx) ? (w & kValMask) : 0ull;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
        excl += v;
        if (incl) break;
        i -= 64;
    }
    excl = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(excl >> 32)) << 32) |
           (uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)excl);
    if (lane == 0 && tile != 0) st_agent(&P.status[tile], kFlagIncl | (excl + (uint64_t)T));
    return excl;
}

// Stores the tile's W words (stream bits [base - head, base + T), head = base
// mod 64): interior words by all threads, the edge words by wave 0. The word
// shared with the previous tile is completed with that tile's published carry
// (its partial last word, bit 0 = ready); the tile's own partial last word is
// published the same way unless it is the last tile.
__device__ __forceinline__ void store_tile(const QsgdParams &P, const uint64_t *obuf, uint32_t tile,
                                           uint64_t base, uint32_t T, uint32_t W, int wave, int lane,
                                           bool last) {
    uint64_t *dst = P.out + (base >> 6);
    for (uint32_t w = 1 + threadIdx.x; w + 1 < W; w += kWG) dst[w] = obuf[w];
    if (wave != 0) return;
    const bool head_shared = (base & 63u) != 0;
    const bool tail_partial = ((base + T) & 63u) != 0;
    if (W > 1) {
        if (tail_partial && !last) {
            if (lane == 0) st_agent(&P.carry[tile], obuf[W - 1] | 1ull);
        } else {
            if (lane == 0) {
                dst[W - 1] = obuf[W - 1];
                st_agent(&P.carry[tile], 1ull);
            }
        }
    }
    uint64_t hw = obuf[0];
    if (head_shared) {
        uint64_t cw;
        while (true) {
            cw = ld_agent(&P.carry[tile - 1]);
            if (__builtin_amdgcn_readfirstlane((uint32_t)cw) & 1u) break;
            __builtin_amdgcn_s_sleep(1);
        }
        hw |= cw & ~1ull;
    }
    if (lane == 0) {
        if (W > 1) {
            dst[0] = hw;
        } else if (tail_partial && !last) {
            st_agent(&P.carry[tile], hw | 1ull);
        } else {
            dst[0] = hw;
            st_agent(&P.carry[tile], 1ull);
        }
    }
}

// Code and length of one record, table path (g <= 16, k <= s <= kTabS) or
// arithmetic path. g = 0 means "no gap code" (resolved later).
template <bool TABLE>
__device__ __forceinline__ uint32_t record_entry(const uint32_t *rt, uint32_t g, uint32_t k,
                                                 uint32_t neg, uint64_t &code) {
    if (TABLE) {
        const uint32_t e = rt[code_index(g, k, neg)];
        code = e >> 5;
        return e & 31u;
    }
    if (k == 0) { code = 0; return 0; }
    uint32_t Lk;
    const uint64_t kc = omega_code(k, Lk);
    code = ((uint64_t)neg << Lk) | kc;
    uint32_t len = Lk + 1;
    if (g) {
        uint32_t Lg;
        const uint64_t gc = omega_code(g, Lg);
        code |= gc << len;
        len += Lg;
    }
    return len;  // <= 11 + 1 + 36 = 48 bits
}

template <bool RAGGED, bool TABLE>
__global__ __launch_bounds__(kWG) void encode_kernel(QsgdParams P) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ uint32_t sh_tile;
    __shared__ uint64_t sh_base;
    __shared__ int sh_mx[kWaves];
    __shared__ uint32_t sh_bits[kWaves];

    const uint32_t rt_entries = TABLE ? code_table_entries(P.s) : 0u;
    EncodeLds L = carve_encode_lds(smem, P, rt_entries);
    if (TABLE) build_code_table(L.rt, P.s);
    const int j = (int)threadIdx.x;
    const int lane = lane_id();
    // the wave index as a scalar, so that branches on it are uniform to the compiler
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());

    for (;;) {
        // Every wait and every single-lane section below sits in wave-uniform
        // control flow (decisions on readfirstlane values): a lane-divergent
        // spin loop inside this persistent loop lets the compiler run the next
        // iteration's barrier for some lanes of wave 0 before the waiting lane
        // has left, which desynchronises the workgroup's barriers.
        if (wave == 0) {
            uint32_t tk = 0;
            if (lane == 0) tk = atomicAdd(P.ticket, 1u);
            tk = __builtin_amdgcn_readfirstlane(tk);
            if (lane == 0) sh_tile = tk;
        }
        __syncthreads();  // also separates this tile's LDS use from the previous one
        const uint32_t tile = __builtin_amdgcn_readfirstlane(sh_tile);
        if (tile >= P.ntiles) break;
        const Tile t = tile_geometry<RAGGED>(P, tile);
        fill_bucket_starts<RAGGED>(P, t, L.f);
        ThreadCoords c;
        load_coords(P, t, c);
        __syncthreads();
        bucket_norms<RAGGED>(P, t, L.f, c);
        ThreadLevels lv;
        quantize_coords(P, t, L.f, c, lv);

        // ---- phase 1: record codes, bit count, last marker ----
        uint32_t ec[kCPT];
        uint64_t ecx[TABLE ? 1 : kCPT];
        uint32_t r = 0;
        int prev = 0;
        int have = 0;
        int pendx = -1;
#pragma unroll
        for (int q = 0; q < kCPT; ++q) {
            const int x = j * kCPT + q;
            if ((lv.bst >> q) & 1u) {
                r += 32u;
                prev = x - 1;
                have = 1;
            }
            const uint32_t k = lv.k[q];
            const uint32_t g = have ? (uint32_t)(x - prev) : 0u;
            uint64_t code;
            const uint32_t len = record_entry<TABLE>(L.rt, g, k, (lv.neg >> q) & 1u, code);
            if (TABLE) ec[q] = ((uint32_t)code << 5) | len;
            else { ec[q] = len; ecx[TABLE ? 0 : q] = code; }
            r += len;
            if (k) {
                if (!have) pendx = x;
                prev = x;
                have = 1;
            }
        }
        const int marker = have ? prev : INT_MIN;

        // ---- exclusive max-scan of markers: origin of the pending first gap ----
        int mi = wave_incl_scan(marker, [](int a, int b) { return a > b ? a : b; });
        if (lane == 63) sh_mx[wave] = mi;
        __syncthreads();
        int mpre = INT_MIN;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            if (w < wave) mpre = mpre > sh_mx[w] ? mpre : sh_mx[w];
        int mex = __shfl_up(mi, 1, 64);
        if (lane == 0) mex = INT_MIN;
        mex = mex > mpre ? mex : mpre;
        uint32_t Lp = 0;
        uint64_t pc = 0;
        if (pendx >= 0) pc = omega_code((uint32_t)(pendx - mex), Lp);
        const uint32_t bits = r + Lp;

        // ---- tile scan of bit counts ----
        const uint32_t bi = wave_incl_scan(bits, [](uint32_t a, uint32_t b) { return a + b; });
        if (lane == 63) sh_bits[wave] = bi;
        __syncthreads();
        uint32_t bpre = 0, T = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            if (w < wave) bpre += sh_bits[w];
            T += sh_bits[w];
        }
        uint32_t off = __shfl_up(bi, 1, 64);
        if (lane == 0) off = 0;
        off += bpre;

        // ---- decoupled lookback: stream offset of this tile ----
        if (wave == 0) {
            const uint64_t excl = tile_lookback(P, tile, T);
            if (lane == 0) sh_base = excl;
        }
        __syncthreads();
        const uint64_t base = sh_base;
        const uint32_t head = (uint32_t)(base & 63u);
        const uint32_t W = (head + T + 63u) >> 6;
        for (uint32_t w = threadIdx.x; w < W; w += kWG) L.obuf[w] = 0;
        const bool last = (tile == P.ntiles - 1);
        if (last && j == 0) {
            P.offsets[P.nb] = base + T;
            *P.out_bits = base + T;
        }
        __syncthreads();

        // ---- phase 2: OR every record into the tile's words at its position ----
        uint32_t p = head + off;
        if (Lp) or_bits(L.obuf, p, pc << (64u - Lp), Lp);
        p += Lp;
        int kb = c.kf;
        if (c.vx0 < c.vx1 && ((lv.bst >> (c.vx0 - j * kCPT)) & 1u)) kb -= 1;
#pragma unroll
        for (int q = 0; q < kCPT; ++q) {
            if ((lv.bst >> q) & 1u) {
                ++kb;
                P.offsets[t.b0 + kb] = base - head + p;
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
        __syncthreads();

        store_tile(P, L.obuf, tile, base, T, W, wave, lane, last);
    }
}

// Aligned fast path, front half: loads the thread's 16 coordinates from g0 (0
// past n) and returns its bucket's norm RN32(sqrt(sum of squares)). The sum:
// fp64 fma per thread in index order, an xor butterfly over the bucket's lanes
// (both operands of every addition are the same pair on each lane, so all lanes
// get the same bits), and for G > 64 the bucket's waves added in wave order
// through red[kWaves] (ends with a barrier in that case; G is uniform).
__device__ __forceinline__ float aligned_front(const QsgdParams &P, uint64_t g0, uint32_t G,
                                               double *red, float (&x)[kCPT]) {
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
    double acc = 0.0;
#pragma unroll
    for (int q = 0; q < kCPT; ++q) {
        const double y = (double)x[q];
        acc = fma(y, y, acc);
    }
    const uint32_t gw = G < 64u ? G : 64u;
    for (uint32_t o = 1; o < gw; o <<= 1) acc += __shfl_xor(acc, (int)o, 64);
    if (G > 64u) {
        const int wave = __builtin_amdgcn_readfirstlane(wave_id());
        if (lane_id() == 0) red[wave] = acc;
        __syncthreads();
        const uint32_t nwb = G >> 6;
        const uint32_t w0 = (uint32_t)wave & ~(nwb - 1u);
        double tsum = red[w0];
        for (uint32_t w = 1; w < nwb; ++w) tsum += red[w0 + w];
        acc = tsum;
    }
    return (float)sqrt(acc);
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
    const float norm = aligned_front(P, g0, G, sh_red, x);
    const double cb = norm == 0.0f ? 0.0 : (double)P.s / (double)norm;
    if ((j & (G - 1)) == 0 && g0 < P.n) P.norms[g0 >> log2d] = norm;
    const uint32_t key0 = (uint32_t)P.seed, key1 = (uint32_t)(P.seed >> 32);
    int32_t lv[kCPT];
#pragma unroll
    for (int g = 0; g < kCPT / 4; ++g) {
        uint32_t w[4];
        const uint64_t blk = (g0 >> 2) + (uint64_t)g;
        philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), key0, key1, w);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int q = 4 * g + e;
            const int k = (int)qlevel(x[q], cb, w[e]);
            lv[q] = (__float_as_uint(x[q]) >> 31) ? -k : k;
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

// Encode fast path for buckets of d = 2^m coordinates, 16 <= d <= 4096, one
// vector, s <= kTabS. Tile t is the 4096 coordinates from 4096 t (4096 / d whole
// buckets); the G = d / 16 threads of a bucket are consecutive, so each thread's
// 16 coordinates lie in one bucket and thread j starts a bucket iff j mod G = 0.
// Coordinates past n read as 0, which quantize to level 0 and add nothing to a
// norm. Per tile:
//   - bucket sums of squares: fp64 per thread in index order, then an xor
//     butterfly over the bucket's lanes and, for d > 1024, the bucket's waves in
//     wave order through LDS; every thread of a bucket ends with the same sum;
//   - levels and record codes as in the general kernel;
//   - each thread packs its bit string (norm or pending first gap, then its
//     records) into a 64-bit register and ORs full registers into the tile's
//     LDS words, so a thread usually issues two LDS atomics per tile.
__host__ __device__ constexpr size_t aligned_encode_lds_bytes(uint32_t obuf_words, uint32_t s) {
    return align16((size_t)obuf_words * 8) + align16((size_t)code_table_entries(s) * 4);
}

__global__ __launch_bounds__(kWG) void encode_aligned_kernel(QsgdParams P, uint32_t log2d) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ uint32_t sh_tile;
    __shared__ uint64_t sh_base;
    __shared__ int sh_mx[kWaves];
    __shared__ uint32_t sh_bits[kWaves];
    __shared__ double sh_red[kWaves];

    // dynamic LDS: [obuf][rt] (aligned_encode_lds_bytes)
    EncodeLds L{};
    L.obuf = reinterpret_cast<uint64_t *>(smem);
    L.rt = reinterpret_cast<uint32_t *>(smem + align16((size_t)P.obuf_words * 8));
    build_code_table(L.rt, P.s);
    const int j = (int)threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());
    const uint32_t G = 1u << (log2d - 4);      // threads per bucket
    const uint32_t key0 = (uint32_t)P.seed, key1 = (uint32_t)(P.seed >> 32);
    const int x0 = j * kCPT;
    const bool first_of_bucket = (j & (G - 1)) == 0;
    uint32_t Wprev = P.obuf_words;  // words to clear before the first tile

    for (;;) {
        // waits and single-lane sections stay in wave-uniform control flow
        if (wave == 0) {
            uint32_t tk = 0;
            if (lane == 0) tk = atomicAdd(P.ticket, 1u);
            tk = __builtin_amdgcn_readfirstlane(tk);
            if (lane == 0) sh_tile = tk;
        }
        __syncthreads();  // also separates this tile's LDS use from the previous one
        const uint32_t tile = __builtin_amdgcn_readfirstlane(sh_tile);
        if (tile >= P.ntiles) break;
        for (uint32_t w = threadIdx.x; w < Wprev; w += kWG) L.obuf[w] = 0;

        const uint64_t g0 = (uint64_t)tile * kTC + (uint64_t)x0;
        float x[kCPT];
        const float norm = aligned_front(P, g0, G, sh_red, x);
        const double cb = norm == 0.0f ? 0.0 : (double)P.s / (double)norm;
        const bool bstart = first_of_bucket && g0 < P.n;

        // ---- levels and record codes; records packed into two 64-bit
        // registers (coordinates 0-7 and 8-15), right-aligned ----
        uint32_t ec[kCPT];
        uint64_t racc[2] = {0, 0};
        uint32_t rlen[2] = {0, 0};
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
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int q = 4 * g + e;
                const int xi = x0 + q;
                const uint32_t k = qlevel(x[q], cb, w[e]);
                const uint32_t neg = __float_as_uint(x[q]) >> 31;
                const uint32_t gg = have ? (uint32_t)(xi - prev) : 0u;
                const uint32_t ent = L.rt[code_index(gg, k, neg)];
                ec[q] = ent;
                const uint32_t len = ent & 31u;
                racc[q >> 3] = (racc[q >> 3] << len) | (uint64_t)(ent >> 5);
                rlen[q >> 3] += len;
                const bool nz = k != 0u;
                pendx = (nz && !have) ? xi : pendx;
                prev = nz ? xi : prev;
                have = have || nz;
            }
        }
        const uint32_t r = (bstart ? 32u : 0u) + rlen[0] + rlen[1];
        const int marker = have ? prev : INT_MIN;

        // ---- exclusive max-scan of markers: origin of the pending first gap ----
        const int mi = wave_incl_scan(marker, [](int a, int b) { return a > b ? a : b; });
        if (lane == 63) sh_mx[wave] = mi;
        __syncthreads();
        int mpre = INT_MIN;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            if (w < wave) mpre = mpre > sh_mx[w] ? mpre : sh_mx[w];
        int mex = __shfl_up(mi, 1, 64);
        if (lane == 0) mex = INT_MIN;
        mex = mex > mpre ? mex : mpre;
        uint32_t Lp = 0;
        uint64_t pc = 0;
        if (pendx >= 0) pc = omega_code((uint32_t)(pendx - mex), Lp);
        const uint32_t bits = r + Lp;

        // ---- tile scan of bit counts ----
        const uint32_t bi = wave_incl_scan(bits, [](uint32_t a, uint32_t b) { return a + b; });
        if (lane == 63) sh_bits[wave] = bi;
        __syncthreads();
        uint32_t bpre = 0, T = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            if (w < wave) bpre += sh_bits[w];
            T += sh_bits[w];
        }
        uint32_t off = __shfl_up(bi, 1, 64);
        if (lane == 0) off = 0;
        off += bpre;

        // ---- decoupled lookback: stream offset of this tile ----
        if (wave == 0) {
            const uint64_t excl = tile_lookback(P, tile, T);
            if (lane == 0) sh_base = excl;
        }
        __syncthreads();
        const uint64_t base = sh_base;
        const uint32_t head = (uint32_t)(base & 63u);
        const uint32_t W = (head + T + 63u) >> 6;
        const bool last = (tile == P.ntiles - 1);
        if (last && j == 0) {
            P.offsets[P.nb] = base + T;
            *P.out_bits = base + T;
        }

        // ---- phase 2: OR the thread's pieces into the tile's words ----
        uint32_t p = head + off;
        if (bstart) {
            P.offsets[((uint64_t)tile << (12 - log2d)) + ((uint32_t)j >> (log2d - 4))] = base + off;
            or_bits(L.obuf, p, (uint64_t)__float_as_uint(norm) << 32, 32u);
            p += 32u;
        } else if (Lp) {
            or_bits(L.obuf, p, pc << (64u - Lp), Lp);
            p += Lp;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (rlen[h] <= 64u) {
                if (rlen[h]) or_bits(L.obuf, p, racc[h] << (64u - rlen[h]), rlen[h]);
                p += rlen[h];
            } else {
                // more than 64 bits in this half: one record at a time
#pragma unroll
                for (int q = 8 * h; q < 8 * h + 8; ++q) {
                    const uint32_t len = ec[q] & 31u;
                    if (len) or_bits(L.obuf, p, (uint64_t)(ec[q] >> 5) << (64u - len), len);
                    p += len;
                }
            }
        }
        __syncthreads();

        store_tile(P, L.obuf, tile, base, T, W, wave, lane, last);
        Wprev = W;
    }
}

}  // namespace qsgd
