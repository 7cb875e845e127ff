// Front half of a tile, shared by the quantize and encode kernels: tile geometry,
// the load of v, per-bucket L2 norms, and the stochastic rounding.
//
// Page "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding":
// definition paragraph (||v||_2, l_i, p_i, the rounding) and the claim on
// bucketed training (paper Section 3.3: Q_s per bucket of d coordinates).
//
// A tile is a run of whole buckets [b0, b1) covering coordinates [c0, c1) with
// c1 - (c0 & ~15) <= 4096. Thread j owns the 16 coordinates starting at
// A + 16 j, A = c0 & ~15, so Philox blocks (4 coordinates) never straddle
// threads and the loads are 16-byte aligned.
#pragma once

#include "qsgd_device.h"

namespace qsgd {

// Workspace of the path for buckets longer than a tile (qsgd_span.h).
struct SpanParams {
    double *partial;          // [ntiles][3] per-window partial sums (or maxima) of bucket pieces
    float *norms;             // [nb] bucket norms
    uint64_t *run_pend;       // [runs] index of the run's pending record, or ~0
    uint32_t *run_pend_tile;  // [runs] its window
    uint64_t *run_mark;       // [runs] index + 2 of the run's last marker, or 0
    uint32_t *lp;             // [runs] length of the pending record's gap code (0: none)
    uint64_t *pc;             // [runs] that code, right-aligned
};

struct QsgdParams {
    const float *v;
    uint64_t n;
    uint64_t nb;
    const uint64_t *bstart;  // ragged bucket table (device), or nullptr
    uint64_t seed;
    uint32_t s;
    uint32_t d;
    uint32_t K;        // buckets per tile
    uint32_t ntiles;
    // quantize outputs
    int32_t *levels;
    float *norms;
    // encode outputs (bucket offsets are tile-relative after the first pass)
    uint64_t *offsets;
    // encode workspace: each tile's bit string from bit 0 of its slot, and its
    // length in bits
    uint64_t *slots;       // [ntiles][obuf_words]
    uint32_t *tile_bits;   // [ntiles]
    uint64_t *run_bits;    // [gridDim.x] total bits of each workgroup's run of tiles
    uint32_t obuf_words;   // words of a tile's bit string bound (+1 spare)
    uint32_t run, rem;     // workgroup b takes run_first(b) .. run_first(b + 1) - 1
    uint32_t code;         // integer code of gaps and levels: 0 Elias omega, 1 Elias gamma
    uint32_t maxnorm;      // bucket scale: 0 the L2 norm, 1 the max-norm max|v_i| (QSGDinf)
    uint32_t sigma;        // odd part of s (ratio_may_tie)
    SpanParams sp;         // buckets longer than a tile only
    SegTable seg;          // ragged layout by tensor lengths (nseg > 0) instead of bstart
};

// Runs of consecutive tiles: the first `rem` workgroups take run + 1 tiles, the
// others run tiles.
__host__ __device__ __forceinline__ uint32_t run_first(uint32_t b, uint32_t run, uint32_t rem) {
    return b * run + (b < rem ? b : rem);
}

// The run that holds tile t.
__host__ __device__ __forceinline__ uint32_t run_of(uint32_t t, uint32_t run, uint32_t rem) {
    const uint32_t big = (run + 1) * rem;
    return t < big ? t / (run + 1) : rem + (t - big) / run;
}

// LDS carved out of the dynamic shared memory block for the front half.
struct FrontLds {
    int32_t *bs;      // [K + 1] bucket starts relative to A
    double *cb;       // [K] sum of squares, then ratio_scale(norm, s), negated where
                      // the bucket's ratios take the midpoint test (ratio_may_tie)
    float *nrm;       // [K] norms
    double *segv;     // [kWaves] scan scratch
    int *segf;        // [kWaves]
};

struct Tile {
    uint64_t b0, b1, c0, c1, A;
    int lo, hi;       // valid range relative to A
    uint32_t K;       // buckets in this tile
};

template <bool RAGGED>
__device__ __forceinline__ Tile tile_geometry(const QsgdParams &P, uint32_t tile) {
    Tile t;
    t.b0 = (uint64_t)tile * P.K;
    t.b1 = t.b0 + P.K < P.nb ? t.b0 + P.K : P.nb;
    if (RAGGED) {
        t.c0 = ragged_start(P.bstart, P.seg, t.b0);
        t.c1 = ragged_start(P.bstart, P.seg, t.b1);
    } else {
        t.c0 = t.b0 * P.d;
        const uint64_t e = t.b1 * P.d;
        t.c1 = e < P.n ? e : P.n;
    }
    t.A = t.c0 & ~(uint64_t)15;
    t.lo = (int)(t.c0 - t.A);
    t.hi = (int)(t.c1 - t.A);
    t.K = (uint32_t)(t.b1 - t.b0);
    return t;
}

template <bool RAGGED>
__device__ __forceinline__ void fill_bucket_starts(const QsgdParams &P, const Tile &t, FrontLds &L) {
    for (uint32_t k = threadIdx.x; k <= t.K; k += kWG) {
        uint64_t g;
        if (RAGGED) {
            g = ragged_start(P.bstart, P.seg, t.b0 + k);
        } else {
            g = (t.b0 + k) * P.d;
            if (g > P.n) g = P.n;
        }
        L.bs[k] = (int32_t)(g - t.A);
    }
}

// Per-thread state after the front half.
struct ThreadCoords {
    float x[kCPT];
    int vx0, vx1;   // valid coordinates [vx0, vx1) relative to A (vx0 >= vx1: none)
    int kf;         // tile-local bucket of coordinate vx0
};

// Loads the thread's 16 coordinates (16-byte vector loads when fully in range).
__device__ __forceinline__ void load_coords(const QsgdParams &P, const Tile &t, ThreadCoords &c) {
    const int j = (int)threadIdx.x;
    const int x0 = j * kCPT;
    c.vx0 = x0 > t.lo ? x0 : t.lo;
    c.vx1 = x0 + kCPT < t.hi ? x0 + kCPT : t.hi;
    const uint64_t g0 = t.A + (uint64_t)x0;
    if (c.vx0 < c.vx1) {
        if (g0 + kCPT <= P.n) {
            const float4 *p = reinterpret_cast<const float4 *>(P.v + g0);
#pragma unroll
            for (int q = 0; q < kCPT / 4; ++q) {
                const float4 f = p[q];
                c.x[4 * q + 0] = f.x;
                c.x[4 * q + 1] = f.y;
                c.x[4 * q + 2] = f.z;
                c.x[4 * q + 3] = f.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < kCPT; ++q) c.x[q] = (g0 + q < P.n) ? P.v[g0 + q] : 0.0f;
        }
    } else {
#pragma unroll
        for (int q = 0; q < kCPT; ++q) c.x[q] = 0.0f;
    }
}

template <bool RAGGED>
__device__ __forceinline__ int first_bucket(const QsgdParams &P, const Tile &t, const FrontLds &L,
                                            int x) {
    if (!RAGGED) return (x - t.lo) / (int)P.d;
    int lo = 0, hi = (int)t.K - 1;  // largest k with bs[k] <= x
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (L.bs[mid] <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Per-bucket norms. Each thread sums its coordinates' squares in fp64 in index
// order per bucket segment; buckets that span threads are combined with a
// segmented scan in thread order. The order is fixed, so results are
// reproducible; it differs from a plain left-to-right sum only in rounding.
// Afterwards L.nrm[k] = RN32(sqrt(sum)) and L.cb[k] = RD64(s / norm) (0 for a
// zero bucket; negated for a bucket whose ratios take the midpoint test, see
// ratio_may_tie and ratio_tiefix). MAXN: the max-norm max|v_i| instead (exact, in any order).
// Ends with a barrier.
template <bool RAGGED, bool MAXN = false>
__device__ __forceinline__ void bucket_norms(const QsgdParams &P, const Tile &t, FrontLds &L,
                                             ThreadCoords &c) {
    const int j = (int)threadIdx.x;
    double acc = 0.0, head = 0.0;
    int head_done = 0, cur_fresh = 0, cur_first = 1, k = 0, nbnd = 0x7fffffff;
    const bool active = c.vx0 < c.vx1;
    if (active) {
        c.kf = first_bucket<RAGGED>(P, t, L, c.vx0);
        k = c.kf;
        nbnd = L.bs[k + 1];
        cur_fresh = (L.bs[k] == c.vx0);
    } else {
        c.kf = 0;
    }
#pragma unroll
    for (int q = 0; q < kCPT; ++q) {
        const int x = j * kCPT + q;
        if (x >= c.vx0 && x < c.vx1) {
            if (x == nbnd) {
                if (cur_first && !cur_fresh) { head = acc; head_done = 1; }
                else L.cb[k] = acc;  // bucket started and ended inside this thread
                acc = 0.0;
                ++k;
                nbnd = L.bs[k + 1];
                cur_fresh = 1;
                cur_first = 0;
            }
            const double y = (double)c.x[q];
            if (MAXN) acc = acc > fabs(y) ? acc : fabs(y);
            else acc = acc + y * y;
        }
    }
    const int ends_here = active && (nbnd == c.vx1);
    if (active && ends_here && cur_fresh) L.cb[k] = acc;
    // scan element: the last segment (flag: it starts a bucket)
    const double ex = block_seg_excl_sum<MAXN>(active ? acc : 0.0, active ? cur_fresh : 0, L.segv, L.segf);
    auto join = [](double a, double b) { return MAXN ? (a > b ? a : b) : a + b; };
    if (head_done) L.cb[c.kf] = join(ex, head);
    else if (active && cur_first && !cur_fresh && ends_here) L.cb[k] = join(ex, acc);
    __syncthreads();
    for (uint32_t b = threadIdx.x; b < t.K; b += kWG) {
        const float nr = MAXN ? (float)L.cb[b] : (float)sqrt(L.cb[b]);
        L.nrm[b] = nr;
        L.cb[b] = ratio_may_tie(nr, P.sigma) ? -ratio_scale(nr, P.s) : ratio_scale(nr, P.s);
    }
    __syncthreads();
}

// Stochastic rounding of the thread's coordinates. Outputs the levels k (0 for
// invalid coordinates), the sign / non-zero / bucket-start masks (bit q for
// coordinate A + 16 j + q).
struct ThreadLevels {
    uint32_t k[kCPT];
    uint32_t neg, nz, bst;
};

__device__ __forceinline__ void quantize_coords(const QsgdParams &P, const Tile &t, const FrontLds &L,
                                                const ThreadCoords &c, ThreadLevels &o) {
    const int j = (int)threadIdx.x;
    const uint32_t key0 = (uint32_t)P.seed, key1 = (uint32_t)(P.seed >> 32);
    const uint64_t blk0 = (t.A >> 2) + (uint64_t)j * (kCPT / 4);
    o.neg = 0; o.nz = 0; o.bst = 0;
    const bool active = c.vx0 < c.vx1;
    int k = c.kf;
    int nbnd = active ? L.bs[k + 1] : 0x7fffffff;
    double cb = active ? L.cb[k] : 0.0;
    if (active && L.bs[k] == c.vx0) o.bst |= 1u << (c.vx0 - j * kCPT);
#pragma unroll
    for (int g = 0; g < kCPT / 4; ++g) {
        uint32_t w[4];
        const uint64_t blk = blk0 + (uint64_t)g;
        philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), key0, key1, w);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int q = 4 * g + e;
            const int x = j * kCPT + q;
            uint32_t kk = 0;
            if (x >= c.vx0 && x < c.vx1) {
                if (x == nbnd) {
                    ++k;
                    nbnd = L.bs[k + 1];
                    cb = L.cb[k];
                    o.bst |= 1u << q;
                }
                kk = level_of_ratio(ratio_of(c.x[q], fabs(cb), cb < 0.0, L.nrm[k], P.s),
                                    w[e]);
                if (__float_as_uint(c.x[q]) >> 31) o.neg |= 1u << q;
            }
            o.k[q] = kk;
            if (kk) o.nz |= 1u << q;
        }
    }
}

}  // namespace qsgd
