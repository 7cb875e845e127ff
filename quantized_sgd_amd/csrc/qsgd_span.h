// Buckets longer than a tile: the whole-vector operator (d = n) and any
// uniform bucket length over the 4081 coordinates a tile of whole buckets
// holds.
//
// Page "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding":
// the definition paragraph states Q_s for a whole vector v in R^n (bucketing is
// the paper's Section 3.3 extension); the stream and its readings are the same
// as for small buckets.
//
// Tiles are the aligned windows [4096 t, 4096 t + 4096) of the vector, so a
// bucket spans several tiles and a window meets at most three buckets (d > 2048).
//   1. span_norm_partial_kernel: per window, the fp64 sum of squares (or the
//      maximum) of each bucket piece, reduced in a fixed order;
//   2. span_norm_fold_kernel: per bucket, its pieces folded in window order
//      (fixed per-thread strides, then a fixed tree) into RN32(sqrt(sum));
//   3. span_encode_kernel (pass 1): workgroup b codes the windows of its run in
//      order, carrying the last "marker" (a non-zero's index, or a bucket start
//      minus one) from window to window, so the first gap of a window's first
//      record is known unless no marker has been seen in the run yet; that
//      record (at most one per run, always the first of its window's string) is
//      written without its gap code;
//   4. span_pending_kernel: each such run's gap, from the last marker of the
//      runs before it, and its code;
//   5. span_finish_kernel (pass 2): window offsets from the run totals plus the
//      pending codes; each stream word gathered from the windows' strings with
//      a pending code in front of its window's slot bits.
// Quantize takes steps 1-2 and span_quantize_kernel.
#pragma once

#include "qsgd_encode.h"

namespace qsgd {

constexpr int kSpanK = 3;  // buckets that meet one 4096-coordinate window when d > 2048
constexpr uint32_t kMaxRunsPerThread = 16;
constexpr uint32_t kSpanMaxRuns = kWG * kMaxRunsPerThread;  // pass-1 workgroups at most

// The window's geometry: buckets kb0 .. kb0 + K - 1 meet [A, end).
struct SpanWin {
    uint64_t A, end, kb0;
    uint32_t K;
};

__device__ __forceinline__ SpanWin span_window(const QsgdParams &P, uint32_t tile) {
    SpanWin w;
    w.A = (uint64_t)tile << 12;
    w.end = w.A + kTC < P.n ? w.A + kTC : P.n;
    w.kb0 = w.A / P.d;
    w.K = (uint32_t)((w.end - 1) / P.d - w.kb0 + 1);
    return w;
}

// Start of bucket kb0 + k relative to A: -1 when it starts before the window,
// and the window's end for k = K.
__device__ __forceinline__ int span_bucket_start(const QsgdParams &P, const SpanWin &w, uint32_t k) {
    if (k >= w.K) return (int)(w.end - w.A);
    const uint64_t g = (w.kb0 + k) * P.d;
    return g >= w.A ? (int)(g - w.A) : -1;
}

// The window-relative bucket (0 .. K - 1) of window coordinate x.
__device__ __forceinline__ uint32_t span_piece(const int (&bs)[kSpanK + 1], uint32_t K, int x) {
    return (K > 1 && x >= bs[1] ? 1u : 0u) + (K > 2 && x >= bs[2] ? 1u : 0u);
}

// The thread's 16 coordinates of the window (0 past the vector's end).
__device__ __forceinline__ void span_load(const QsgdParams &P, uint64_t g0, float (&x)[kCPT]) {
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

// 1. Per window and bucket piece: the sum of squares (MAXN: the maximum of
// |v_i|), fp64 in index order per thread, then the wave's DPP tree and the
// waves in order.
template <bool MAXN>
__global__ __launch_bounds__(kWG) void span_norm_partial_kernel(QsgdParams P) {
    __shared__ double red[kSpanK][kWaves];
    __shared__ int s_bs[kSpanK + 1];
    auto op = [](double a, double b) { return MAXN ? (a > b ? a : b) : a + b; };
    const uint32_t tile = blockIdx.x;
    const SpanWin w = span_window(P, tile);
    const int j = (int)threadIdx.x;
    if (j <= kSpanK) s_bs[j] = span_bucket_start(P, w, (uint32_t)j);
    float x[kCPT];
    span_load(P, w.A + (uint64_t)j * kCPT, x);
    __syncthreads();
    int bs[kSpanK + 1];
#pragma unroll
    for (int k = 0; k <= kSpanK; ++k) bs[k] = s_bs[k];
    double acc[kSpanK] = {0.0, 0.0, 0.0};
#pragma unroll
    for (int q = 0; q < kCPT; ++q) {
        const int xi = j * kCPT + q;
        const uint32_t k = span_piece(bs, w.K, xi);
        const double y = (double)x[q];
        const double t = MAXN ? fabs(y) : y * y;
        // coordinates past the vector's end are 0 and add nothing
#pragma unroll
        for (uint32_t kk = 0; kk < (uint32_t)kSpanK; ++kk)
            if (kk == k) acc[kk] = MAXN ? op(acc[kk], t) : acc[kk] + t;
    }
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());
#pragma unroll
    for (int k = 0; k < kSpanK; ++k) {
        const double tot = wave_total_f64<MAXN>(acc[k]);
        if (lane_id() == 0) red[k][wave] = tot;
    }
    __syncthreads();
    if (j < (int)w.K) {
        double s = red[j][0];
        for (int v = 1; v < kWaves; ++v) s = op(s, red[j][v]);
        P.sp.partial[(uint64_t)tile * kSpanK + j] = s;
    }
}

// 2. Per bucket: its pieces in window order (thread j takes windows tf + j,
// tf + j + 256, ... in turn), then the threads' values by the wave's DPP tree
// and the waves in order. Writes the bucket norm (and the quantize output).
template <bool MAXN>
__global__ __launch_bounds__(kWG) void span_norm_fold_kernel(QsgdParams P) {
    __shared__ double red[kWaves];
    auto op = [](double a, double b) { return MAXN ? (a > b ? a : b) : a + b; };
    const uint64_t b = blockIdx.x;
    const uint64_t c0 = b * P.d;
    const uint64_t c1 = c0 + P.d < P.n ? c0 + P.d : P.n;
    const uint64_t tf = c0 >> 12, tl = (c1 - 1) >> 12;
    // the bucket's piece in window t: every window after its first one starts
    // inside it, so only the first window needs the division; eight loads in
    // flight per thread, folded in the same order as one at a time
    const uint64_t kf = b - (tf << 12) / P.d;
    double acc = 0.0;
    for (uint64_t t = tf + threadIdx.x; t <= tl; t += 8u * kWG) {
        double pv[8];
#pragma unroll
        for (uint32_t u = 0; u < 8u; ++u) {
            const uint64_t tu = t + (uint64_t)u * kWG;
            pv[u] = tu <= tl ? P.sp.partial[tu * kSpanK + (tu == tf ? kf : 0u)] : 0.0;
        }
#pragma unroll
        for (uint32_t u = 0; u < 8u; ++u)
            if (t + (uint64_t)u * kWG <= tl) acc = op(acc, pv[u]);
    }
    const double tot = wave_total_f64<MAXN>(acc);
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());
    if (lane_id() == 0) red[wave] = tot;
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = red[0];
        for (int v = 1; v < kWaves; ++v) s = op(s, red[v]);
        const float norm = MAXN ? (float)s : (float)sqrt(s);
        P.sp.norms[b] = norm;
        if (P.norms) P.norms[b] = norm;
    }
}

// The window's bucket constants in LDS: norms, ratio scales (negated: midpoint test)
// and bucket starts.
__device__ __forceinline__ void span_constants(const QsgdParams &P, const SpanWin &w, float *s_nrm,
                                               double *s_cb, int *s_bs) {
    const uint32_t j = threadIdx.x;
    if (j < w.K) {
        const float norm = P.sp.norms[w.kb0 + j];
        s_nrm[j] = norm;
        s_cb[j] = ratio_may_tie(norm, P.sigma) ? -ratio_scale(norm, P.s) : ratio_scale(norm, P.s);
    }
    if (j <= (uint32_t)kSpanK) s_bs[j] = span_bucket_start(P, w, j);
}

// Levels of the thread's 16 coordinates (k = 0 past the vector's end).
__device__ __forceinline__ void span_levels(const QsgdParams &P, const SpanWin &w, const float (&x)[kCPT],
                                            const float *s_nrm, const double *s_cb, const int (&bs)[kSpanK + 1],
                                            uint32_t (&k)[kCPT], uint32_t &neg) {
    const int j = (int)threadIdx.x;
    const uint32_t key0 = (uint32_t)P.seed, key1 = (uint32_t)(P.seed >> 32);
    const uint64_t blk0 = (w.A >> 2) + (uint64_t)j * (kCPT / 4);
    neg = 0;
#pragma unroll
    for (int g = 0; g < kCPT / 4; ++g) {
        uint32_t wd[4];
        const uint64_t blk = blk0 + (uint64_t)g;
        philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), key0, key1, wd);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int q = 4 * g + e;
            const int xi = j * kCPT + q;
            uint32_t kk = 0;
            if (w.A + (uint64_t)xi < w.end) {
                const uint32_t b = span_piece(bs, w.K, xi);
                const double cb = s_cb[b];
                kk = level_of_ratio(ratio_of(x[q], fabs(cb), cb < 0.0, s_nrm[b], P.s), wd[e]);
                if (__float_as_uint(x[q]) >> 31) neg |= 1u << q;
            }
            k[q] = kk;
        }
    }
}

// Quantize with the folded norms: levels sgn * k of every window.
__global__ __launch_bounds__(kWG) void span_quantize_kernel(QsgdParams P) {
    __shared__ float s_nrm[kSpanK];
    __shared__ double s_cb[kSpanK];
    __shared__ int s_bs[kSpanK + 1];
    const SpanWin w = span_window(P, blockIdx.x);
    const int j = (int)threadIdx.x;
    span_constants(P, w, s_nrm, s_cb, s_bs);
    const uint64_t g0 = w.A + (uint64_t)j * kCPT;
    float x[kCPT];
    span_load(P, g0, x);
    __syncthreads();
    int bs[kSpanK + 1];
#pragma unroll
    for (int k = 0; k <= kSpanK; ++k) bs[k] = s_bs[k];
    uint32_t k[kCPT], neg;
    span_levels(P, w, x, s_nrm, s_cb, bs, k, neg);
    if (g0 + kCPT <= P.n) {
        int4 *dst = reinterpret_cast<int4 *>(P.levels + g0);
#pragma unroll
        for (int q = 0; q < kCPT / 4; ++q) {
            int4 o;
            o.x = (neg >> (4 * q + 0)) & 1 ? -(int)k[4 * q + 0] : (int)k[4 * q + 0];
            o.y = (neg >> (4 * q + 1)) & 1 ? -(int)k[4 * q + 1] : (int)k[4 * q + 1];
            o.z = (neg >> (4 * q + 2)) & 1 ? -(int)k[4 * q + 2] : (int)k[4 * q + 2];
            o.w = (neg >> (4 * q + 3)) & 1 ? -(int)k[4 * q + 3] : (int)k[4 * q + 3];
            dst[q] = o;
        }
    } else {
#pragma unroll
        for (int q = 0; q < kCPT; ++q)
            if (g0 + q < P.n) P.levels[g0 + q] = (neg >> q) & 1 ? -(int)k[q] : (int)k[q];
    }
}

// 3. Pass 1 over the windows of each run (see the file comment). Dynamic LDS:
// the window's bit-string words.
template <bool TABLE>
__global__ __launch_bounds__(kWG) void span_encode_kernel(QsgdParams P) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int sh_mx[kWaves];
    __shared__ uint32_t sh_bits[kWaves];
    __shared__ float s_nrm[kSpanK];
    __shared__ double s_cb[kSpanK];
    __shared__ int s_bs[kSpanK + 1];
    __shared__ uint64_t s_pend;
    __shared__ uint32_t s_pend_tile;
    uint64_t *obuf = reinterpret_cast<uint64_t *>(smem);
    const uint32_t *rt = P.code ? kCodeTableGamma.e : kCodeTableOmega.e;
    const int j = (int)threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());
    if (j == 0) {
        s_pend = ~0ull;
        s_pend_tile = 0;
    }
    // absolute index + 2 of the run's latest marker so far (0: none yet; a
    // marker can be -1, the start of bucket 0 minus one); the same value on
    // every thread
    uint64_t carry = 0;
    uint64_t run_total = 0;
    const uint32_t tend = run_first(blockIdx.x + 1, P.run, P.rem);
    for (uint32_t tile = run_first(blockIdx.x, P.run, P.rem); tile < tend; ++tile) {
        __syncthreads();  // separates this window's LDS use from the previous one
        const SpanWin w = span_window(P, tile);
        span_constants(P, w, s_nrm, s_cb, s_bs);
        const int x0 = j * kCPT;
        float x[kCPT];
        span_load(P, w.A + (uint64_t)x0, x);
        __syncthreads();
        int bs[kSpanK + 1];
#pragma unroll
        for (int k = 0; k <= kSpanK; ++k) bs[k] = s_bs[k];
        uint32_t lv[kCPT], neg;
        span_levels(P, w, x, s_nrm, s_cb, bs, lv, neg);

        // ---- records: codes and lengths; markers ----
        uint32_t ec[kCPT];
        uint64_t ecx[kCPT];
        uint32_t bst = 0;
        uint32_t r = 0;
        int prev = 0, pendx = -1;
        int have = 0;
#pragma unroll
        for (int q = 0; q < kCPT; ++q) {
            const int xi = x0 + q;
            const bool valid = w.A + (uint64_t)xi < w.end;
            const uint32_t b = span_piece(bs, w.K, xi);
            if (valid && xi == bs[b]) {
                bst |= 1u << q;
                r += 32u;
                prev = xi - 1;
                have = 1;
            }
            const uint32_t k = lv[q];
            const uint32_t g = have ? (uint32_t)(xi - prev) : 0u;
            uint64_t code;
            const uint32_t len = record_entry<TABLE>(rt, g, k, (neg >> q) & 1u, code, P.code);
            ec[q] = len;
            ecx[q] = code;
            r += len;
            if (k) {
                if (!have) pendx = xi;
                prev = xi;
                have = 1;
            }
            // markers formed four coordinates at a time, not left to sink below
            // the loop with 16 lane masks live in SGPRs
            if ((q & 3) == 3) asm volatile("" : "+v"(pendx), "+v"(prev), "+v"(have));
        }
        const int marker = have ? prev : INT_MIN;

        // ---- exclusive max-scan of markers, the window's last marker ----
        const int mi = wave_incl_max_i32(marker);
        if (lane == 63) sh_mx[wave] = mi;
        __syncthreads();
        int mpre = INT_MIN, mtot = INT_MIN;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            if (v < wave) mpre = mpre > sh_mx[v] ? mpre : sh_mx[v];
            mtot = mtot > sh_mx[v] ? mtot : sh_mx[v];
        }
        int mex = wave_shr1_i32(INT_MIN, mi);
        mex = mex > mpre ? mex : mpre;
        uint32_t Lp = 0;
        uint64_t pc = 0;
        if (pendx >= 0) {
            if (mex != INT_MIN) {
                pc = field_code(P.code, (uint32_t)(pendx - mex), Lp);
            } else if (carry != 0) {
                pc = field_code(P.code, (uint32_t)(w.A + (uint64_t)pendx + 2 - carry), Lp);
            } else {
                // the run's first record of a bucket that started before the run
                s_pend = w.A + (uint64_t)pendx;
                s_pend_tile = tile;
            }
        }
        if (mtot != INT_MIN) carry = w.A + (uint64_t)((int64_t)mtot + 2);
        const uint32_t bits = r + Lp;

        // ---- window scan of bit counts ----
        const uint32_t bi = wave_incl_add_u32(bits);
        if (lane == 63) sh_bits[wave] = bi;
        __syncthreads();
        uint32_t bpre = 0, T = 0;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            if (v < wave) bpre += sh_bits[v];
            T += sh_bits[v];
        }
        const uint32_t off = (uint32_t)wave_shr1_i32(0, (int)bi) + bpre;
        const uint32_t W = (T + 63u) >> 6;
        for (uint32_t wd = threadIdx.x; wd <= W; wd += kWG) obuf[wd] = 0;
        __syncthreads();

        // ---- OR every piece into the window's words ----
        uint32_t p = off;
        if (Lp) or_bits(obuf, p, pc << (64u - Lp), Lp);
        p += Lp;
#pragma unroll
        for (int q = 0; q < kCPT; ++q) {
            if ((bst >> q) & 1u) {
                const uint32_t b = span_piece(bs, w.K, x0 + q);
                P.offsets[w.kb0 + b] = p;  // window-relative; pass 2 adds the window's offset
                or_bits(obuf, p, (uint64_t)__float_as_uint(s_nrm[b]) << 32, 32u);
                p += 32u;
            }
            if (ec[q]) or_bits(obuf, p, ecx[q] << (64u - ec[q]), ec[q]);
            p += ec[q];
        }
        __syncthreads();

        uint64_t *slot = P.slots + (uint64_t)tile * P.obuf_words;
        for (uint32_t wd = threadIdx.x; wd < W; wd += kWG) slot[wd] = obuf[wd];
        if (j == 0) P.tile_bits[tile] = T;
        run_total += T;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        P.run_bits[blockIdx.x] = run_total;
        P.sp.run_mark[blockIdx.x] = carry;
        P.sp.run_pend[blockIdx.x] = s_pend;
        P.sp.run_pend_tile[blockIdx.x] = s_pend_tile;
    }
}

// 4. One workgroup: for every run with a pending record, its gap from the last
// marker of the runs before it (markers only grow with the run index), and
// the gap's code. Thread j takes runs [16 j, 16 j + 16).
__global__ __launch_bounds__(kWG) void span_pending_kernel(QsgdParams P, uint32_t runs) {
    __shared__ uint64_t tot[kWG];
    const uint32_t j = threadIdx.x;
    constexpr uint32_t kPer = kMaxRunsPerThread;
    uint64_t m[kPer];
    uint64_t mx = 0;  // marker + 2; 0: none
#pragma unroll
    for (uint32_t i = 0; i < kPer; ++i) {
        const uint32_t r = j * kPer + i;
        m[i] = r < runs ? P.sp.run_mark[r] : 0;
        mx = m[i] > mx ? m[i] : mx;
    }
    tot[j] = mx;
    __syncthreads();
    uint64_t before = 0;
    for (uint32_t v = 0; v < j; ++v) before = tot[v] > before ? tot[v] : before;
#pragma unroll
    for (uint32_t i = 0; i < kPer; ++i) {
        const uint32_t r = j * kPer + i;
        if (r < runs) {
            const uint64_t pend = P.sp.run_pend[r];
            uint32_t L = 0;
            uint64_t code = 0;
            if (pend != ~0ull && before != 0)
                code = field_code(P.code, (uint32_t)(pend + 2 - before), L);
            P.sp.lp[r] = L;
            P.sp.pc[r] = code;
        }
        before = m[i] > before ? m[i] : before;
    }
}

// 5. Pass 2 of the span path. Workgroup w takes windows [t0, t1) (8 of them).
struct SpanFinishParams {
    FinishParams F;
    SpanParams sp;
    uint64_t n;
    uint32_t d;
};

// A window's string: its pending code (Lp bits, if its run's pending record is
// its first record) in front of its slot bits.
struct SpanStr {
    uint32_t Lp;
    uint64_t pc;
    uint32_t T;  // length with the pending code
};

__device__ __forceinline__ SpanStr span_str(const SpanFinishParams &S, uint32_t tt) {
    const uint32_t r = run_of(tt, S.F.run, S.F.rem);
    SpanStr v;
    const bool pend = S.sp.run_pend[r] != ~0ull && S.sp.run_pend_tile[r] == tt;
    v.Lp = pend ? S.sp.lp[r] : 0u;
    v.pc = pend ? S.sp.pc[r] : 0ull;
    v.T = S.F.tile_bits[tt] + v.Lp;
    return v;
}

// `take` (1..64) bits of window tt's string from bit rel on, at the top.
__device__ __forceinline__ uint64_t span_str_bits(const SpanFinishParams &S, uint32_t tt, const SpanStr &v,
                                                  uint32_t rel, uint32_t take) {
    uint64_t x;
    if (rel >= v.Lp) {
        x = slot_bits(S.F, tt, rel - v.Lp, 64u);
    } else {
        const uint32_t pl = v.Lp - rel;  // pending bits still to come (1..63)
        x = (v.pc << (64u - v.Lp)) << rel;
        x |= slot_bits(S.F, tt, 0u, 64u) >> pl;
    }
    return take >= 64u ? x : (x & ~(~0ull >> take));
}

__global__ __launch_bounds__(kWG) void span_finish_kernel(SpanFinishParams S) {
    __shared__ uint64_t sh_base[kFinishTiles + 1];
    __shared__ uint64_t sh_red[kWaves];
    __shared__ uint64_t sh_scan[kWaves];
    const FinishParams &F = S.F;
    const uint32_t t0 = blockIdx.x * F.chunk;
    const uint32_t t1 = t0 + F.chunk < F.ntiles ? t0 + F.chunk : F.ntiles;
    if (t0 >= t1) return;
    const int j = (int)threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());

    // offset of t0: the runs before t0's run with their pending codes, then the
    // windows of that run before t0
    const uint32_t r0 = run_of(t0, F.run, F.rem);
    const uint32_t m = t1 - t0;
    const uint64_t mine = (uint32_t)j < m ? (uint64_t)span_str(S, t0 + j).T : 0ull;
    uint64_t acc = 0;
    // (eight pairs of loads in flight per thread)
    for (uint32_t i = (uint32_t)j; i < r0; i += 8u * kWG) {
        uint64_t rb[8];
        uint32_t lp[8];
#pragma unroll
        for (uint32_t u = 0; u < 8u; ++u) {
            const bool in = i + u * kWG < r0;
            rb[u] = in ? F.run_bits[i + u * kWG] : 0ull;
            lp[u] = in ? S.sp.lp[i + u * kWG] : 0u;
        }
#pragma unroll
        for (uint32_t u = 0; u < 8u; ++u) acc += rb[u] + lp[u];
    }
    for (uint32_t t = run_first(r0, F.run, F.rem) + (uint32_t)j; t < t0; t += kWG) acc += span_str(S, t).T;
    acc = wave_incl_add_u64(acc);
    if (lane == 63) sh_red[wave] = acc;
    __syncthreads();
    uint64_t pre = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) pre += sh_red[v];
    uint64_t total = 0;
    const uint64_t ex = block_excl_add_u64(mine, sh_scan, total);
    if ((uint32_t)j < m) sh_base[j] = pre + ex;
    if (j == 0) sh_base[m] = pre + total;
    __syncthreads();

    // every stream word whose first bit lies in this share's windows
    const uint64_t wbeg = (sh_base[0] + 63) >> 6, wend = (sh_base[m] + 63) >> 6;
    for (uint64_t wd = wbeg + (uint64_t)j; wd < wend; wd += kWG) {
        const uint64_t g = wd << 6;
        uint32_t i = 0;
        while (sh_base[i + 1] <= g) ++i;
        uint32_t tt = t0 + i;
        uint32_t rel = (uint32_t)(g - sh_base[i]);
        uint64_t v = 0;
        uint32_t have = 0;
        while (have < 64u && tt < F.ntiles) {
            const SpanStr st = span_str(S, tt);
            if (rel < st.T) {
                const uint32_t take = 64u - have < st.T - rel ? 64u - have : st.T - rel;
                v |= span_str_bits(S, tt, st, rel, take) >> have;
                have += take;
            }
            ++tt;
            rel = 0;
        }
        F.out[wd] = v;
    }
    // bucket offsets of buckets starting in this share's windows
    const uint64_t c_lo = (uint64_t)t0 << 12;
    const uint64_t c_hi = ((uint64_t)t1 << 12) < S.n ? ((uint64_t)t1 << 12) : S.n;
    const uint64_t b_lo = (c_lo + S.d - 1) / S.d;
    const uint64_t b_hi = (c_hi + S.d - 1) / S.d < F.nb ? (c_hi + S.d - 1) / S.d : F.nb;
    for (uint64_t b = b_lo + (uint64_t)j; b < b_hi; b += kWG) {
        const uint32_t tt = (uint32_t)((b * S.d) >> 12);
        F.offsets[b] += sh_base[tt - t0] + span_str(S, tt).Lp;
    }
    if (t1 == F.ntiles && j == 0) {
        F.offsets[F.nb] = sh_base[m];
        *F.out_bits = sh_base[m];
    }
}

}  // namespace qsgd
