// Device-side building blocks of the QSGD compressor for gfx950 (CDNA4, wave64).
//
// Method: page "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding",
// definition paragraph (Q_s, Elias recursive coding of the quantized tuple) and
// its claims on Elias coding (F = 32 bit norm) and bucketed training (paper
// Section 3.3). The exact floating-point and stream-layout readings are stated in
// include/qsgd.h and repeated at each helper below.
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

namespace qsgd {

constexpr int kWG = 256;           // threads per workgroup: 4 wave64
constexpr int kWaves = kWG / 64;
constexpr int kCPT = 16;           // contiguous coordinates per thread
constexpr int kTC = kWG * kCPT;    // coordinates per tile (4096)
constexpr int kKMax = 512;         // buckets per tile at most

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32->64
// multiplies with the round key bumped by the Weyl constants after each round.
// Counter words 2 and 3 are zero in this library (the counter is the 64-bit
// block index i >> 2), so the first round's second product is 0. The two
// three-way XORs of a round are single v_bitop3_b32 instructions on gfx950
// (truth table 0x96 = a ^ b ^ c).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t k0,
                                              uint32_t k1, uint32_t (&o)[4]) {
    uint32_t x0 = c0, x1 = c1, x2 = 0u, x3 = 0u;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * x0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
        const uint32_t y0 = xor3((uint32_t)(p1 >> 32), x1, k0);
        const uint32_t y2 = xor3((uint32_t)(p0 >> 32), x3, k1);
        x1 = (uint32_t)p1;
        x3 = (uint32_t)p0;
        x0 = y0;
        x2 = y2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    o[0] = x0; o[1] = x1; o[2] = x2; o[3] = x3;
}

// The ratio r = RN32(s |v| / norm) of the page's l and p, the binary32 value
// nearest to the exact quotient (ties to even). Fast form: r = RN32(|v| * c)
// with c = RD64(s / norm), the fp64 quotient rounded toward zero, per bucket.
// Exactness of the fast form. The fp64 value |v| c lies within 2^-51 (relative)
// of the exact quotient q and never above it when q is an fp64 number. With
// |v| = alpha 2^ea, norm = nu 2^en (alpha, nu < 2^24) and s <= 2^24, q differs
// from any number M = mu 2^em with mu < 2^25 (an fp32 rounding boundary) by
// more than 2^-49 relative unless q = M exactly, since s |v| - M norm is a
// non-zero multiple of 2^min(ea, em + en) then. So RN32 agrees unless q is
// exactly a boundary:
//  - q = 2^-150 (half the least subnormal, which rounds to 0): |v| c <= q
//    then, so the fast form gives 0 as well;
//  - other boundaries of the subnormal range: both neighbours are positive and
//    below 2^-126, where the decision u < p is the same for both;
//  - a midpoint of the normal range (25-bit odd mu): the odd parts of s, |v| and
//    norm then satisfy sigma alpha' = mu nu' with alpha' < 2^24 < mu, so the odd
//    part of norm's significand is below the odd part sigma of s. In a bucket
//    where that can happen (never for s a power of two) |v| c may fall just below
//    q = M and round to the neighbour below, where the correct rounding takes the
//    even one of the two; ratio_tiefix tests for exactly that case.
__device__ __forceinline__ double ratio_scale(float norm, uint32_t s) {
    if (norm == 0.0f) return 0.0;
    const double q = (double)s / (double)norm;                 // RN64
    const double rem = __builtin_fma(q, (double)norm, -(double)s);  // exact: q norm - s
    return rem > 0.0 ? __longlong_as_double(__double_as_longlong(q) - 1) : q;
}

// True when the ratio of some coordinate of a bucket with this norm can be an
// exact fp32 midpoint: the odd part of norm's integer significand is below
// sigma, the odd part of s (norm > 0).
__device__ __forceinline__ bool ratio_may_tie(float norm, uint32_t sigma) {
    if (norm == 0.0f) return false;
    const uint32_t b = __float_as_uint(norm);
    uint32_t m = b & 0x7fffffu;
    if (b >> 23) m |= 0x800000u;
    return (m >> __builtin_ctz(m)) < sigma;
}

// The fast form of the signed ratio: sign of v, magnitude RN32(|v| c).
__device__ __forceinline__ float ratio_fast(float v, double c) { return (float)((double)v * c); }

// The fast form r = ratio_fast(v, c) corrected at exact midpoints (a bucket
// where ratio_may_tie): with a = |r| and a+ the next binary32 value above it,
// q = s |v| / norm is the midpoint M = (a + a+) / 2 exactly when s |v| = M norm,
// a comparison of two exact fp64 products (48 and 49 significant bits); then
// the correct rounding is the one of a, a+ with an even significand.
__device__ __forceinline__ float ratio_tiefix(float v, float r, float norm, uint32_t s) {
    const float a = fabsf(r);
    const float up = __uint_as_float(__float_as_uint(a) + 1u);
    const double M = ((double)a + (double)up) * 0.5;  // exact
    const bool tie = (double)s * (double)fabsf(v) == M * (double)norm;
    const float m = (tie && (__float_as_uint(a) & 1u)) ? up : a;
    return __builtin_copysignf(m, v);
}

// The signed ratio of a coordinate: c = ratio_scale, tie = ratio_may_tie.
__device__ __forceinline__ float ratio_of(float v, double c, bool tie, float norm, uint32_t s) {
    const float r = ratio_fast(v, c);
    return tie ? ratio_tiefix(v, r, norm, s) : r;
}

// Level k from the signed ratio r of a coordinate: l = floor(|r|),
// p = |r| - l (exact), uniform u = (w >> 8) 2^-24, k = l + [u < p]. Each
// operation is one IEEE op (the library is built with -ffp-contract=off).
__device__ __forceinline__ uint32_t level_of_ratio(float r, uint32_t w) {
    const float a = fabsf(r);
    // a >= 0: truncation is the floor, and fract gives a - floor(a) exactly
    const uint32_t l = (uint32_t)a;
    const float p = __builtin_amdgcn_fractf(a);
    const float u = (float)(w >> 8) * 0x1p-24f;
    return l + (u < p ? 1u : 0u);
}

// Level of one coordinate of a bucket (c = ratio_scale, tie = ratio_may_tie).
__device__ __forceinline__ uint32_t qlevel(float v, double c, bool tie, float norm, uint32_t s,
                                           uint32_t w) {
    return level_of_ratio(ratio_of(v, c, tie, norm, s), w);
}

// Odd part of s.
__host__ __device__ __forceinline__ uint32_t odd_part(uint32_t s) {
    while (s && !(s & 1u)) s >>= 1;
    return s;
}

// Dequantized magnitude RN32(norm k / s), the binary32 value nearest to the exact
// quotient: norm k is exact in fp64, so the fp64 quotient rounded to fp32 is it.
// For s a power of two (pow2) the quotient norm / s is exact and a product serves.
__device__ __forceinline__ float dequant_value(double norm, uint32_t k, uint32_t s, bool pow2,
                                               double inv_s) {
    return pow2 ? (float)((double)k * (norm * inv_s)) : (float)(((double)k * norm) / (double)s);
}

// Elias omega codeword of N >= 1 (Elias 1975), right-aligned: a final 0 bit, and
// in front of it the binary forms of N, floor(log2 N), ... while the value is > 1.
// At most 43 bits for N < 2^32.
__device__ __forceinline__ uint64_t omega_code(uint32_t N, uint32_t &len) {
    uint64_t code = 0;
    uint32_t L = 1;
    uint32_t m = N;
    while (m > 1u) {
        const uint32_t b = 32u - (uint32_t)__clz(m);
        code |= (uint64_t)m << L;
        L += b;
        m = b - 1u;
    }
    len = L;
    return code;
}

// Elias gamma codeword of N >= 1 (Elias 1975), right-aligned: floor(log2 N) zero
// bits, then N in binary; that is the value N in 2 floor(log2 N) + 1 bits.
__device__ __forceinline__ uint64_t gamma_code(uint32_t N, uint32_t &len) {
    len = 2u * (32u - (uint32_t)__clz(N)) - 1u;
    return N;
}

// Codeword of a record field (gap or level): Elias omega (code 0) or gamma (1).
__device__ __forceinline__ uint64_t field_code(uint32_t code, uint32_t N, uint32_t &len) {
    return code ? gamma_code(N, len) : omega_code(N, len);
}

__device__ __forceinline__ uint32_t omega_len(uint32_t N) {
    uint32_t L = 1;
    uint32_t m = N;
    while (m > 1u) {
        const uint32_t b = 32u - (uint32_t)__clz(m);
        L += b;
        m = b - 1u;
    }
    return L;
}

// ---- wave/block scans (wave64, fixed combination order: deterministic) ----

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x >> 6); }

// Wave64 inclusive scans of 32-bit values in registers with DPP lane moves
// (CDNA data-parallel primitives): row_shr 1, 2, 4, 8 scan each row of 16
// lanes, then row_bcast 15 and row_bcast 31 carry row totals into the later
// rows. A lane whose source lies outside its row (or a row outside the row
// mask) reads the identity. wave_shr1 moves each lane's value to the next lane
// (lane 0 gets the identity), turning an inclusive scan into an exclusive one.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143, kDppWaveShr1 = 0x138, kDppWaveShl1 = 0x130;

template <int CTRL, int ROWS>
struct DppPair {
    static constexpr int first = CTRL, second = ROWS;
};

template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_move(int identity, int x) {
    return __builtin_amdgcn_update_dpp(identity, x, CTRL, ROWS, 0xf, false);
}

// A 64-bit value moved as two 32-bit halves (identity 0).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_move64(uint64_t x) {
    const int lo = dpp_move<CTRL, ROWS>(0, (int)(uint32_t)x);
    const int hi = dpp_move<CTRL, ROWS>(0, (int)(uint32_t)(x >> 32));
    return ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo;
}

__device__ __forceinline__ uint64_t wave_incl_add_u64(uint64_t x) {
    x += dpp_move64<kDppRowShr1, 0xf>(x);
    x += dpp_move64<kDppRowShr2, 0xf>(x);
    x += dpp_move64<kDppRowShr4, 0xf>(x);
    x += dpp_move64<kDppRowShr8, 0xf>(x);
    x += dpp_move64<kDppRowBcast15, 0xa>(x);
    x += dpp_move64<kDppRowBcast31, 0xc>(x);
    return x;
}

__device__ __forceinline__ int wave_incl_max_i32(int x) {
    constexpr int id = INT_MIN;
    auto mx = [](int a, int b) { return a > b ? a : b; };
    x = mx(x, dpp_move<kDppRowShr1, 0xf>(id, x));
    x = mx(x, dpp_move<kDppRowShr2, 0xf>(id, x));
    x = mx(x, dpp_move<kDppRowShr4, 0xf>(id, x));
    x = mx(x, dpp_move<kDppRowShr8, 0xf>(id, x));
    x = mx(x, dpp_move<kDppRowBcast15, 0xa>(id, x));
    x = mx(x, dpp_move<kDppRowBcast31, 0xc>(id, x));
    return x;
}

__device__ __forceinline__ uint32_t wave_incl_add_u32(uint32_t v) {
    int x = (int)v;
    x += dpp_move<kDppRowShr1, 0xf>(0, x);
    x += dpp_move<kDppRowShr2, 0xf>(0, x);
    x += dpp_move<kDppRowShr4, 0xf>(0, x);
    x += dpp_move<kDppRowShr8, 0xf>(0, x);
    x += dpp_move<kDppRowBcast15, 0xa>(0, x);
    x += dpp_move<kDppRowBcast31, 0xc>(0, x);
    return (uint32_t)x;
}

__device__ __forceinline__ int wave_shr1_i32(int identity, int x) {
    return dpp_move<kDppWaveShr1, 0xf>(identity, x);
}

// Total of a double over the wave (MAXN: the maximum of values >= 0), given to
// every lane. The same DPP steps as above bring the total to lane 63, moving
// the two 32-bit halves of each double (identity +0.0); a read of lane 63
// broadcasts it. The combination order is fixed (rows by shifts, then rows
// 0-1 and 2-3, then the halves), so every call rounds the same way.
template <bool MAXN>
__device__ __forceinline__ double wave_total_f64(double v) {
    auto op = [](double a, double b) { return MAXN ? (a > b ? a : b) : a + b; };
    auto mv = [](double x, auto ctrl_rows) -> double {
        return __longlong_as_double((long long)dpp_move64<decltype(ctrl_rows)::first, decltype(ctrl_rows)::second>(
            (uint64_t)__double_as_longlong(x)));
    };
    v = op(v, mv(v, DppPair<kDppRowShr1, 0xf>{}));
    v = op(v, mv(v, DppPair<kDppRowShr2, 0xf>{}));
    v = op(v, mv(v, DppPair<kDppRowShr4, 0xf>{}));
    v = op(v, mv(v, DppPair<kDppRowShr8, 0xf>{}));
    v = op(v, mv(v, DppPair<kDppRowBcast15, 0xa>{}));
    v = op(v, mv(v, DppPair<kDppRowBcast31, 0xc>{}));
    const uint64_t b = __double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// The previous (next) lane's value within aligned groups of `width` lanes, a
// lane at its group's edge getting its own value: __shfl_up (__shfl_down) by
// one, with a DPP wave shift when the group is the whole wave.
__device__ __forceinline__ uint32_t lane_prev(uint32_t x, uint32_t width) {
    if (width == 64u) return (uint32_t)dpp_move<kDppWaveShr1, 0xf>((int)x, (int)x);
    return __shfl_up(x, 1, (int)width);
}

__device__ __forceinline__ uint32_t lane_next(uint32_t x, uint32_t width) {
    if (width == 64u) return (uint32_t)dpp_move<kDppWaveShl1, 0xf>((int)x, (int)x);
    return __shfl_down(x, 1, (int)width);
}

__device__ __forceinline__ uint64_t lane_next64(uint64_t x, uint32_t width) {
    return ((uint64_t)lane_next((uint32_t)(x >> 32), width) << 32) | lane_next((uint32_t)x, width);
}

// Total of a double over each half of the wave (lanes 0-31 and 32-63; MAXN:
// the maximum of values >= 0), given to the lanes of that half: the row steps
// of wave_total_f64, then row_bcast 15 into rows 1 and 3 only, so lanes 31 and
// 63 hold the halves' totals.
template <bool MAXN>
__device__ __forceinline__ double half_wave_total_f64(double v) {
    auto op = [](double a, double b) { return MAXN ? (a > b ? a : b) : a + b; };
    auto mv = [](double x, auto ctrl_rows) -> double {
        return __longlong_as_double((long long)dpp_move64<decltype(ctrl_rows)::first, decltype(ctrl_rows)::second>(
            (uint64_t)__double_as_longlong(x)));
    };
    v = op(v, mv(v, DppPair<kDppRowShr1, 0xf>{}));
    v = op(v, mv(v, DppPair<kDppRowShr2, 0xf>{}));
    v = op(v, mv(v, DppPair<kDppRowShr4, 0xf>{}));
    v = op(v, mv(v, DppPair<kDppRowShr8, 0xf>{}));
    v = op(v, mv(v, DppPair<kDppRowBcast15, 0xa>{}));
    const uint64_t b = __double_as_longlong(v);
    const uint32_t src = lane_id() < 32 ? 31u : 63u;
    const uint32_t lo0 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 31);
    const uint32_t hi0 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 31);
    const uint32_t lo1 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
    const uint32_t hi1 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
    const uint32_t lo = src == 31u ? lo0 : lo1, hi = src == 31u ? hi0 : hi1;
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Exclusive block sum of 64-bit values in thread order (DPP wave scans, the
// waves' totals through `scratch`, kWaves entries, not reused before the next
// __syncthreads()); also returns the block total.
__device__ __forceinline__ uint64_t block_excl_add_u64(uint64_t x, uint64_t *scratch, uint64_t &total) {
    const uint64_t incl = wave_incl_add_u64(x);
    const int lane = lane_id(), wave = wave_id();
    if (lane == 63) scratch[wave] = incl;
    __syncthreads();
    uint64_t prefix = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        if (w < wave) prefix += scratch[w];
        tot += scratch[w];
    }
    total = tot;
    return prefix + dpp_move64<kDppWaveShr1, 0xf>(incl);
}

// Segmented inclusive scan over the wave in lane order with DPP lane moves (the
// row shifts and broadcasts of the scans above; a lane that receives nothing
// takes (0, 0), the identity): (v, f) becomes the combination of lanes
// 0..lane, a set flag starting a new segment.
template <bool MAXN>
__device__ __forceinline__ void wave_seg_incl_f64(double &v, int &f) {
    auto op = [](double a, double b) { return MAXN ? (a > b ? a : b) : a + b; };
    auto step = [&](auto ctrl_rows) {
        constexpr int C = decltype(ctrl_rows)::first, R = decltype(ctrl_rows)::second;
        const double yv = __longlong_as_double((long long)dpp_move64<C, R>((uint64_t)__double_as_longlong(v)));
        const int yf = dpp_move<C, R>(0, f);
        if (!f) v = op(yv, v);
        f |= yf;
    };
    step(DppPair<kDppRowShr1, 0xf>{});
    step(DppPair<kDppRowShr2, 0xf>{});
    step(DppPair<kDppRowShr4, 0xf>{});
    step(DppPair<kDppRowShr8, 0xf>{});
    step(DppPair<kDppRowBcast15, 0xa>{});
    step(DppPair<kDppRowBcast31, 0xc>{});
}

// Segmented inclusive scan of (flag, value) over the block in thread order (the
// waves by wave_seg_incl_f64, then in wave order through sv/sf):
// S_j = v_j if f_j else S_{j-1} + v_j. Returns S_{j-1} (the exclusive value; 0
// for thread 0). Used for bucket sums of squares that span several threads.
// MAXN: the same scan with max in place of + (for bucket max-norms; the values
// are >= 0, so 0 is the identity).
template <bool MAXN = false>
__device__ __forceinline__ double block_seg_excl_sum(double v, int f, double *sv, int *sf) {
    const int lane = lane_id(), wave = wave_id();
    auto op = [](double a, double b) { return MAXN ? (a > b ? a : b) : a + b; };
    wave_seg_incl_f64<MAXN>(v, f);
    if (lane == 63) { sv[wave] = v; sf[wave] = f; }
    __syncthreads();
    double pv = 0.0;
    for (int w = 0; w < wave; ++w) {  // combine the earlier waves in order
        if (sf[w]) pv = sv[w]; else pv = op(pv, sv[w]);
    }
    const double incl = f ? v : op(pv, v);
    // the previous lane's inclusive value; lane 0 takes the earlier waves'
    double ex = __longlong_as_double(
        (long long)dpp_move64<kDppWaveShr1, 0xf>((uint64_t)__double_as_longlong(incl)));
    if (lane == 0) ex = pv;
    return ex;
}

// ---- ragged bucket layout carried in the kernel arguments ----
// A batch of at most kMaxSegs tensors given by their lengths: tensor i starts
// at coordinate start[i] and its buckets (of d coordinates, the last one
// shorter) are first[i] .. first[i + 1] - 1; start[nseg] = n, first[nseg] = nb.
// nseg = 0: the layout is the device bucket table instead.
constexpr uint32_t kMaxSegs = 160;

struct SegTable {
    uint32_t nseg, d;
    uint64_t start[kMaxSegs + 1];
    uint32_t first[kMaxSegs + 1];
};

// First coordinate of bucket b (b = nb: n): from the segment table, or the
// device table.
__device__ __forceinline__ uint64_t ragged_start(const uint64_t *table, const SegTable &S, uint64_t b) {
    if (S.nseg == 0) return table[b];
    uint32_t lo = 0, hi = S.nseg;  // the last segment whose first bucket is <= b
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if ((uint64_t)S.first[mid] <= b) lo = mid; else hi = mid - 1;
    }
    if (lo == S.nseg) return S.start[S.nseg];
    const uint64_t g = S.start[lo] + (b - S.first[lo]) * (uint64_t)S.d;
    return g < S.start[lo + 1] ? g : S.start[lo + 1];
}

// ---- agent-scope flags for the cross-workgroup protocol ----
__device__ __forceinline__ uint64_t ld_agent(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace qsgd
