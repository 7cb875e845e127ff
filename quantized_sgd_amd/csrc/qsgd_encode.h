// Quantize kernel and the fused single-pass encode kernel.
//
// Page "QSGD (Quantized Stochastic Gradient Descent) with Elias Coding":
// definition paragraph (Q_s and the Elias-coded tuple of norm, signs, non-zero
// gaps and levels) and the claim on Elias coding (F = 32 bit norm).
//
// Encode, per tile (a run of whole buckets, <= 4096 coordinates, one workgroup):
//   1. load v once from HBM, per-bucket norms, Philox rounding (qsgd_front.h);
//   2. each thread stages the records of its 16 coordinates in LDS: the 32-bit
//      norm at a bucket start, and omega(gap) | sign | omega(k) per non-zero;
//      the gap of a thread's first non-zero, when its origin lies in an earlier
//      thread, is resolved after an exclusive max-scan of "last marker" positions;
//   3. an exclusive sum-scan of per-thread bit counts gives each thread's offset
//      in the tile and the tile's size T;
//   4. decoupled lookback over earlier tiles' status words (agent-scope atomics,
//      flag and value packed in one 64-bit word) gives the tile's stream offset;
//   5. the tile's bits are assembled into 64-bit words in LDS and stored with
//      coalesced 8-byte stores. The word shared with the previous tile is
//      completed with that tile's published "carry" (its partial last word); the
//      tile's own partial last word is published the same way for the next tile.
// Every output word is written by exactly one tile; no pass re-reads v.
#pragma once

#include "qsgd_front.h"

namespace qsgd {

// Appends bit strings MSB-first into 64-bit LDS words.
struct Stager {
    uint64_t *w;
    uint64_t acc;
    uint32_t nacc;
    uint32_t widx;
    __device__ __forceinline__ uint32_t bitpos() const { return widx * 64u + nacc; }
    // bits right-aligned, 1 <= len <= 64
    __device__ __forceinline__ void put(uint64_t bits, uint32_t len) {
        const uint32_t total = nacc + len;
        if (total < 64u) {
            acc |= bits << (64u - total);
            nacc = total;
        } else {
            const uint32_t over = total - 64u;
            acc |= bits >> over;
            w[widx++] = acc;
            acc = over ? bits << (64u - over) : 0ull;
            nacc = over;
        }
    }
    __device__ __forceinline__ void flush() {
        if (nacc) w[widx] = acc;
    }
};

// OR a left-aligned 64-bit word into the LDS bit window at bit position pos.
__device__ __forceinline__ void or_bits(uint64_t *buf, uint32_t pos, uint64_t word) {
    const uint32_t idx = pos >> 6, sh = pos & 63u;
    atomicOr(reinterpret_cast<unsigned long long *>(buf + idx), (unsigned long long)(word >> sh));
    if (sh) {
        const uint64_t lo = word << (64u - sh);
        if (lo) atomicOr(reinterpret_cast<unsigned long long *>(buf + idx + 1), (unsigned long long)lo);
    }
}

struct EncodeLds {
    FrontLds f;
    uint64_t *stage;
    uint64_t *obuf;
    uint32_t *bpos;  // [K] staged bit position of each bucket's norm
    uint32_t *tb;    // [kWG] per-thread offset of the staged bits within the tile
};

__device__ __forceinline__ size_t align8(size_t x) { return (x + 7) & ~(size_t)7; }

// Carves the dynamic LDS block. K = P.K (the largest tile).
__device__ __forceinline__ EncodeLds carve_encode_lds(unsigned char *smem, const QsgdParams &P) {
    EncodeLds L;
    size_t off = 0;
    L.stage = reinterpret_cast<uint64_t *>(smem + off); off += (size_t)P.stage_words * 8;
    L.obuf = reinterpret_cast<uint64_t *>(smem + off); off += (size_t)P.obuf_words * 8;
    L.f.cb = reinterpret_cast<double *>(smem + off); off += (size_t)P.K * 8;
    L.f.segv = reinterpret_cast<double *>(smem + off); off += kWaves * 8;
    L.f.bs = reinterpret_cast<int32_t *>(smem + off); off = align8(off + (size_t)(P.K + 1) * 4);
    L.f.nrm = reinterpret_cast<float *>(smem + off); off = align8(off + (size_t)P.K * 4);
    L.f.segf = reinterpret_cast<int *>(smem + off); off = align8(off + kWaves * 4);
    L.bpos = reinterpret_cast<uint32_t *>(smem + off); off = align8(off + (size_t)P.K * 4);
    L.tb = reinterpret_cast<uint32_t *>(smem + off);
    return L;
}

// Bytes of dynamic LDS the encode / quantize kernels need (host side mirror in
// the API file).

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

template <bool RAGGED>
__global__ __launch_bounds__(kWG) void encode_kernel(QsgdParams P) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ uint32_t sh_tile;
    __shared__ uint64_t sh_base;
    __shared__ int sh_mx[kWaves];
    __shared__ uint32_t sh_ub[kWaves];
    __shared__ uint32_t sh_bits[kWaves];

    EncodeLds L = carve_encode_lds(smem, P);
    const int j = (int)threadIdx.x;
    const int lane = lane_id(), wave = wave_id();
    if (j == 0) sh_tile = atomicAdd(P.ticket, 1u);
    __syncthreads();
    const uint32_t tile = sh_tile;
    const Tile t = tile_geometry<RAGGED>(P, tile);
    fill_bucket_starts<RAGGED>(P, t, L.f);
    ThreadCoords c;
    load_coords(P, t, c);
    __syncthreads();
    bucket_norms<RAGGED>(P, t, L.f, c);
    ThreadLevels lv;
    quantize_coords(P, t, L.f, c, lv);

    // ---- events, markers and staging bounds ----
    const uint32_t ev = lv.nz | lv.bst;
    int marker = INT_MIN;
    if (ev) {
        const int h = 31 - __clz(ev);
        marker = j * kCPT + h - (((lv.nz >> h) & 1u) ? 0 : 1);
    }
    const uint32_t Ls = omega_len(P.s);
    const uint32_t ub_bits = (uint32_t)__popc(lv.nz) * (12u + Ls) + 32u * (uint32_t)__popc(lv.bst);
    const uint32_t ub_words = (ub_bits + 63u) >> 6;
    // fused exclusive scans: max of markers, sum of staging words
    int mi = wave_incl_scan(marker, [](int a, int b) { return a > b ? a : b; });
    uint32_t ui = wave_incl_scan(ub_words, [](uint32_t a, uint32_t b) { return a + b; });
    if (lane == 63) { sh_mx[wave] = mi; sh_ub[wave] = ui; }
    __syncthreads();
    int mpre = INT_MIN;
    uint32_t upre = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        if (w < wave) {
            mpre = mpre > sh_mx[w] ? mpre : sh_mx[w];
            upre += sh_ub[w];
        }
    }
    int mex = __shfl_up(mi, 1, 64);
    uint32_t uex = __shfl_up(ui, 1, 64);
    if (lane == 0) { mex = INT_MIN; uex = 0; }
    mex = mex > mpre ? mex : mpre;
    uex += upre;

    // ---- stage records ----
    Stager st{L.stage + uex, 0ull, 0u, 0u};
    int prev = 0;
    int have = 0;
    int pendx = -1;
    int kb = c.kf;
    if (c.vx0 < c.vx1 && ((lv.bst >> (c.vx0 - j * kCPT)) & 1u)) kb -= 1;
#pragma unroll
    for (int q = 0; q < kCPT; ++q) {
        const int x = j * kCPT + q;
        if ((lv.bst >> q) & 1u) {
            ++kb;
            L.bpos[kb] = st.bitpos();
            st.put((uint64_t)__float_as_uint(L.f.nrm[kb]), 32u);
            prev = x - 1;
            have = 1;
        }
        if ((lv.nz >> q) & 1u) {
            uint32_t Lk;
            uint64_t kc = omega_code(lv.k[q], Lk);
            kc |= (uint64_t)((lv.neg >> q) & 1u) << Lk;
            Lk += 1u;
            if (have) {
                uint32_t Lg;
                const uint64_t gc = omega_code((uint32_t)(x - prev), Lg);
                if (Lg + Lk <= 64u) {
                    st.put((gc << Lk) | kc, Lg + Lk);
                } else {
                    st.put(gc, Lg);
                    st.put(kc, Lk);
                }
            } else {
                pendx = x;
                have = 1;
                st.put(kc, Lk);
            }
            prev = x;
        }
    }
    st.flush();
    const uint32_t staged = st.bitpos();
    uint32_t Lp = 0;
    uint64_t pc = 0;
    if (pendx >= 0) pc = omega_code((uint32_t)(pendx - mex), Lp);
    const uint32_t bits = staged + Lp;

    // ---- tile scan of bit counts ----
    uint32_t bi = wave_incl_scan(bits, [](uint32_t a, uint32_t b) { return a + b; });
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
    if (j == 0) {
        uint64_t excl = 0;
        if (tile == 0) {
            st_agent(&P.status[0], kFlagIncl | (uint64_t)T);
        } else {
            st_agent(&P.status[tile], kFlagAgg | (uint64_t)T);
            int64_t i = (int64_t)tile - 1;
            while (true) {
                const uint64_t w = ld_acquire_agent(&P.status[i]);
                const uint64_t f = w & ~kValMask;
                if (f == 0) { __builtin_amdgcn_s_sleep(1); continue; }
                excl += w & kValMask;
                if (f == kFlagIncl) break;
                --i;
            }
            st_agent(&P.status[tile], kFlagIncl | (excl + (uint64_t)T));
        }
        sh_base = excl;
    }
    L.tb[j] = off + Lp;
    __syncthreads();
    const uint64_t base = sh_base;

    // ---- bucket offsets ----
    for (uint32_t b = threadIdx.x; b < t.K; b += kWG)
        P.offsets[t.b0 + b] = base + L.tb[L.f.bs[b] >> 4] + L.bpos[b];
    const bool last = (tile == P.ntiles - 1);
    if (last && j == 0) {
        P.offsets[P.nb] = base + T;
        *P.out_bits = base + T;
    }

    // ---- assemble the tile's words in LDS ----
    const uint32_t head = (uint32_t)(base & 63u);
    const uint32_t W = (head + T + 63u) >> 6;
    for (uint32_t w = threadIdx.x; w < W; w += kWG) L.obuf[w] = 0;
    __syncthreads();
    uint32_t pos = head + off;
    if (Lp) or_bits(L.obuf, pos, pc << (64u - Lp));
    pos += Lp;
    const uint32_t nw = (staged + 63u) >> 6;
    for (uint32_t i = 0; i < nw; ++i) or_bits(L.obuf, pos + 64u * i, L.stage[uex + i]);
    __syncthreads();

    // ---- store: interior words by all threads, edge words by thread 0 ----
    uint64_t *dst = P.out + (base >> 6);
    for (uint32_t w = 1 + threadIdx.x; w + 1 < W; w += kWG) dst[w] = L.obuf[w];
    if (j == 0) {
        const bool head_shared = head != 0;
        const bool tail_partial = ((base + T) & 63u) != 0;
        if (W > 1) {
            if (tail_partial && !last) {
                st_agent(&P.carry[tile], L.obuf[W - 1] | 1ull);
            } else {
                dst[W - 1] = L.obuf[W - 1];
                st_agent(&P.carry[tile], 1ull);
            }
        }
        uint64_t hw = L.obuf[0];
        if (head_shared) {
            uint64_t cw;
            while (((cw = ld_acquire_agent(&P.carry[tile - 1])) & 1ull) == 0) __builtin_amdgcn_s_sleep(1);
            hw |= cw & ~1ull;
        }
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

}  // namespace qsgd
