// Top-k selection of one unit by one workgroup of NT threads (gfx950),
// shared by the selection kernel and the fused prefill tail.
//
// Pith review of MiniKV, "What carries the argument": heavy hitters are
// picked once, at the end of prefill, from the cumulative attention scores;
// "Assumptions & free parameters": a recent window is kept next to them.
// Reading taken: the window is the last n_recent tokens; heavy hitters are
// the n_hh best candidates of [0, n - n_recent) by (score descending, index
// ascending); the kept set is written in ascending token order.
//
// The n_hh-th largest score is found by a three-pass radix select (11 + 11 +
// 10 bits) over order-preserving 32-bit keys built from the fp32 bits,
// histograms in LDS.  A final pass in index order keeps every score above the
// threshold and the lowest-index scores equal to it (per-wave chunks, ballot
// prefixes), so the output is ascending and the result exact and
// deterministic.
#pragma once

#include "common.h"

namespace minikv {

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t b = __builtin_bit_cast(uint32_t, f);
    if (b == 0x80000000u) b = 0u;                   // -0 ranks as +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int NT>
struct SelLds {
    uint32_t hist[2048];
    uint32_t wsum[NT / 64 + 1];
    uint32_t s_bin, s_above;
};

// Exclusive prefix sum over the block in thread order; returns the thread's
// exclusive prefix, and the block total through *total.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *wsum,
                                                    uint32_t *total) {
    constexpr int W = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t acc = 0;
        for (int w = 0; w < W; ++w) {
            const uint32_t t = wsum[w];
            wsum[w] = acc;
            acc += t;
        }
        wsum[W] = acc;
    }
    __syncthreads();
    const uint32_t r = wsum[wave] + x - v;
    *total = wsum[W];
    __syncthreads();
    return r;
}

// The k-th largest order key of c[0 .. nc) (1 <= k <= nc) by a three-pass
// radix select; returns it, and through *need_eq how many of the keys
// equal to it belong to the top k (the lowest indices among them).
template <int NT>
__device__ uint32_t kth_key(const float *c, int nc, uint32_t k, SelLds<NT> &L,
                            uint32_t *need_eq) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, pmask = 0;
    uint32_t remaining = k;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = shifts[pass];
        const int nb = 1 << widths[pass];
        for (int i = tid; i < nb; i += NT) L.hist[i] = 0;
        __syncthreads();
        for (int j = tid; j < nc; j += NT) {
            const uint32_t u = order_key(c[j]);
            if ((u & pmask) == prefix) atomicAdd(&L.hist[(u >> shift) & (nb - 1)], 1u);
        }
        __syncthreads();
        // thread t owns bins nb-1-bpt*t ... nb-bpt*(t+1), highest first
        const int bpt = nb / NT;
        const int top = nb - 1 - bpt * tid;
        uint32_t mine = 0;
        for (int i = 0; i < bpt; ++i) mine += L.hist[top - i];
        uint32_t total;
        uint32_t above = block_excl_scan<NT>(mine, L.wsum, &total);
        if (above < remaining && remaining <= above + mine) {
            for (int i = 0; i < bpt; ++i) {
                const uint32_t h = L.hist[top - i];
                if (remaining <= above + h) {
                    L.s_bin = (uint32_t)(top - i);
                    L.s_above = above;
                    break;
                }
                above += h;
            }
        }
        __syncthreads();
        prefix |= L.s_bin << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
        remaining -= L.s_above;
        __syncthreads();
    }
    *need_eq = remaining;
    return prefix;
}

// Within-wave exclusive prefix count of a predicate, and its wave total.
__device__ __forceinline__ uint32_t wave_prefix(bool p, uint32_t *total) {
    const uint64_t m = __ballot(p);
    *total = (uint32_t)__popcll(m);
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// sel[0 .. n_hh + n_recent) of one unit from its scores c[0 .. n).
// Compaction: each wave owns one contiguous chunk of the candidates; it
// counts its keys above the threshold and equal to it, one block scan turns
// the counts into the chunk's output offset and tie rank, and each wave
// then writes its chunk in order with ballot prefixes (two block scans in
// all, instead of two per NT candidates).
template <int NT>
__device__ void select_unit(const float *c, int n, int n_hh, int n_recent, int32_t *out,
                            SelLds<NT> &L) {
    constexpr int W = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nc = n - n_recent;
    for (int t = tid; t < n_recent; t += NT) out[n_hh + t] = nc + t;
    if (n_hh == 0) return;
    if (n_hh == nc) {
        for (int t = tid; t < nc; t += NT) out[t] = t;
        return;
    }
    // T is the n_hh-th largest key; need_eq equal keys are taken, lowest
    // indices first.
    uint32_t need_eq;
    const uint32_t T = kth_key<NT>(c, nc, (uint32_t)n_hh, L, &need_eq);
    const int chunk = (nc + W - 1) / W;
    const int j0 = min(wave * chunk, nc), j1 = min(j0 + chunk, nc);
    uint32_t gt = 0, eq = 0;
    for (int j = j0 + lane; j < j1; j += 64) {
        const uint32_t u = order_key(c[j]);
        gt += u > T ? 1u : 0u;
        eq += u == T ? 1u : 0u;
    }
    for (int off = 32; off > 0; off >>= 1) {
        gt += __shfl_xor(gt, off, 64);
        eq += __shfl_xor(eq, off, 64);
    }
    // (gt, eq) of this wave -> offsets of the waves before it
    uint32_t tot;
    const uint32_t eq_before = block_excl_scan<NT>(lane == 0 ? eq : 0u, L.wsum, &tot);
    const uint32_t eq_base = __shfl(eq_before, 0, 64);
    const uint32_t eq_take = min(eq, need_eq > eq_base ? need_eq - eq_base : 0u);
    const uint32_t take_before = block_excl_scan<NT>(lane == 0 ? gt + eq_take : 0u, L.wsum, &tot);
    uint32_t pos = __shfl(take_before, 0, 64);
    uint32_t eq_seen = eq_base;
    for (int t0 = j0; t0 < j1; t0 += 64) {
        const int j = t0 + lane;
        const uint32_t u = j < j1 ? order_key(c[j]) : 0u;
        const bool is_eq = j < j1 && u == T;
        uint32_t eq_tot;
        const uint32_t rank = eq_seen + wave_prefix(is_eq, &eq_tot);
        const bool take = j < j1 && (u > T || (is_eq && rank < need_eq));
        uint32_t take_tot;
        const uint32_t p = pos + wave_prefix(take, &take_tot);
        if (take && p < (uint32_t)n_hh) out[p] = j;
        pos += take_tot;
        eq_seen += eq_tot;
    }
}

}  // namespace minikv
