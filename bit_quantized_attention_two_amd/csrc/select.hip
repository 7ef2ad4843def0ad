// Persistent heavy-hitter + recent-window selection, gfx950.
//
// Pith review of MiniKV, "What carries the argument": heavy hitters are
// picked once, at the end of prefill, from the cumulative attention scores
// and are never re-selected; "Assumptions & free parameters": a recent window
// is kept next to them.  Reading taken: the window is the last n_recent
// tokens; heavy hitters are the n_hh best candidates of [0, n - n_recent) by
// (score descending, index ascending); the kept set is written in ascending
// token order (attention does not depend on the order of a common
// permutation of keys and values -- the MiKV rebuttal page on permutation
// invariance).
//
// One workgroup per (batch, kv head).  The n_hh-th largest score is found by
// a three-pass radix select (11 + 11 + 10 bits) over order-preserving 32-bit
// keys built from the fp32 bits, histograms in LDS.  A final pass in index
// order keeps every score above the threshold and the lowest-index scores
// equal to it, compacting with wave ballots, so the output is ascending and
// the whole result is exact and deterministic.
#include "common.h"
#include "launch.h"

namespace minikv {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kWaves = kSelThreads / 64;

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t b = __builtin_bit_cast(uint32_t, f);
    if (b == 0x80000000u) b = 0u;                   // -0 ranks as +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Exclusive prefix sum over the block in thread order; returns the thread's
// exclusive prefix, and the block total through *total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *wsum,
                                                    uint32_t *total) {
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
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t t = wsum[w];
            wsum[w] = acc;
            acc += t;
        }
        wsum[kWaves] = acc;
    }
    __syncthreads();
    const uint32_t r = wsum[wave] + x - v;
    *total = wsum[kWaves];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float *__restrict__ col, int n, int n_hh, int n_recent,
    int32_t *__restrict__ sel) {
    const int unit = blockIdx.x;
    const int tid = threadIdx.x;
    const float *c = col + (size_t)unit * n;
    int32_t *out = sel + (size_t)unit * (n_hh + n_recent);
    const int nc = n - n_recent;

    for (int t = tid; t < n_recent; t += kSelThreads) out[n_hh + t] = nc + t;
    if (n_hh == 0) return;
    if (n_hh == nc) {
        for (int t = tid; t < nc; t += kSelThreads) out[t] = t;
        return;
    }

    __shared__ uint32_t hist[2048];
    __shared__ uint32_t wsum[kWaves + 1];
    __shared__ uint32_t s_bin, s_above;

    uint32_t prefix = 0, pmask = 0;
    uint32_t remaining = (uint32_t)n_hh;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = shifts[pass];
        const int nb = 1 << widths[pass];
        for (int i = tid; i < nb; i += kSelThreads) hist[i] = 0;
        __syncthreads();
        for (int j = tid; j < nc; j += kSelThreads) {
            const uint32_t u = order_key(c[j]);
            if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
        }
        __syncthreads();
        // thread t owns bins nb-1-bpt*t ... nb-bpt*(t+1), highest first
        const int bpt = nb / kSelThreads;
        const int top = nb - 1 - bpt * tid;
        uint32_t mine = 0;
        for (int i = 0; i < bpt; ++i) mine += hist[top - i];
        uint32_t total;
        uint32_t above = block_excl_scan(mine, wsum, &total);
        if (above < remaining && remaining <= above + mine) {
            for (int i = 0; i < bpt; ++i) {
                const uint32_t h = hist[top - i];
                if (remaining <= above + h) {
                    s_bin = (uint32_t)(top - i);
                    s_above = above;
                    break;
                }
                above += h;
            }
        }
        __syncthreads();
        prefix |= s_bin << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
        remaining -= s_above;
        __syncthreads();
    }
    // prefix is the n_hh-th largest key; `remaining` equal keys are taken,
    // lowest indices first.
    const uint32_t T = prefix;
    const uint32_t need_eq = remaining;
    uint32_t base = 0, eq_seen = 0;
    for (int t0 = 0; t0 < nc; t0 += kSelThreads) {
        const int j = t0 + tid;
        const uint32_t u = j < nc ? order_key(c[j]) : 0u;
        const uint32_t gt = (j < nc && u > T) ? 1u : 0u;
        const uint32_t eq = (j < nc && u == T) ? 1u : 0u;
        uint32_t eq_tot;
        const uint32_t eq_rank = eq_seen + block_excl_scan(eq, wsum, &eq_tot);
        const uint32_t take = gt | (eq & (eq_rank < need_eq ? 1u : 0u));
        uint32_t take_tot;
        const uint32_t pos = base + block_excl_scan(take, wsum, &take_tot);
        if (take && pos < (uint32_t)n_hh) out[pos] = j;
        base += take_tot;
        eq_seen += eq_tot;
    }
}

}  // namespace

hipError_t launch_select(const float *col, int units, int n, int n_hh,
                         int n_recent, int32_t *sel, hipStream_t stream) {
    select_kernel<<<units, kSelThreads, 0, stream>>>(col, n, n_hh, n_recent, sel);
    return hipGetLastError();
}

}  // namespace minikv
