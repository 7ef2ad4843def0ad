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
// One workgroup of 1024 threads per (batch, kv head); the selection itself
// (a radix select and an ordered compaction) is in topk.h.
#include "launch.h"
#include "topk.h"

namespace minikv {
namespace {

constexpr int kSelThreads = 1024;

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float *__restrict__ col, int n, int n_hh, int n_recent,
    int32_t *__restrict__ sel) {
    __shared__ SelLds<kSelThreads> L;
    const int unit = blockIdx.x;
    select_unit<kSelThreads>(col + (size_t)unit * n, n, n_hh, n_recent,
                             sel + (size_t)unit * (n_hh + n_recent), L);
}

// DiffKV tiers of one unit (one workgroup): the counts of significance
// scores above the two thresholds, each rounded up to whole key groups;
// the k-th largest key for both counts; then one pass in index order
// writes the high tier (among the top c_hi) and the low tier (among the top
// c_kept but not the top c_hi), both ascending.  The order is (score
// descending, index ascending), so the top c_hi is part of the top c_kept.
__global__ __launch_bounds__(kSelThreads) void tier_kernel(
    const float *__restrict__ score, int n, float thr_hi, float thr_lo, int Gk,
    int32_t *__restrict__ idx_hi, int32_t *__restrict__ idx_lo,
    int32_t *__restrict__ n_hi, int32_t *__restrict__ n_lo) {
    const int unit = blockIdx.x;
    const int tid = threadIdx.x;
    const float *c = score + (size_t)unit * n;
    __shared__ SelLds<kSelThreads> L;
    __shared__ uint32_t s_cnt[2];
    if (tid == 0) s_cnt[0] = s_cnt[1] = 0;
    __syncthreads();
    uint32_t a = 0, b = 0;
    for (int j = tid; j < n; j += kSelThreads) {
        a += c[j] > thr_hi ? 1u : 0u;
        b += c[j] > thr_lo ? 1u : 0u;
    }
    atomicAdd(&s_cnt[0], a);
    atomicAdd(&s_cnt[1], b);
    __syncthreads();
    const int cap = n / Gk * Gk;
    const int c_hi = min((int)((s_cnt[0] + Gk - 1) / Gk) * Gk, cap);
    const int c_kept = max(min((int)((s_cnt[1] + Gk - 1) / Gk) * Gk, cap), c_hi);
    // thresholds as keys: (T, need_eq) for both counts; k = 0 takes nothing
    uint32_t need_hi = 0, need_kept = 0, T_hi = 0xffffffffu, T_kept = 0xffffffffu;
    if (c_hi > 0) T_hi = kth_key<kSelThreads>(c, n, (uint32_t)c_hi, L, &need_hi);
    if (c_kept > 0) T_kept = kth_key<kSelThreads>(c, n, (uint32_t)c_kept, L, &need_kept);
    int32_t *oh = idx_hi + (size_t)unit * n;
    int32_t *ol = idx_lo + (size_t)unit * n;
    uint32_t base_h = 0, base_l = 0, eqh_seen = 0, eqk_seen = 0;
    for (int t0 = 0; t0 < n; t0 += kSelThreads) {
        const int j = t0 + tid;
        const uint32_t u = j < n ? order_key(c[j]) : 0u;
        const uint32_t eqh = (j < n && c_hi > 0 && u == T_hi) ? 1u : 0u;
        const uint32_t eqk = (j < n && c_kept > 0 && u == T_kept) ? 1u : 0u;
        uint32_t tot;
        const uint32_t rh = eqh_seen + block_excl_scan<kSelThreads>(eqh, L.wsum, &tot);
        eqh_seen += tot;
        const uint32_t rk = eqk_seen + block_excl_scan<kSelThreads>(eqk, L.wsum, &tot);
        eqk_seen += tot;
        const bool in_hi = j < n && c_hi > 0 && (u > T_hi || (eqh && rh < need_hi));
        const bool in_kept = j < n && c_kept > 0 && (u > T_kept || (eqk && rk < need_kept));
        const uint32_t th = in_hi ? 1u : 0u;
        const uint32_t tl = (in_kept && !in_hi) ? 1u : 0u;
        const uint32_t ph = base_h + block_excl_scan<kSelThreads>(th, L.wsum, &tot);
        base_h += tot;
        const uint32_t pl = base_l + block_excl_scan<kSelThreads>(tl, L.wsum, &tot);
        base_l += tot;
        if (th && ph < (uint32_t)c_hi) oh[ph] = j;
        if (tl && pl < (uint32_t)(c_kept - c_hi)) ol[pl] = j;
    }
    if (tid == 0) {
        n_hi[unit] = c_hi;
        n_lo[unit] = c_kept - c_hi;
    }
}

}  // namespace

hipError_t launch_select(const float *col, int units, int n, int n_hh,
                         int n_recent, int32_t *sel, hipStream_t stream) {
    select_kernel<<<units, kSelThreads, 0, stream>>>(col, n, n_hh, n_recent, sel);
    return hipGetLastError();
}

hipError_t launch_tier(const float *score, int units, int n, float alpha_hi,
                       float alpha_lo, int Gk, int32_t *idx_hi, int32_t *idx_lo,
                       int32_t *n_hi, int32_t *n_lo, hipStream_t stream) {
    // thresholds alpha / n, one fp32 division each
    const float thr_hi = alpha_hi / (float)n, thr_lo = alpha_lo / (float)n;
    tier_kernel<<<units, kSelThreads, 0, stream>>>(score, n, thr_hi, thr_lo, Gk, idx_hi,
                                                   idx_lo, n_hi, n_lo);
    return hipGetLastError();
}

}  // namespace minikv
