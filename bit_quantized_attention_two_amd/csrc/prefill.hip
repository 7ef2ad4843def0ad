// Two-pass prefill attention with per-key cumulative scores, gfx950 MFMA.
//
// Pith review of MiniKV, "What carries the argument" and the verdict record's
// key_machinery: the prefill kernel returns the attention output and, for
// each key, the attention it received summed over the query rows, without
// storing the n x n matrix (memory linear in n).  Fig. 4 of the paper shows a
// two-pass parallelisation; its caption is cut off on the page.  Reading
// taken here: pass 1 is parallel over query blocks and produces O and the
// row log-sum-exp; pass 2 is parallel over key blocks, recomputes Q K^T and
// sums exp(s - LSE) down each column, so every column is owned by one
// workgroup (no atomics, deterministic).
//
// Causal mask including the diagonal, scale 1/sqrt(D), GQA: query head hq
// reads kv head hq / g, and pass 2 sums the g query heads of a kv head.
//
// MFMA: v_mfma_f32_32x32x16_f16 (fp16 inputs, fp32 accumulate).
#include "common.h"
#include "launch.h"

// The compensated column sum below relies on each fp32 operation being
// rounded separately.
#pragma clang fp contract(off)

namespace minikv {
namespace {

constexpr int kBM = 128;      // pass 1: queries per block (32 per wave)
constexpr int kBN = 64;       // pass 1: keys per iteration
constexpr int kBK2 = 128;     // pass 2: keys per block (32 per wave)
constexpr int kBQ2 = 64;      // pass 2: queries per iteration

__device__ __forceinline__ half8_t load_h8(const uint16_t *p) {
    return *reinterpret_cast<const half8_t *>(p);
}

// ---------------------------------------------------------------- pass 1
//
// Per wave: 32 query rows.  S^T = K Q^T (keys as MFMA rows, queries as
// columns) so that each lane owns one query column: the row max needs a
// single exchange between the two lane halves.  O^T = V^T P^T re-uses the
// S^T accumulator registers directly as the P operand: the contraction slots
// of k-step (st, a2) are mapped onto the keys those registers hold, and the
// V^T operand is read from a transposed LDS tile with the same key order.
//
// Pipeline: the K/V tile of iteration kt+1 is loaded from HBM into registers
// while tile kt is multiplied, then written to the other half of a
// double-buffered LDS tile; one barrier per iteration.  Two waves per SIMD
// (<= 256 registers) let one wave's MFMAs overlap the other's softmax.
template <int D>
__global__ __launch_bounds__(256, 2) void prefill_fwd_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, uint16_t *__restrict__ o,
    float *__restrict__ lse, int Hq, int Hkv, int n, float sl2) {
    constexpr int KS = D / 16;
    constexpr int DT = D / 32;
    constexpr int KPAD = D + 8;       // K tile row stride in halves (+16 B)
    constexpr int VPAD = kBN + 4;     // V^T tile row stride in halves (+8 B)
    constexpr int KLD = kBN * D / 8 / 256;        // uint4 K loads per thread
    constexpr int VTOT = (kBN / 4) * (D / 8);     // 4-key x 8-channel V groups
    constexpr int VLD = (VTOT + 255) / 256;       // V groups per thread
    static_assert(KLD >= 1 && KLD * 256 * 8 == kBN * D, "K tile / threads");
    __shared__ __attribute__((aligned(16))) uint16_t k_s[2][kBN * KPAD];
    __shared__ __attribute__((aligned(16))) uint16_t vt_s[2][D * VPAD];

    const int nqb = (n + kBM - 1) / kBM;
    const int qb = nqb - 1 - (int)blockIdx.x;       // longest rows first
    const int bh = blockIdx.y;                      // b * Hq + hq
    const int b = bh / Hq, hq = bh % Hq;
    const int kvh = hq / (Hq / Hkv);
    const uint16_t *qp = q + (size_t)bh * n * D;
    const uint16_t *kp = k + ((size_t)b * Hkv + kvh) * n * D;
    const uint16_t *vp = v + ((size_t)b * Hkv + kvh) * n * D;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int q0 = qb * kBM + wave * 32;
    const int qrow = q0 + l32;

    half8_t qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (qrow < n)
            qf[ks] = load_h8(qp + (size_t)qrow * D + ks * 16 + 8 * hi);
        else
            qf[ks] = half8_t{};
    }
    float16_t oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = float16_t{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    const int kend = min(n, qb * kBM + kBM);
    const int ntiles = (kend + kBN - 1) / kBN;

    uint4 kreg[KLD], vreg[VLD][4];
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int idx = tid + 256 * i;
            const int r = idx / (D / 8), cc = idx % (D / 8);
            kreg[i] = k0 + r < n ? *reinterpret_cast<const uint4 *>(
                                       kp + (size_t)(k0 + r) * D + cc * 8)
                                 : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int idx = tid + 256 * i;
            const int kq4 = idx / (D / 8), dof = idx % (D / 8);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = k0 + 4 * kq4 + r;
                vreg[i][r] = (idx < VTOT && key < n)
                                 ? *reinterpret_cast<const uint4 *>(
                                       vp + (size_t)key * D + dof * 8)
                                 : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int idx = tid + 256 * i;
            const int r = idx / (D / 8), cc = idx % (D / 8);
            *reinterpret_cast<uint4 *>(k_s[buf] + r * KPAD + cc * 8) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int idx = tid + 256 * i;
            const int kq4 = idx / (D / 8), dof = idx % (D / 8);
            if (idx >= VTOT) break;
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                uint32_t h[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t w[4] = {vreg[i][r].x, vreg[i][r].y,
                                           vreg[i][r].z, vreg[i][r].w};
                    h[r] = (w[d >> 1] >> (16 * (d & 1))) & 0xffffu;
                }
                *reinterpret_cast<uint2 *>(vt_s[buf] + (dof * 8 + d) * VPAD + 4 * kq4) =
                    make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            }
        }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
        const int buf = kt & 1;
        const int k0 = kt * kBN;
        const bool more = kt + 1 < ntiles;
        if (more) load_tile(k0 + kBN);

        if (k0 <= q0 + 31) {                        // not fully masked
            float16_t s[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                s[st] = float16_t{};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const half8_t a =
                        load_h8(k_s[buf] + (st * 32 + l32) * KPAD + ks * 16 + 8 * hi);
                    s[st] = mfma32(a, qf[ks], s[st]);
                }
            }
            // s[st][i] = S[key = k0 + 32 st + 8(i/4) + 4 hi + i%4][query = qrow]
            const bool need_mask = (k0 + kBN - 1 > q0) || (k0 + kBN > n);
            if (need_mask) {
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = k0 + st * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
                        if (key > qrow || key >= n) s[st][i] = -INFINITY;
                    }
            }
            float tmax = -INFINITY;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[st][i]);
            tmax = fmaxf(tmax, shfl_xor(tmax, 32)) * sl2;
            const float m_new = fmaxf(m_run, tmax);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            // rescale only when some row max of the wave moved
            if (__ballot(m_new > m_run) != 0) {
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
            }
            m_run = m_new;

            half8_t pf[4];                          // k-step (st, a2) = 2 st + a2
            float l_tile = 0.f;                     // tile sum first: no drift
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = __builtin_amdgcn_exp2f(
                        __builtin_fmaf(s[st][i], sl2, -m_use));
                    l_tile += p;
                    pf[st * 2 + (i >> 3)][i & 7] = (half_t)p;
                }
            l_run += l_tile;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int st = kk >> 1, a2 = kk & 1;
                    const uint16_t *base = vt_s[buf] + (dt * 32 + l32) * VPAD + st * 32 +
                                           16 * a2 + 4 * hi;
                    const half4_t lo4 = *reinterpret_cast<const half4_t *>(base);
                    const half4_t hi4 = *reinterpret_cast<const half4_t *>(base + 8);
                    const half8_t a = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3,
                                                              4, 5, 6, 7);
                    oacc[dt] = mfma32(a, pf[kk], oacc[dt]);
                }
            }
        }
        if (more) store_tile(buf ^ 1);
        __syncthreads();
    }

    const float l_tot = l_run + shfl_xor(l_run, 32);
    if (qrow < n) {
        const float inv = 1.f / l_tot;
        uint16_t *orow = o + ((size_t)bh * n + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d0 = dt * 32 + 8 * a4 + 4 * hi;
                const uint32_t w0 = (uint32_t)f2h_bits(oacc[dt][4 * a4 + 0] * inv) |
                                    ((uint32_t)f2h_bits(oacc[dt][4 * a4 + 1] * inv) << 16);
                const uint32_t w1 = (uint32_t)f2h_bits(oacc[dt][4 * a4 + 2] * inv) |
                                    ((uint32_t)f2h_bits(oacc[dt][4 * a4 + 3] * inv) << 16);
                *reinterpret_cast<uint2 *>(orow + d0) = make_uint2(w0, w1);
            }
        if (hi == 0) lse[(size_t)bh * n + qrow] = (m_run + log2f(l_tot)) * kLn2;
    }
}

// ---------------------------------------------------------------- pass 2
//
// Per wave: 32 key columns, K^T held in registers as the MFMA B operand.
// S = Q K^T with queries as rows: each lane owns one key column and adds the
// probabilities of its 16 query rows per 32-row sub-tile; the two lane halves
// are combined once at the end.  The next 64-query tile (and its LSE) is
// loaded into registers while the current one is used, into a double-buffered
// LDS tile, with one barrier per tile.
template <int D>
__global__ __launch_bounds__(256, 2) void prefill_col_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const float *__restrict__ lse, float *__restrict__ col, int Hq, int Hkv,
    int n, float sl2) {
    constexpr int KS = D / 16;
    constexpr int QPAD = D + 8;
    constexpr int QLD = kBQ2 * D / 8 / 256;         // uint4 loads per thread
    __shared__ __attribute__((aligned(16))) uint16_t q_s[2][kBQ2 * QPAD];
    __shared__ float lse_s[2][kBQ2];

    const int kb = blockIdx.x;                      // block 0 has most rows
    const int unit = blockIdx.y;                    // b * Hkv + kvh
    const int b = unit / Hkv, kvh = unit % Hkv;
    const int g = Hq / Hkv;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int k0w = kb * kBK2 + wave * 32;
    const int key = k0w + l32;
    const uint16_t *kp = k + (size_t)unit * n * D;

    half8_t kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (key < n)
            kf[ks] = load_h8(kp + (size_t)key * D + ks * 16 + 8 * hi);
        else
            kf[ks] = half8_t{};
    }
    // Column sum: each 64-row tile is summed on its own, then added to a
    // compensated (Kahan) running sum, so tens of thousands of small
    // probabilities added to a large column total do not drift low.
    float colacc = 0.f, colcomp = 0.f;

    // flattened (head, query tile) sequence
    const int qstart = kb * kBK2;
    const int tiles_per_head = (n - qstart + kBQ2 - 1) / kBQ2;
    const int ntiles = g * tiles_per_head;
    uint4 qreg[QLD];
    float lreg = 0.f;
    auto load_tile = [&](int t) {
        const int h = t / tiles_per_head;
        const int qt0 = qstart + (t % tiles_per_head) * kBQ2;
        const size_t bhq = (size_t)b * Hq + kvh * g + h;
        const uint16_t *qp = q + bhq * n * D;
#pragma unroll
        for (int i = 0; i < QLD; ++i) {
            const int idx = tid + 256 * i;
            const int r = idx / (D / 8), cc = idx % (D / 8);
            qreg[i] = qt0 + r < n ? *reinterpret_cast<const uint4 *>(
                                        qp + (size_t)(qt0 + r) * D + cc * 8)
                                  : make_uint4(0, 0, 0, 0);
        }
        if (tid < kBQ2)
            lreg = (qt0 + tid < n) ? lse[bhq * n + qt0 + tid] * kLog2e : INFINITY;
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < QLD; ++i) {
            const int idx = tid + 256 * i;
            const int r = idx / (D / 8), cc = idx % (D / 8);
            *reinterpret_cast<uint4 *>(q_s[buf] + r * QPAD + cc * 8) = qreg[i];
        }
        if (tid < kBQ2) lse_s[buf][tid] = lreg;
    };

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const int qt0 = qstart + (t % tiles_per_head) * kBQ2;
        const bool more = t + 1 < ntiles;
        if (more) load_tile(t + 1);
        if (qt0 + kBQ2 - 1 >= k0w) {               // some query sees some key
            float tile = 0.f;
#pragma unroll
            for (int qs = 0; qs < 2; ++qs) {
                float16_t s = float16_t{};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const half8_t a =
                        load_h8(q_s[buf] + (qs * 32 + l32) * QPAD + ks * 16 + 8 * hi);
                    s = mfma32(a, kf[ks], s);
                }
                // s[i] = S[query = qt0 + 32 qs + 8(i/4) + 4 hi + i%4][key]
                const int qb0 = qt0 + qs * 32;
                const bool need_mask = (qb0 < k0w + 31) || (qb0 + 32 > n);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = qs * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
                    float p = __builtin_amdgcn_exp2f(
                        __builtin_fmaf(s[i], sl2, -lse_s[buf][r]));
                    if (need_mask && (qt0 + r < key || qt0 + r >= n)) p = 0.f;
                    tile += p;
                }
            }
            const float y = tile - colcomp;
            const float tt = colacc + y;
            colcomp = (tt - colacc) - y;
            colacc = tt;
        }
        if (more) store_tile(buf ^ 1);
        __syncthreads();
    }
    colacc += shfl_xor(colacc, 32);
    if (hi == 0 && key < n) col[(size_t)unit * n + key] = colacc;
}

}  // namespace

hipError_t launch_prefill(const uint16_t *q, const uint16_t *k,
                          const uint16_t *v, uint16_t *o, float *lse,
                          float *col, int B, int Hq, int Hkv, int n, int D,
                          hipStream_t stream) {
    const float sl2 = kLog2e / sqrtf((float)D);
    dim3 g1((n + kBM - 1) / kBM, B * Hq);
    dim3 g2((n + kBK2 - 1) / kBK2, B * Hkv);
    if (D == 128) {
        prefill_fwd_kernel<128><<<g1, 256, 0, stream>>>(q, k, v, o, lse, Hq, Hkv, n, sl2);
        prefill_col_kernel<128><<<g2, 256, 0, stream>>>(q, k, lse, col, Hq, Hkv, n, sl2);
    } else {
        prefill_fwd_kernel<64><<<g1, 256, 0, stream>>>(q, k, v, o, lse, Hq, Hkv, n, sl2);
        prefill_col_kernel<64><<<g2, 256, 0, stream>>>(q, k, lse, col, Hq, Hkv, n, sl2);
    }
    return hipGetLastError();
}

}  // namespace minikv
