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

typedef short short4_lds __attribute__((ext_vector_type(4)));
// Native 16-byte vector; HIP's uint4 struct in a small array is not promoted
// to registers when filled from global memory.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// gfx950 transposing LDS read.  Within each group of 16 lanes, lane i gets
// element i % 4 of the 8-byte rows addressed by lanes i/4, i/4+4, i/4+8 and
// i/4+12 of its group (checked on the device).  With lane L addressing key
// row (kb + L/4) at channel (d0 + 4 (L%4)) of a row-major [key][d] tile,
// lane L receives channel d0 + L of keys kb .. kb+3: the K-contiguous
// operand layout the MFMA wants, without a transposed copy of the tile.
__device__ __forceinline__ half4_t ds_read_tr16(const uint16_t *lds) {
    const short4_lds v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4_lds *)(lds));
    return __builtin_bit_cast(half4_t, v);
}

template <bool B> struct bool_c { static constexpr bool value = B; };

// ---------------------------------------------------------------- pass 1
//
// Per wave: 32 query rows.  S^T = K Q^T (keys as MFMA rows, queries as
// columns) so that each lane owns one query column: the row max needs a
// single exchange between the two lane halves.  O^T = V^T P^T re-uses the
// S^T accumulator registers directly as the P operand: the contraction slots
// of k-step (st, a2) are mapped onto the keys those registers hold, and the
// matching V^T operand is read from the row-major V tile with the
// transposing LDS read.
//
// Pipeline: the K/V tile of iteration kt+1 is loaded from HBM into registers
// while tile kt is multiplied, then written to the other half of a
// double-buffered LDS tile; one barrier per iteration.  Loads are never
// predicated: rows past n re-read row n-1 and are masked.  Tiles that touch
// the diagonal or the end of the sequence take a masked copy of the softmax;
// the others a mask-free one.  Two waves per SIMD (<= 256 registers).
template <int D>
__global__ __launch_bounds__(256, 2) void prefill_fwd_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, uint16_t *__restrict__ o,
    float *__restrict__ lse, int Hq, int Hkv, int n, float sl2) {
    constexpr int KS = D / 16;
    constexpr int DT = D / 32;
    constexpr int KPAD = D + 8;       // K row stride (halves): 4 dwords mod 64
    constexpr int VSTR = D + 32;      // V row stride (halves): 16 dwords mod 32
    constexpr int LD = kBN * D / 8 / 256;          // uint4 loads per thread
    static_assert(LD >= 1 && LD * 256 * 8 == kBN * D, "tile / threads");
    __shared__ __attribute__((aligned(16))) uint16_t k_s[2][kBN * KPAD];
    __shared__ __attribute__((aligned(16))) uint16_t v_s[2][kBN * VSTR];

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
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = load_h8(qp + (size_t)min(qrow, n - 1) * D + ks * 16 + 8 * hi);
    float16_t oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = float16_t{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    const int kend = min(n, qb * kBM + kBM);
    const int ntiles = (kend + kBN - 1) / kBN;

    u32x4 kreg[LD], vreg[LD];
    auto load_tile = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int idx = tid + 256 * i;
            const int r = idx / (D / 8), cc = idx % (D / 8);
            const size_t off = (size_t)min(k0 + r, n - 1) * D + cc * 8;
            kreg[i] = *reinterpret_cast<const u32x4 *>(kp + off);
            vreg[i] = *reinterpret_cast<const u32x4 *>(vp + off);
        }
    };
    auto store_tile = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int idx = tid + 256 * i;
            const int r = idx / (D / 8), cc = idx % (D / 8);
            *reinterpret_cast<u32x4 *>(k_s[buf] + r * KPAD + cc * 8) = kreg[i];
            *reinterpret_cast<u32x4 *>(v_s[buf] + r * VSTR + cc * 8) = vreg[i];
        }
    };

    // lane-constant parts of the transposed V reads
    const int grp = lane >> 4, L = lane & 15;
    const int v_lane_off = (4 * (grp >> 1) + (L >> 2)) * VSTR + 16 * (grp & 1) + 4 * (L & 3);

    auto tile_step = [&](auto MASKED, int buf, int k0) __attribute__((always_inline)) {
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
        if constexpr (decltype(MASKED)::value) {
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
            for (int i = 0; i < 16; i += 2) tmax = fmaxf(tmax, fmaxf(s[st][i], s[st][i + 1]));
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

        half8_t pf[4];                              // k-step (st, a2) = 2 st + a2
        float l0 = 0.f, l1 = 0.f;                   // tile sum first: no drift
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][i], sl2, -m_use));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][i + 1], sl2, -m_use));
                l0 += p0;
                l1 += p1;
                pf[st * 2 + (i >> 3)][i & 7] = (half_t)p0;
                pf[st * 2 + (i >> 3)][(i & 7) + 1] = (half_t)p1;
            }
        l_run += l0 + l1;
        const uint16_t *vb = v_s[buf] + v_lane_off;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int st = kk >> 1, a2 = kk & 1;
            const uint16_t *vk = vb + (st * 32 + 16 * a2) * VSTR;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const half4_t lo4 = ds_read_tr16(vk + dt * 32);
                const half4_t hi4 = ds_read_tr16(vk + 8 * VSTR + dt * 32);
                const half8_t a = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3,
                                                          4, 5, 6, 7);
                oacc[dt] = mfma32(a, pf[kk], oacc[dt]);
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
            if ((k0 + kBN - 1 > q0) || (k0 + kBN > n))
                tile_step(bool_c<true>{}, buf, k0);
            else
                tile_step(bool_c<false>{}, buf, k0);
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
// LDS tile, with one barrier per tile.  Rows past n get LSE = +inf, so their
// probabilities are exactly 0; only sub-tiles that cross the diagonal take
// the masked copy of the update.
template <int D>
__global__ __launch_bounds__(256, 2) void prefill_col_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const float *__restrict__ lse, float *__restrict__ col, int Hq, int Hkv,
    int n, float sl2) {
    constexpr int KS = D / 16;
    constexpr int QPAD = D + 8;
    constexpr int QLD = kBQ2 * D / 8 / 256;         // uint4 loads per thread
    __shared__ __attribute__((aligned(16))) uint16_t q_s[2][kBQ2 * QPAD];
    __shared__ __attribute__((aligned(16))) float lse_s[2][kBQ2];

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
    for (int ks = 0; ks < KS; ++ks)
        kf[ks] = load_h8(kp + (size_t)min(key, n - 1) * D + ks * 16 + 8 * hi);
    // Column sum: each 64-row tile is summed on its own, then added to a
    // compensated (Kahan) running sum, so tens of thousands of small
    // probabilities added to a large column total do not drift low.
    float colacc = 0.f, colcomp = 0.f;

    // flattened (head, query tile) sequence
    const int qstart = kb * kBK2;
    const int tiles_per_head = (n - qstart + kBQ2 - 1) / kBQ2;
    const int ntiles = g * tiles_per_head;
    u32x4 qreg[QLD];
    float lreg = 0.f;
    auto load_tile = [&](int t) __attribute__((always_inline)) {
        const int h = t / tiles_per_head;
        const int qt0 = qstart + (t % tiles_per_head) * kBQ2;
        const size_t bhq = (size_t)b * Hq + kvh * g + h;
        const uint16_t *qp = q + bhq * n * D;
#pragma unroll
        for (int i = 0; i < QLD; ++i) {
            const int idx = tid + 256 * i;
            const int r = idx / (D / 8), cc = idx % (D / 8);
            qreg[i] = *reinterpret_cast<const u32x4 *>(
                qp + (size_t)min(qt0 + r, n - 1) * D + cc * 8);
        }
        if (tid < kBQ2) {
            const float x = lse[bhq * n + min(qt0 + tid, n - 1)] * kLog2e;
            lreg = qt0 + tid < n ? x : INFINITY;
        }
    };
    auto store_tile = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < QLD; ++i) {
            const int idx = tid + 256 * i;
            const int r = idx / (D / 8), cc = idx % (D / 8);
            *reinterpret_cast<u32x4 *>(q_s[buf] + r * QPAD + cc * 8) = qreg[i];
        }
        if (tid < kBQ2) lse_s[buf][tid] = lreg;
    };

    auto sub_tile = [&](auto MASKED, int buf, int qt0, int qs) __attribute__((always_inline)) -> float {
        float16_t s = float16_t{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const half8_t a =
                load_h8(q_s[buf] + (qs * 32 + l32) * QPAD + ks * 16 + 8 * hi);
            s = mfma32(a, kf[ks], s);
        }
        // s[i] = S[query = qt0 + 32 qs + 8(i/4) + 4 hi + i%4][key]
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const float4_t l4 = *reinterpret_cast<const float4_t *>(
                &lse_s[buf][qs * 32 + 8 * i4 + 4 * hi]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * i4 + j], sl2, -l4[j]));
                if constexpr (decltype(MASKED)::value) {
                    if (qt0 + qs * 32 + 8 * i4 + 4 * hi + j < key) p = 0.f;
                }
                if (j & 1) t1 += p; else t0 += p;
            }
        }
        return t0 + t1;
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
                if (qt0 + qs * 32 < k0w + 31)       // crosses the diagonal
                    tile += sub_tile(bool_c<true>{}, buf, qt0, qs);
                else
                    tile += sub_tile(bool_c<false>{}, buf, qt0, qs);
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
