// INT2 asymmetric packing of selected KV tokens (KIVI-style), gfx950.
//
// Pith review of MiniKV, "Assumptions & free parameters": keys are quantised
// per channel over groups of 16 tokens, values per token over groups of 16
// channels; verdict record, key_machinery: sixteen 2-bit codes per 32-bit
// word with fp16 scale and zero-point; supporting citation of KIVI: 2-bit
// asymmetric quantisation.
//
// The codec must agree bit for bit with a separately written reference, so
// every fp32 operation below is a single round-to-nearest-even operation in
// a fixed order: range = max - min, s = range / 3 (correctly rounded
// division), scale = fp16(s), zero = min + 0 (turns -0 into +0), and the code
// of x is decided by exact comparisons of d = x - zero against (c + 1/2) *
// scale (exact products), i.e. round-half-even of d / scale clamped to
// [0, 3].  Contraction into FMAs is switched off for this file.
#pragma clang fp contract(off)

#include "common.h"
#include "launch.h"

namespace minikv {
namespace {

struct QParams {
    uint16_t sh, zh;
    float sf, zf, t0, t1, t2;
};

__device__ __forceinline__ QParams qparams(float mn, float mx) {
    QParams p;
    float range = __fsub_rn(mx, mn);
    float s32 = __fdiv_rn(range, 3.0f);
    p.sh = f2h_bits(s32);
    p.zh = f2h_bits(__fadd_rn(mn, 0.0f));
    p.sf = h2f(p.sh);
    p.zf = h2f(p.zh);
    p.t0 = __fmul_rn(0.5f, p.sf);
    p.t1 = __fmul_rn(1.5f, p.sf);
    p.t2 = __fmul_rn(2.5f, p.sf);
    return p;
}

__device__ __forceinline__ uint32_t code_of(float x, const QParams &p) {
    if (p.sf == 0.0f) return 0u;
    float d = __fsub_rn(x, p.zf);
    return (uint32_t)(d > p.t0) + (uint32_t)(d >= p.t1) +
           (uint32_t)(d > p.t2);
}

// OR of a value over the 16 lanes of a DPP row; every lane gets the result.
__device__ __forceinline__ uint32_t row16_or(uint32_t v) {
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xf, 0xf, false);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xf, 0xf, false);
    return v;
}

__device__ __forceinline__ void unpack8(uint4 x, float *f) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = h2f((uint16_t)(w[j >> 1] >> (16 * (j & 1))));
}

// Keys: one thread per (key group, 8 channels), 16-byte loads of each of the
// group's Gk source rows.  Rows come sixteen at a time: the sixteen
// selection indices are requested together, then the sixteen rows, so a
// 16-token group costs two round trips to memory and its rows stay in
// registers for both the min/max pass and the code pass (longer groups
// read each 16-row chunk again for the codes; the second read hits the
// cache).  A key word holds 16 channels of one token, so the two threads of
// a 16-channel block combine their halves of each word.
template <int D>
__global__ __launch_bounds__(256) void pack_keys_kernel(
    PackSrc src, int n_groups, int dst_group_off, CacheView c) {
    constexpr int TPG = D / 8;                   // threads per group
    constexpr int GPB = 256 / TPG;               // groups per block
    const int unit = blockIdx.y;
    const int gi = blockIdx.x * GPB + threadIdx.x / TPG;
    const int oct = threadIdx.x % TPG;           // channels 8 oct .. 8 oct + 7
    if (gi >= n_groups) return;                  // whole channel blocks leave
    const int Gk = c.Gk;
    const uint16_t *base = src.k + (size_t)unit * src.src_unit + oct * 8;
    const int32_t *sel = src.sel ? src.sel + (size_t)unit * src.sel_unit
                                 : nullptr;
    const int p0 = gi * Gk;

    constexpr int RB = 16;                       // Gk is a multiple of 16
    uint4 rr[RB];
    auto load_rows = [&](int t0) {
        int row[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i)
            row[i] = sel ? (int)min((uint32_t)sel[p0 + t0 + i], (uint32_t)(src.n_rows - 1))
                         : p0 + t0 + i;
#pragma unroll
        for (int i = 0; i < RB; ++i)
            rr[i] = *reinterpret_cast<const uint4 *>(base + (size_t)row[i] * D);
    };
    float mn[8], mx[8];
    for (int t0 = 0; t0 < Gk; t0 += RB) {
        load_rows(t0);
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            float x[8];
            unpack8(rr[i], x);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (t0 + i == 0) {
                    mn[j] = x[j];
                    mx[j] = x[j];
                } else {
                    if (x[j] < mn[j]) mn[j] = x[j];
                    if (x[j] > mx[j]) mx[j] = x[j];
                }
            }
        }
    }
    QParams qp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) qp[j] = qparams(mn[j], mx[j]);

    const int g_out = dst_group_off + gi;
    int32_t *kq = c.kq + (size_t)unit * c.kq_unit() +
                  (size_t)g_out * Gk * (D / 16) + oct / 2;
    const int sh = 16 * (oct & 1);               // this thread's half-word
    for (int t0 = 0; t0 < Gk; t0 += RB) {
        if (Gk > RB) load_rows(t0);              // a 16-token group kept its rows
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            float x[8];
            unpack8(rr[i], x);
            uint32_t half = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) half |= code_of(x[j], qp[j]) << (sh + 2 * j);
            const uint32_t word = half | (uint32_t)__shfl_xor((int)half, 1);
            if ((oct & 1) == 0) kq[(size_t)(t0 + i) * (D / 16)] = (int32_t)word;
        }
    }
    const size_t mo = (size_t)unit * c.km_unit() + (size_t)g_out * D + oct * 8;
    uint32_t sw[4], zw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        sw[j] = (uint32_t)qp[2 * j].sh | ((uint32_t)qp[2 * j + 1].sh << 16);
        zw[j] = (uint32_t)qp[2 * j].zh | ((uint32_t)qp[2 * j + 1].zh << 16);
    }
    *reinterpret_cast<uint4 *>(c.ks + mo) = make_uint4(sw[0], sw[1], sw[2], sw[3]);
    *reinterpret_cast<uint4 *>(c.kz + mo) = make_uint4(zw[0], zw[1], zw[2], zw[3]);
}

// Values: one thread per (token, channel group); the group's Gv halves are
// read with 16-byte loads.  A value word holds 16 tokens of one channel: the
// 16 lanes of a DPP row take 16 consecutive tokens of the same channel group
// and OR their codes together, lane e keeping the words of channels
// 16 j + e of the group.  Token counts are multiples of 16.
//
// The threads after the packed tokens' ones copy the next n_tail source
// rows of K and V, unchanged, into residual slots 0..n_tail-1 (the ragged
// tail of the selection stays fp16), 16 bytes each.  The boundary falls on
// a multiple of 16 threads, so no DPP row mixes the two kinds.
template <int D>
__global__ __launch_bounds__(256) void pack_values_kernel(
    PackSrc src, int n_tok, int n_tail, int dst_off, CacheView c) {
    const int unit = blockIdx.y;
    const int Gv = c.Gv;
    const int gpt = D / Gv;                      // groups per token
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= n_tok * gpt) {
        constexpr int PER_ROW = D / 8;           // uint4 per row
        const int tidx = idx - n_tok * gpt;
        const int slot = tidx / PER_ROW;
        const int part = tidx % PER_ROW;
        if (slot >= n_tail) return;
        const int p = n_tok + slot;
        const int row = src.sel ? (int)min((uint32_t)src.sel[(size_t)unit * src.sel_unit + p],
                                           (uint32_t)(src.n_rows - 1))
                                : p;
        const size_t s_off = (size_t)unit * src.src_unit + (size_t)row * D;
        const size_t d_off = (size_t)unit * c.res_unit() + (size_t)slot * D;
        reinterpret_cast<uint4 *>(c.kres + d_off)[part] =
            reinterpret_cast<const uint4 *>(src.k + s_off)[part];
        reinterpret_cast<uint4 *>(c.vres + d_off)[part] =
            reinterpret_cast<const uint4 *>(src.v + s_off)[part];
        return;
    }
    const int e = idx & 15;                      // token within its block
    const int bg = idx >> 4;
    const int blk = bg / gpt;                    // 16-token block
    const int G = bg % gpt;
    const int p = blk * 16 + e;
    if (p >= n_tok) return;                      // whole rows leave
    const int row = src.sel ? (int)min((uint32_t)src.sel[(size_t)unit * src.sel_unit + p],
                                       (uint32_t)(src.n_rows - 1))
                            : p;
    const uint4 *x4 = reinterpret_cast<const uint4 *>(
        src.v + (size_t)unit * src.src_unit + (size_t)row * D + G * Gv);

    float mn = 0.f, mx = 0.f;
    for (int i = 0; i < Gv / 8; ++i) {
        float x[8];
        unpack8(x4[i], x);
        for (int j = 0; j < 8; ++j) {
            if (i == 0 && j == 0) {
                mn = x[j];
                mx = x[j];
            } else {
                if (x[j] < mn) mn = x[j];
                if (x[j] > mx) mx = x[j];
            }
        }
    }
    const QParams qp = qparams(mn, mx);

    const int t_out = dst_off + p;
    int32_t *vq = c.vq + (size_t)unit * c.vq_unit() +
                  (size_t)(t_out >> 4) * D + G * Gv + e;
    for (int wi = 0; wi < Gv / 16; ++wi) {
        uint32_t mine = 0;
        for (int hh = 0; hh < 2; ++hh) {
            float x[8];
            unpack8(x4[wi * 2 + hh], x);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t w = row16_or(code_of(x[j], qp) << (2 * e));
                if (hh * 8 + j == e) mine = w;
            }
        }
        vq[wi * 16] = (int32_t)mine;
    }
    const size_t mo = (size_t)unit * c.vm_unit() + (size_t)t_out * gpt + G;
    c.vs[mo] = qp.sh;
    c.vz[mo] = qp.zh;
}

__global__ __launch_bounds__(256) void append_copy_kernel(
    const uint16_t *k_new, const uint16_t *v_new, int units, int slot,
    CacheView c) {
    const int per_row = c.D / 8;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    const int unit = idx / per_row;
    const int part = idx % per_row;
    if (unit >= units) return;
    const size_t d_off = (size_t)unit * c.res_unit() + (size_t)slot * c.D;
    reinterpret_cast<uint4 *>(c.kres + d_off)[part] =
        reinterpret_cast<const uint4 *>(k_new + (size_t)unit * c.D)[part];
    reinterpret_cast<uint4 *>(c.vres + d_off)[part] =
        reinterpret_cast<const uint4 *>(v_new + (size_t)unit * c.D)[part];
}

}  // namespace

hipError_t launch_pack(const PackSrc &src, int units, int n_tok, int n_tail,
                       int dst_off, const CacheView &c, hipStream_t stream) {
    if (n_tok > 0) {
        const int n_groups = n_tok / c.Gk;
        const int gpb = 256 / (c.D / 8);
        dim3 gk((n_groups + gpb - 1) / gpb, units);
        if (c.D == 128)
            pack_keys_kernel<128><<<gk, 256, 0, stream>>>(src, n_groups, dst_off / c.Gk, c);
        else
            pack_keys_kernel<64><<<gk, 256, 0, stream>>>(src, n_groups, dst_off / c.Gk, c);
    }
    if (n_tok + n_tail > 0) {
        // packed tokens' value threads (n_tok % 16 == 0), then the tail copy
        const int vthreads = n_tok * (c.D / c.Gv) + n_tail * (c.D / 8);
        dim3 gv((vthreads + 255) / 256, units);
        if (c.D == 128)
            pack_values_kernel<128><<<gv, 256, 0, stream>>>(src, n_tok, n_tail, dst_off, c);
        else
            pack_values_kernel<64><<<gv, 256, 0, stream>>>(src, n_tok, n_tail, dst_off, c);
    }
    return hipGetLastError();
}

hipError_t launch_append_copy(const uint16_t *k_new, const uint16_t *v_new,
                              int units, int slot, const CacheView &c,
                              hipStream_t stream) {
    const int threads = units * (c.D / 8);
    append_copy_kernel<<<(threads + 255) / 256, 256, 0, stream>>>(
        k_new, v_new, units, slot, c);
    return hipGetLastError();
}

}  // namespace minikv
