// Decode attention over the INT2-packed cache plus the fp16 residual, gfx950.
//
// Verdict record for MiniKV (arXiv 2411.18077), forward implications: the
// selection is fixed after prefill, so the retained cache has a fixed layout
// and decoding can dequantise inside the attention kernel.  This kernel never
// materialises fp16 keys or values; both contractions run on the matrix
// cores in the code domain:
//
//   logit(t) = sum_c q_c (code_tc s_k[g(t),c] + z_k[g(t),c])
//            = sum_c code_tc (q_c s_k[g,c])   +   sum_c q_c z_k[g,c]
//   o_c      = sum_t p_t (code_tc s_v[t,G(c)] + z_v[t,G(c)])
//            = sum_t code_tc (p_t s_v[t,G])   +   sum_t p_t z_v[t,G]
//
// Codes as MFMA operands.  A key word holds 16 channels of one token and a
// value word 16 tokens of one channel, both along the summed dimension.
// Masking a word with 0x00030003 << 2i leaves two 2-bit fields in the
// mantissas of two fp16 halves: the subnormals code * 4^i * 2^-24, exact.
// The matching weights (q s for keys, p s for values) are scaled by 4^-i and
// split into two fp16 parts hi + lo, which hold the weight to 2^-25
// absolute (to about 22 bits where lo is a normal fp16); each product code *
// weight is exact in the fp32 accumulator, so the other rounding is the fp32
// accumulation, as in a plain fp32 dot product.  Key weights: q is scaled per
// head by 2^-e (|q| < 1) and per slot by 4^-i once, in fp16 (exact unless
// subnormal), and each weight is the exact TwoProduct hi + lo of that q and
// the fp16 scale.  Value weights: the fp32 product p s, split.  Every fp16
// operand stays within range: p <= 1, and a scale is at most 65504 * 2 / 3.
//
// The per-group scale s_k[g, c] makes the key weights differ per key group.
// One 16-column B operand holds the weights of (head, group) pairs for 16/g
// groups at once; a 16-token tile multiplies it and keeps the columns of its
// own group.  The value weights use columns (head, channel group); each
// channel row keeps the column of its own group.  The z terms: per key
// group an MFMA of the zero-points with q, and per token a VALU sum.
//
// Work split: block (unit, split) covers `chunk` packed tokens of one unit,
// each of its waves (4, or 12 in the one-round GQA form) an equal share;
// the fp16 residual runs on the idle waves of the unit's last packed split,
// or on a split of its own when those are too few.  A wave computes all its
// logits (phase K), its softmax statistics, then P.V (phase V); the block
// merges its waves in LDS and writes one partial (max, sum, unnormalised o)
// to the workspace.
// A second kernel merges the partials of each (unit, head) and writes o.
// Small calls (64 tokens per wave) use a form that requests all of a
// wave's loads at once (ONE below); the persistence audit adds a third
// kernel that turns stored logits into per-token attention mass.
//
// Fused append: when the caller passes a new token, the residual waves read
// it from the call's input, uses it as residual slot `new_slot`, and stores
// it there for later calls.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace minikv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kMinWaveChunk = 64;
constexpr int kMaxWaveChunk = 256;
constexpr int kMaxSplit = 512;
// GQA calls whose grid fills the chip in one round use one 12-wave block
// per CU (pick_chunk explains why); its splits are 12 wave shares.
constexpr int kBigWaves = 12;

struct DecArgs {
    const uint16_t *q;
    uint16_t *o;
    CacheView c;
    int n_packed, n_res, chunk, n_chunks, nsplit;
    int res_split, res_wave0;        // the residual's waves: split res_split,
                                     // waves res_wave0.. (-1: no residual)
    int waves;                       // waves per block: kWaves or kBigWaves
    float qscale;
    const uint16_t *k_new, *v_new;   // nullable: fused append of one token
    int new_slot;                    // residual slot of the new token
    int split_off, nsplit_total;     // this launch's splits start at
                                     //   split_off of nsplit_total per unit
    float *part_ml;                  // [units][nsplit_total][G][2]
    float *part_o;                   // [units][nsplit_total][G][D]
    float *lg;                       // nullable: logits out, log2 units,
    int lg_stride;                   //   [units][G][lg_stride], cache order
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// Views of the per-wave LDS rows whose contents change type between phases
// (fp32 logits, then fp16 probability parts read as dwords): accesses
// through them may alias any other, so no load or store is moved across
// one of another type.
typedef _Float16 half_ma __attribute__((may_alias));
typedef unsigned int u32x4_ma __attribute__((ext_vector_type(4), may_alias));

// 16x16x32 fp16 MFMA: A lane l holds A[l%16][8(l/16)+j], B lane l holds
// B[8(l/16)+j][l%16], C lane l register i holds C[4(l/16)+i][l%16].
__device__ __forceinline__ float4_t mfma16(half8_t a, half8_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                           CTRL, 0xf, 0xf, false));
}
// Sum over the 16 lanes of a DPP row; every lane receives the total.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<0x128>(v);       // row_ror:8
    v += dpp<0x124>(v);       // row_ror:4
    v += dpp<0x122>(v);       // row_ror:2
    v += dpp<0x121>(v);       // row_ror:1
    return v;
}
// The values of lane l and lane l ^ 16 (or l ^ 32) in every lane:
// v_permlane16_swap / v_permlane32_swap with both operands x return them as
// the two result elements (the copy is hidden from the compiler so that the
// swap of a value with itself is not folded).  Used with symmetric
// operations only, so which element is which does not matter.
__device__ __forceinline__ float xor16_sum(float x) {
    unsigned a = __builtin_bit_cast(unsigned, x), b = a;
    asm volatile("" : "+v"(b));
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
    unsigned a = __builtin_bit_cast(unsigned, x), b = a;
    asm volatile("" : "+v"(b));
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
    unsigned a = __builtin_bit_cast(unsigned, x), b = a;
    asm volatile("" : "+v"(b));
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
    unsigned a = __builtin_bit_cast(unsigned, x), b = a;
    asm volatile("" : "+v"(b));
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
// Sum over the wave, in every lane (the same value in each: every step adds
// a lane pair's two values, which both lanes of the pair hold alike).
__device__ __forceinline__ float wave_sum(float v) {
    return xor32_sum(xor16_sum(row16_sum(v)));
}
// Max over the lanes l' with l' = l (mod S) in every lane l, S | 16.
template <int S>
__device__ __forceinline__ float strided_max(float m) {
    if constexpr (S <= 1) m = fmaxf(m, dpp<0x121>(m));    // row_ror:1
    if constexpr (S <= 2) m = fmaxf(m, dpp<0x122>(m));    // row_ror:2
    if constexpr (S <= 4) m = fmaxf(m, dpp<0x124>(m));    // row_ror:4
    if constexpr (S <= 8) m = fmaxf(m, dpp<0x128>(m));    // row_ror:8
    return xor32_max(xor16_max(m));
}
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

// The two code fields of dword i of a shifted word, as fp16 subnormals
// code * 4^i * 2^-24 in the low and high half.
__device__ __forceinline__ half8_t code_operand(uint32_t x) {
    const u32x4 v = {x & 0x00030003u, x & 0x000c000cu, x & 0x00300030u,
                     x & 0x00c000c0u};
    return __builtin_bit_cast(half8_t, v);
}

// The same for 4-bit codes stored as two 2-bit planes (plane 1 = bits 2..3):
// dword i holds (c0 + 4 c1) * 4^i * 2^-24 per half, at most 15 * 64 * 2^-24,
// still an exact subnormal.  x0, x1: the two planes' words, shifted alike.
__device__ __forceinline__ half8_t code_operand2(uint32_t x0, uint32_t x1) {
    const uint32_t y = x1 << 2;
    const u32x4 v = {(x0 & 0x00030003u) | (y & 0x000c000cu),
                     (x0 & 0x000c000cu) | (y & 0x00300030u),
                     (x0 & 0x00300030u) | (y & 0x00c000c0u),
                     (x0 & 0x00c000c0u) | (y & 0x03000300u)};
    return __builtin_bit_cast(half8_t, v);
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
// fp16 hi + lo of two fp32 weights: hi truncated (one v_cvt_pkrtz for both),
// lo the rest w - hi, exact in fp32, rounded to fp16 (one mixed-precision
// FMA per weight, written into its half: the compiler would otherwise widen
// hi, subtract and repack).  hi + lo holds w to 2^-25 absolute, and to about
// 22 bits where lo stays in fp16's normal range.
__device__ __forceinline__ void split2x2(float w0, float w1, uint32_t &hi, uint32_t &lo) {
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(w0, w1));
    uint32_t l;
    asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(l) : "v"(h), "s"(-1.0f), "v"(w0));
    asm("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "+v"(l) : "v"(h), "s"(-1.0f), "v"(w1));
    hi = h;
    lo = l;
}

// hi + lo = a * b for fp16 pairs (TwoProduct with a fused fp16 FMA): hi is
// the rounded product, lo = a b - hi rounded once, exact while it stays in
// fp16's normal range, else within 2^-25.
__device__ __forceinline__ void two_product2(uint32_t a, uint32_t b, uint32_t &hi, uint32_t &lo) {
    const half2_t x = __builtin_bit_cast(half2_t, a), y = __builtin_bit_cast(half2_t, b);
    const half2_t h = x * y;
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(x, y, -h));
}

// The fp16 pair (low half of a, low half of b), and (high half of a, high
// half of b).
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ void unpack8h(uint4 x, float *f) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = h2f((uint16_t)(w[i >> 1] >> (16 * (i & 1))));
}

// Per-wave LDS.  `ls` holds the logits of the wave's tokens, [h][t]; then
// each head's row holds the probabilities times 4^-(t%4) as two fp16 parts,
// hi at halves [0, 256) and lo at [kPLo, kPLo + 256) of the row, at token
// slot pslot(t); at the end, aliased, the wave's unnormalised output [h][D].
// `sv` / `zv` hold the value scales and zero-points per 16-channel group,
// [g16][pslot(t)] (a value group of more than 16 channels repeats its
// scale in each of its 16-channel parts).  Row strides are padded so that
// rows read by different lanes fall in different LDS banks.
constexpr int kLsStride = kMaxWaveChunk + 4;      // floats
constexpr int kSvStride = kMaxWaveChunk + 8;      // halves
constexpr int kPLo = kMaxWaveChunk + 8;           // halves: lo parts (16-byte aligned)
static_assert(kPLo + kMaxWaveChunk <= 2 * kLsStride, "both parts fit a row");
// Token t's slot: within each 16-token block, tokens t and t + 8 side by
// side, so that one dword holds the pair (t, t + 8) that a value B-operand
// dword takes (its low and high half).
__device__ __forceinline__ int pslot(int t) {
    return (t & ~15) | ((t & 7) << 1) | ((t >> 3) & 1);
}
template <int D, int G>
struct alignas(16) WaveLds {
    static constexpr int NG16 = D / 16;
    float ls[G * kLsStride];
    half_t sv[NG16 * kSvStride];
    half_t zv[NG16 * kSvStride];
    float bias[16 * G];                           // key z terms [group][h]
};

// ------------------------------------------------------ packed tokens
// Tokens [t0, t0 + nt) of the packed region; t0 and nt are multiples of Gk
// and of 16, nt <= kMaxWaveChunk.
//
// Phase K: all logits of the wave's tokens, in batches of 64 (four 16-token
// tiles); the key words of the next batch are loaded while a batch is
// multiplied.  Softmax: the wave's maxima, the probabilities and the value
// meta are staged in LDS.  Phase V: NPASS passes over the value channels;
// pass P covers 16-channel groups [P*GPP, (P+1)*GPP) for every head, so its
// 16 B-operand columns are exactly the (head, group) pairs its rows need.
//
// ONE: the wave holds at most 64 tokens (one key batch, two value steps).
// Its value meta and every value word are then requested at the start,
// together with the key loads, so the wave waits for memory once instead
// of once per phase; this is the form for small calls, whose time is the
// latency of that chain rather than bandwidth.
//
// KP, VP: 2-bit planes of the key and value codes (1: INT2; 2: 4-bit codes,
// combined into one code operand; KP 4: 8-bit keys as a low and a high
// 4-bit operand with their own accumulators, logit = low + 16 high).
// SL: the instance for a full wave share (straight-line steps; SLF below
// names the forms that have it).
template <int D, int G, bool FULLV, bool ONE, bool MASS, int KP = 1, int VP = 1, bool SL = false>
__device__ __forceinline__ void packed_wave(const DecArgs &a, int unit, int t0,
                                            int nt, WaveLds<D, G> &L,
                                            float *m_out, float *l_out) {
    static_assert(!ONE || (KP == 1 && VP == 1), "single-batch form is INT2 only");
    constexpr int KB = D / 32;                    // key k-blocks
    constexpr int KW = D / 16;                    // key words per token
    constexpr int NG16 = D / 16;                  // 16-channel value groups
    constexpr int NG = 16 / G;                    // key groups per B operand
    // tokens per key batch (within one key operand: 256 / G >= BT); planes
    // multiply the key words held per batch, so those batches are halved
    constexpr int BT = (G == 8 || KP > 1) ? 32 : 64;
    constexpr int TPB = BT / 16;                  // key tiles per batch
    constexpr int NPASS = (G * NG16 + 15) / 16;   // value passes
    constexpr int GPP = NG16 / NPASS;             // value groups per pass
    constexpr int MBP = GPP;                      // row blocks per pass
    constexpr int CP = D / NPASS;                 // channels per pass
    const CacheView &c = a.c;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, qd = lane >> 4;
    const int Gk = c.Gk;
    const int gk_sh = __builtin_ctz(Gk);          // Gk is a power of two
    constexpr int NG_SH = G == 1 ? 4 : G == 2 ? 3 : G == 4 ? 2 : 1;   // log2(16 / G)
    const int NGV = D / c.Gv;                     // stored value groups
    const uint16_t *qu = a.q + (size_t)unit * G * D;
    const uint32_t *kq = reinterpret_cast<const uint32_t *>(c.kq) +
                         (size_t)unit * c.kq_unit();
    const size_t kpl = c.kplane(), vpl = c.vplane();
    const uint16_t *ks = c.ks + (size_t)unit * c.km_unit();
    const uint16_t *kz = c.kz + (size_t)unit * c.km_unit();
    const uint32_t *vq = reinterpret_cast<const uint32_t *>(c.vq) +
                         (size_t)unit * c.vq_unit();
    const uint16_t *vs = c.vs + (size_t)unit * c.vm_unit();
    const uint16_t *vz = c.vz + (size_t)unit * c.vm_unit();
    const int g_first = t0 >> gk_sh;
    const int n_grp = nt >> gk_sh;
    // (a full share, SL, has every batch: nt > kMaxWaveChunk - 32); the
    // 2-bit form takes them as straight-line code (the 4-bit forms measured
    // slower so)
    constexpr bool SLK = SL && KP == 1 && VP == 1;
    const int nbatch = SLK ? kMaxWaveChunk / BT : (nt + BT - 1) / BT;
    const int bb_sh = NG_SH + gk_sh;
    const int bblk = 1 << bb_sh;                  // tokens per key B operand (NG Gk)
    const int last = (nbatch - 1) * BT;           // start of the last batch

    // ---- key B operand columns: column r = (group r / G of the operand,
    // head r % G); k-slot (i, hf) of k-block kb is channel
    // 16 w + 4 (qd & 1) + i + 8 hf with w = (qd >> 1) KB + kb.
    const int hk = r % G;
    const int gcol = r / G;

    // ---- this lane's q channels, k-block kb, halves hf = 0, 1 (requested
    // here, used after the first key loads are issued)
    uint2 qx[KB][2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int w = (qd >> 1) * KB + kb;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
            qx[kb][hf] = *reinterpret_cast<const uint2 *>(
                qu + (size_t)hk * D + 16 * w + 4 * (qd & 1) + 8 * hf);
    }
    uint32_t qh[KB][4];                           // q 2^(-e-2i), set below
    float kfac, zfac;                             // logit and z-term factors

    // ---- loaders (indices clamped, never predicated)
    uint2 ksr[KB][2];                             // key scales of a B operand
    // the lane's channels within a scale row, in bytes
    const uint32_t ks_lane = (uint32_t)(16 * (qd >> 1) * KB + 4 * (qd & 1)) * 2u;
    auto load_kscale = [&](int tok) {             // B operand holding tok
        const int gb = (tok >> bb_sh) << NG_SH;   // uniform
        // the operand's row of this lane's column (the last row past the end)
        const uint32_t off = (uint32_t)min(gcol, n_grp - 1 - gb) * (uint32_t)(D * 2) + ks_lane;
        const char *rowp = reinterpret_cast<const char *>(ks + (size_t)(g_first + gb) * D) + off;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                ksr[kb][hf] = *reinterpret_cast<const uint2 *>(rowp + 2 * (16 * kb + 8 * hf));
    };
    // key zeros, rows = the 16 groups of the window [16 m, 16 m + 16) of
    // wave-relative groups that holds tok's group (a window spans 16 / NG key
    // operands, so its z terms are computed once for all of them)
    uint2 kzr[KB][2];
    auto load_kzero = [&](int tok) {
        const int gz = g_first + min(((tok >> gk_sh) & ~15) + r, n_grp - 1);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int w = (qd >> 1) * KB + kb;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                kzr[kb][hf] = *reinterpret_cast<const uint2 *>(
                    kz + (size_t)gz * D + 16 * w + 4 * (qd & 1) + 8 * hf);
        }
    };
    typedef uint32_t KWords[KP][TPB][KB];         // key words of a batch
    KWords kw;
    // tile j's words of the batch at tok: the tile's first row is uniform
    // (a tile past the end takes the last tile's rows, never read), the
    // lane's row and k-block a fixed offset
    const uint32_t kw_lane = (uint32_t)(r * KW + (qd >> 1) * KB) * 4u;   // bytes
    auto load_ktile = [&](int tok, int j, KWords &kw) {
        const int ts = min(tok + 16 * j, nt - 16);
#pragma unroll
        for (int pl = 0; pl < KP; ++pl) {
            const uint32_t *wp = reinterpret_cast<const uint32_t *>(
                reinterpret_cast<const char *>(kq + pl * kpl + (size_t)(t0 + ts) * KW) + kw_lane);
            if constexpr (KB == 4) {
                const uint4 x = *reinterpret_cast<const uint4 *>(wp);
                kw[pl][j][0] = x.x; kw[pl][j][1] = x.y; kw[pl][j][2] = x.z; kw[pl][j][3] = x.w;
            } else {
                const uint2 x = *reinterpret_cast<const uint2 *>(wp);
                kw[pl][j][0] = x.x; kw[pl][j][1] = x.y;
            }
        }
    };
    auto load_kwords = [&](int tok, KWords &kw) {
#pragma unroll
        for (int j = 0; j < TPB; ++j) load_ktile(tok, j, kw);
    };
    // the key code operand of tile j, k-block kb, from planes pl, pl + 1
    auto key_operand = [&](const KWords &kw, int j, int kb, int pl) -> half8_t {
        const int sh = 8 * (qd & 1);
        if constexpr (KP == 1) return code_operand(kw[0][j][kb] >> sh);
        else return code_operand2(kw[pl][j][kb] >> sh, kw[pl + 1][j][kb] >> sh);
    };

    // key weights (B operand) from the scales in ksr: slot (i, hf) pairs the
    // scales of channels c + i and c + 8 + i, the halves of qh[kb][i]
    half8_t bhi[KB], blo[KB];
    auto build_b = [&]() {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const uint32_t sp[4] = {pair_lo(ksr[kb][0].x, ksr[kb][1].x),
                                    pair_hi(ksr[kb][0].x, ksr[kb][1].x),
                                    pair_lo(ksr[kb][0].y, ksr[kb][1].y),
                                    pair_hi(ksr[kb][0].y, ksr[kb][1].y)};
            u32x4 hw, lw;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t h_, l_;
                two_product2(qh[kb][i], sp[i], h_, l_);
                hw[i] = h_;
                lw[i] = l_;
            }
            bhi[kb] = __builtin_bit_cast(half8_t, hw);
            blo[kb] = __builtin_bit_cast(half8_t, lw);
        }
    };
    // z terms of the operand's groups (rows) for every head (columns), in
    // log2 units, with the key operands' channel order on both sides: z
    // 4^(i-3) (exact unless subnormal; never larger than z) against q
    // 2^(-e-2i), so every product is z q 2^(-e-6)
    auto build_bias = [&]() {
        float4_t cb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const uint32_t zp[4] = {pair_lo(kzr[kb][0].x, kzr[kb][1].x),
                                    pair_hi(kzr[kb][0].x, kzr[kb][1].x),
                                    pair_lo(kzr[kb][0].y, kzr[kb][1].y),
                                    pair_hi(kzr[kb][0].y, kzr[kb][1].y)};
            u32x4 zb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half_t f = (half_t)(1.f / (float)(1 << (6 - 2 * i)));
                const half2_t ff = {f, f};
                zb[i] = i == 3 ? zp[i]
                               : __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, zp[i]) * ff);
            }
            const u32x4 qv = {qh[kb][0], qh[kb][1], qh[kb][2], qh[kb][3]};
            cb = mfma16(__builtin_bit_cast(half8_t, zb), __builtin_bit_cast(half8_t, qv), cb);
        }
        if (r < G)
#pragma unroll
            for (int i = 0; i < 4; ++i) L.bias[(4 * qd + i) * G + r] = cb[i] * zfac;
    };

    // value meta of the lane's token lane + 64 k (indices clamped)
    constexpr int NK = ONE ? 1 : kMaxWaveChunk / 64;
    constexpr int MW = NG16 / 2;                  // dwords of fp16 per token
    uint32_t msr[NK][MW], mzr[NK][MW];
    auto load_vmeta = [&](int k) {
        const size_t row = (size_t)(t0 + min(lane + 64 * k, nt - 1)) * NGV;
        if constexpr (FULLV && MW == 4) {
            const uint4 xs = *reinterpret_cast<const uint4 *>(vs + row);
            const uint4 xz = *reinterpret_cast<const uint4 *>(vz + row);
            msr[k][0] = xs.x; msr[k][1] = xs.y; msr[k][2] = xs.z; msr[k][3] = xs.w;
            mzr[k][0] = xz.x; mzr[k][1] = xz.y; mzr[k][2] = xz.z; mzr[k][3] = xz.w;
        } else if constexpr (FULLV) {
            const uint2 xs = *reinterpret_cast<const uint2 *>(vs + row);
            const uint2 xz = *reinterpret_cast<const uint2 *>(vz + row);
            msr[k][0] = xs.x; msr[k][1] = xs.y;
            mzr[k][0] = xz.x; mzr[k][1] = xz.y;
        } else {
            // value groups of Gv > 16 channels: repeat per 16-channel part
            const int per = NG16 / NGV;
#pragma unroll
            for (int j = 0; j < MW; ++j) {
                msr[k][j] = (uint32_t)vs[row + (2 * j) / per] |
                            ((uint32_t)vs[row + (2 * j + 1) / per] << 16);
                mzr[k][j] = (uint32_t)vz[row + (2 * j) / per] |
                            ((uint32_t)vz[row + (2 * j + 1) / per] << 16);
            }
        }
    };
    // value words of pass P, 32-token step st: channels P CP + r MBP + mb
    // of the 16-token block that lane quarter qd >> 1 multiplies
    const int last_blk = (t0 + nt) / 16 - 1;
    // (vw holds VP planes of MBP words: vw[pl * MBP + mb])
    auto load_vw = [&](int P, int st, uint32_t *vw) {
        const int blk = min((t0 + st) / 16 + (qd >> 1), last_blk);
#pragma unroll
        for (int pl = 0; pl < VP; ++pl) {
            const uint32_t *wp = vq + pl * vpl + (uint32_t)(blk * D + P * CP + r * MBP);
            uint32_t *w = vw + pl * MBP;
            if constexpr (MBP == 8) {
                const uint4 x0 = *reinterpret_cast<const uint4 *>(wp);
                const uint4 x1 = *reinterpret_cast<const uint4 *>(wp + 4);
                w[0] = x0.x; w[1] = x0.y; w[2] = x0.z; w[3] = x0.w;
                w[4] = x1.x; w[5] = x1.y; w[6] = x1.z; w[7] = x1.w;
            } else if constexpr (MBP == 4) {
                const uint4 x0 = *reinterpret_cast<const uint4 *>(wp);
                w[0] = x0.x; w[1] = x0.y; w[2] = x0.z; w[3] = x0.w;
            } else if constexpr (MBP == 2) {
                const uint2 x0 = *reinterpret_cast<const uint2 *>(wp);
                w[0] = x0.x; w[1] = x0.y;
            } else {
                w[0] = wp[0];
            }
        }
    };

    // ============================================================ phase K
    // the first batch's key loads go out with q's, so they share its trip
    __builtin_amdgcn_sched_barrier(0);
    load_kscale(0);
    load_kzero(0);
    __builtin_amdgcn_sched_barrier(0);
    load_kwords(0, kw);
    __builtin_amdgcn_sched_barrier(0);
    constexpr int NVE = ONE ? 2 : 1;              // value steps held early
    uint32_t vwe[NPASS][NVE][MBP * VP];
    if constexpr (ONE) {
        static_assert(BT == 64, "one key batch must cover the wave's tokens");
        load_vmeta(0);
#pragma unroll
        for (int P = 0; P < NPASS; ++P)
#pragma unroll
            for (int e = 0; e < NVE; ++e) load_vw(P, 32 * e, vwe[P][e]);
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- q as fp16 pairs (hf = 0, 1) per (kb, i), in the k-slot order of
    // the key operands; the power of two 2^e > max |q_h| per head; then
    // q 2^(-e-2i) in place.
    float qmax = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const uint32_t a0[2] = {qx[kb][0].x, qx[kb][0].y}, a1[2] = {qx[kb][1].x, qx[kb][1].y};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = (a0[i >> 1] >> (16 * (i & 1))) & 0xffffu;
            const uint32_t hi = (a1[i >> 1] >> (16 * (i & 1))) & 0xffffu;
            qh[kb][i] = lo | (hi << 16);
            qmax = fmaxf(qmax, fmaxf(fabsf(h2f((uint16_t)lo)), fabsf(h2f((uint16_t)hi))));
        }
    }
    qmax = xor32_max(xor16_max(qmax));
    // any e with 2^e > max |q| keeps |q 2^-e| < 1; e >= -8 keeps the factors
    // 2^(-e-2i) within fp16
    const int qe = max(__builtin_amdgcn_frexp_expf(qmax), -8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half_t f = (half_t)__builtin_amdgcn_ldexpf(1.f, -qe - 2 * i);   // exact
        const half2_t ff = {f, f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            qh[kb][i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, qh[kb][i]) * ff);
    }
    // logit (log2 units) = (acc * 2^(24 + e) + z term) * qscale
    kfac = __builtin_amdgcn_ldexpf(a.qscale, 24 + qe);
    // the z terms' MFMA takes z 4^(i-3) against q 2^(-e-2i)
    zfac = __builtin_amdgcn_ldexpf(a.qscale, 6 + qe);

    if constexpr (G == 1) {                       // 16 groups cover the wave
        build_b();
        build_bias();
        wave_lds_sync();
    }
    float mloc = -INFINITY;
    // With 16-token key groups, column group T of a key operand belongs to
    // the operand's tile T, so each lane keeps the accumulator of its own
    // column's tile (a select per tile) and the logit epilogue runs once per
    // operand on every lane instead of once per tile on a fraction of them.
    const bool per_lane = Gk == 16;               // uniform
    float4_t keep = {0.f, 0.f, 0.f, 0.f};
    auto store_logits = [&](const float4_t &acc, float bz, int tt) {
        float4_t lg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lg[i] = __builtin_fmaf(acc[i], kfac, bz);
            mloc = fmaxf(mloc, lg[i]);
        }
        *reinterpret_cast<float4_t *>(&L.ls[hk * kLsStride + tt + 4 * qd]) = lg;
        if constexpr (MASS)                       // the mass audit's logits
            *reinterpret_cast<float4_t *>(
                a.lg + ((size_t)unit * G + hk) * a.lg_stride + t0 + tt + 4 * qd) = lg;
    };
    // PF (GQA, several batches): the last key batch requests the value meta
    // and the first two value steps where the other batches request the next
    // batch's keys, so phase V's first loads overlap the last logits (these
    // kernels have the registers to spare at their occupancy).
    constexpr bool PF = G > 1 && !ONE && KP < 4;
    const int nt32 = (nt + 31) & ~31;
    // Value words: NVB steps in flight, in buffer step mod NVB (A even
    // steps, B odd when NVB = 2).  A full wave share (nt32 = kMaxWaveChunk)
    // of the forms SLF names runs as its own instance (SL), whose value
    // steps, and for 2-bit codes key batches, are straight-line code: in
    // one instance with the loop form, the register allocator moved the
    // value buffers where the two paths part, and a copy of a register whose
    // load is still in flight waits for every load.
    // SLF: 16-channel value groups and keys of at most 4 bits with several
    // value passes (wider value groups spilled in this instance, 8-bit keys
    // measured slower; those keep the pair steps below in one instance), or
    // g = 1 with 2-bit codes (four waves per SIMD without the mass audit's
    // stores; its 4-bit forms measured slower).
    constexpr bool SLF = FULLV && !ONE && KP < 4 &&
                         (NPASS > 1 || (G == 1 && !MASS && KP == 1 && VP == 1));
    static_assert(!SL || SLF, "straight-line form: see SLF");
    // 4-bit values three buffers; 2-bit values two (three or four measured
    // slower)
    constexpr int NVB = SL && VP == 2 ? 3 : 2;
    uint32_t vwS[NVB][NPASS][MBP * VP];
    uint32_t(&vwA)[NPASS][MBP * VP] = vwS[0];
    uint32_t(&vwB)[NPASS][MBP * VP] = vwS[1];
    auto load_v_first = [&]() {
#pragma unroll
        for (int k = 0; k < NK; ++k) load_vmeta(k);
#pragma unroll
        for (int P = 0; P < NPASS; ++P) load_vw(P, 0, vwA[P]);
#pragma unroll
        for (int P = 0; P < NPASS; ++P) load_vw(P, min(32, nt32 - 32), vwB[P]);
        if constexpr (SL)
#pragma unroll
            for (int e = 2; e < NVB; ++e)
#pragma unroll
                for (int P = 0; P < NPASS; ++P) load_vw(P, 32 * e, vwS[e][P]);
    };
    // One key batch.  The next batch's words of tile j are requested into
    // tile j's registers as soon as its MFMAs have read them, so each tile's
    // words have one batch of work to arrive.
    auto kbatch = [&](int b, auto lastb) {
        constexpr bool LASTB = decltype(lastb)::value;
        const int tok = b * BT;                   // wave-relative
        const int nxt = min(tok + BT, last);      // next batch (clamped)
        const int gb = (tok >> bb_sh) << NG_SH;   // first group of the operand
        const int gw = gb & 15;                   // its row in the z-term window
        if constexpr (G > 1) {
            if ((tok & (bblk - 1)) == 0) {        // a new key operand
                build_b();
                if (gw == 0) build_bias();        // a new window
                wave_lds_sync();
            }
            if constexpr (!ONE) {
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (LASTB) {
                    load_v_first();
                } else {
                    load_kscale(nxt);
                    if (((nxt >> gk_sh) ^ (tok >> gk_sh)) & ~15) load_kzero(nxt);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int j = 0; j < TPB; ++j) {
            // tiles past the end use clamped rows and are never read
            const int tl = min(tok + 16 * j, nt - 16);
            float4_t acc = {0.f, 0.f, 0.f, 0.f};
            half8_t av[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) av[kb] = key_operand(kw, j, kb, 0);
            if constexpr (!ONE && KP < 4 && !LASTB) {
                __builtin_amdgcn_sched_barrier(0);
                load_ktile(nxt, j, kw);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                acc = mfma16(av[kb], bhi[kb], acc);
                acc = mfma16(av[kb], blo[kb], acc);
            }
            if constexpr (KP == 4) {              // the high 4 bits of 8-bit codes
                float4_t acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const half8_t av2 = key_operand(kw, j, kb, 2);
                    acc2 = mfma16(av2, bhi[kb], acc2);
                    acc2 = mfma16(av2, blo[kb], acc2);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(acc2[i], 16.f, acc[i]);
            }
            const int grp = (tl >> gk_sh) - gb;   // the tile's column group
            if (per_lane) {                       // a select, not a branch
                const bool take = tok + 16 * j < nt && gcol == grp;
#pragma unroll
                for (int i = 0; i < 4; ++i) keep[i] = take ? acc[i] : keep[i];
            } else if (gcol == grp && tok + 16 * j < nt) {
                store_logits(acc, L.bias[(gw + grp) * G + hk], tok + 16 * j);
            }
        }
        // the operand's last batch: the kept tiles' logits
        if (per_lane && (((tok + BT) & (bblk - 1)) == 0 || tok + BT >= nt)) {
            const int tt = (tok & ~(bblk - 1)) + 16 * gcol;
            if (tt < nt) store_logits(keep, L.bias[(gw + gcol) * G + hk], tt);
        }
        if constexpr (!ONE && KP == 4) {          // four planes: all at the end
            __builtin_amdgcn_sched_barrier(0);
            load_kwords(nxt, kw);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if constexpr (PF) {
        if constexpr (SLK) {
            // straight-line batches
#pragma unroll
            for (int b = 0; b + 1 < kMaxWaveChunk / BT; ++b) kbatch(b, std::false_type{});
        } else {
            for (int b = 0; b + 1 < nbatch; ++b) kbatch(b, std::false_type{});
        }
        kbatch(nbatch - 1, std::true_type{});
    } else {
        for (int b = 0; b < nbatch; ++b) kbatch(b, std::false_type{});
    }

    // ================================================== softmax, staging
    mloc = strided_max<G>(mloc);                  // lane l: head l % G
    float m_h[G], l_h[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_h[h] = __builtin_amdgcn_readlane(mloc, h);
        l_h[h] = 0.f;
    }
    wave_lds_sync();
    // the value meta of all of this lane's tokens (t = lane + 64 k), loads
    // issued together so that their latencies overlap
    if constexpr (!ONE && !PF)
#pragma unroll
        for (int k = 0; k < NK; ++k) load_vmeta(k);
    // every logit of the lane's tokens is read first (one LDS wait, not one
    // per token and head); slots past the wave's tokens hold stale values
    // that only meet a select, and slots past nt32 are never read by phase V
    float lgv[NK][G];
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
        for (int h = 0; h < G; ++h) lgv[k][h] = L.ls[h * kLsStride + lane + 64 * k];
    // (an empty asm use keeps the reads here rather than sunk into the
    // token loop below, one wait per 64 tokens)
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
        for (int h = 0; h < G; ++h) asm volatile("" : : "v"(lgv[k][h]));
    // (every logit is in registers now, so the rows can take the fp16
    // parts, at other slots, without overwriting an unread logit)
    half_ma *const ph = reinterpret_cast<half_ma *>(L.ls);
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        const int t = lane + 64 * k;
        if (64 * k >= nt32) break;                // uniform
        const bool ok = t < nt;
        const int ps = pslot(t);
        const float q4 = __builtin_amdgcn_ldexpf(1.f, -2 * (t & 3));
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float p = ok ? __builtin_amdgcn_exp2f(lgv[k][h] - m_h[h]) : 0.f;
            l_h[h] += p;
            // p 4^-i as hi + lo: hi rounded to fp16, lo = the exact fp32
            // remainder rounded to fp16
            const float w = p * q4;
            const half_t whi = (half_t)w;
            ph[h * 2 * kLsStride + ps] = whi;
            ph[h * 2 * kLsStride + kPLo + ps] = (half_t)(w - (float)whi);
        }
#pragma unroll
        for (int j = 0; j < MW; ++j) {
            const uint32_t sw = ok ? msr[k][j] : 0u, zw = ok ? mzr[k][j] : 0u;
            L.sv[(2 * j) * kSvStride + ps] = __builtin_bit_cast(half_t, (uint16_t)(sw & 0xffffu));
            L.sv[(2 * j + 1) * kSvStride + ps] = __builtin_bit_cast(half_t, (uint16_t)(sw >> 16));
            L.zv[(2 * j) * kSvStride + ps] = __builtin_bit_cast(half_t, (uint16_t)(zw & 0xffffu));
            L.zv[(2 * j + 1) * kSvStride + ps] = __builtin_bit_cast(half_t, (uint16_t)(zw >> 16));
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) l_h[h] = wave_sum(l_h[h]);
    wave_lds_sync();

    // ============================================================ phase V
    // token slots of this lane in a 32-token step: tb + i, tb + 8 + i
    const int tb = 16 * (qd >> 1) + 4 * (qd & 1);
    // Column r of pass P is (head r / GPP, group P GPP + r % GPP): the head
    // does not depend on the pass, so every pass of a step shares the
    // lane's probabilities, and the passes run inside one walk over the
    // steps (one chain of dependent value loads, not NPASS of them).
    const int hc = min(r / GPP, G - 1);
    float4_t outv[NPASS][MBP];                    // kept columns, see below
    float za[NPASS][4];
#pragma unroll
    for (int P = 0; P < NPASS; ++P) {
#pragma unroll
        for (int mb = 0; mb < MBP; ++mb) outv[P][mb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) za[P][i] = 0.f;
    }
    const int nsteps = nt32 >> 5;
    // one 32-token step of every pass; `code(P, mb)` gives the step's value
    // word, `after(P)` runs once the pass's words are in code operands.  A
    // step with `live` false (the padding step of an odd count) re-reads
    // the last step's LDS rows and multiplies with zero probabilities, so
    // it adds exactly nothing; the step pair then has no branch, and the
    // loads two steps ahead keep their place in the wait counts.
    // the lane's 8 token slots of a step: tokens tb + i and tb + 8 + i side
    // by side (pslot), as dword i of its B operand takes them
    const int pb0 = 16 * (qd >> 1) + 8 * (qd & 1);
    const half_ma *const phr = reinterpret_cast<const half_ma *>(L.ls) + hc * 2 * kLsStride;
    auto step = [&](int e, bool live, auto &&code, auto &&after) {
        const int pb = 32 * min(e, nsteps - 1) + pb0;
        const half8_t phv = *reinterpret_cast<const half8_t *>(phr + pb);
        const half8_t plv = *reinterpret_cast<const half8_t *>(phr + kPLo + pb);
        u32x4 phi = __builtin_bit_cast(u32x4, phv);
        u32x4 plo = __builtin_bit_cast(u32x4, plv);
        // several passes: every pass's scale and zero reads up front, so the
        // step waits for LDS once
        u32x4 svh[NPASS], zvh[NPASS];
        auto read_meta = [&](int P) {
            const int vg = P * GPP + r % GPP;
            svh[P] = *reinterpret_cast<const u32x4_ma *>(&L.sv[vg * kSvStride + pb]);
            zvh[P] = *reinterpret_cast<const u32x4_ma *>(&L.zv[vg * kSvStride + pb]);
        };
        if constexpr (NPASS > 1)
#pragma unroll
            for (int P = 0; P < NPASS; ++P) read_meta(P);
        if (!live) {
            phi = u32x4{0u, 0u, 0u, 0u};
            plo = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int P = 0; P < NPASS; ++P) {
            half8_t av[MBP];
#pragma unroll
            for (int mb = 0; mb < MBP; ++mb) {
                if constexpr (VP == 1)
                    av[mb] = code_operand(code(P, mb) >> (8 * (qd & 1)));
                else
                    av[mb] = code_operand2(code(P, mb) >> (8 * (qd & 1)),
                                           code(P, MBP + mb) >> (8 * (qd & 1)));
            }
            after(P);
            if constexpr (NPASS == 1) read_meta(P);
            u32x4 bhw, blw;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // weights (p 4^-i) s as hi + lo: the TwoProduct of the hi
                // part and s, plus the lo part times s
                // (each vector element copied out first: a bit cast of an
                // element of a vector-typed value reads element 0)
                const uint32_t ahw = phi[i], alw = plo[i], scw = svh[P][i], zcw = zvh[P][i];
                const half2_t ah = __builtin_bit_cast(half2_t, ahw);
                const half2_t al = __builtin_bit_cast(half2_t, alw);
                const half2_t sc = __builtin_bit_cast(half2_t, scw);
                const half2_t zc = __builtin_bit_cast(half2_t, zcw);
                const half2_t wh = ah * sc;
                const half2_t wl = __builtin_elementwise_fma(
                    al, sc, __builtin_elementwise_fma(ah, sc, -wh));
                bhw[i] = __builtin_bit_cast(uint32_t, wh);
                blw[i] = __builtin_bit_cast(uint32_t, wl);
                // p is stored times 4^-i: keep one z sum per i
                za[P][i] = __builtin_amdgcn_fdot2(ah, zc, za[P][i], false);
                za[P][i] = __builtin_amdgcn_fdot2(al, zc, za[P][i], false);
            }
            const half8_t bh = __builtin_bit_cast(half8_t, bhw);
            const half8_t bl = __builtin_bit_cast(half8_t, blw);
#pragma unroll
            for (int mb = 0; mb < MBP; ++mb) {
                outv[P][mb] = mfma16(av[mb], bh, outv[P][mb]);
                outv[P][mb] = mfma16(av[mb], bl, outv[P][mb]);
            }
        }
    };
    if constexpr (ONE) {
#pragma unroll
        for (int e = 0; e < NVE; ++e) {
            if (e >= nsteps) break;               // uniform
            step(e, true, [&](int P, int mb) { return vwe[P][e][mb]; }, [](int) {});
        }
    } else {
        // value words two steps ahead: buffer A holds even steps, B odd
        // (issued A before B, as the loop issues them, so that the waits
        // at the loop's top, which merge this order with the loop's own,
        // leave B's words in flight while A's are used)
        if constexpr (!PF) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int P = 0; P < NPASS; ++P) load_vw(P, 0, vwA[P]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int P = 0; P < NPASS; ++P) load_vw(P, min(32, nt32 - 32), vwB[P]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (SL)
#pragma unroll
                for (int e = 2; e < NVB; ++e) {
#pragma unroll
                    for (int P = 0; P < NPASS; ++P) load_vw(P, 32 * e, vwS[e][P]);
                    __builtin_amdgcn_sched_barrier(0);
                }
        }
        auto pair = [&](int e, bool full) {
            step(e, true, [&](int P, int mb) { return vwA[P][mb]; }, [&](int P) {
                __builtin_amdgcn_sched_barrier(0);
                load_vw(P, min(32 * (e + 2), nt32 - 32), vwA[P]);
                __builtin_amdgcn_sched_barrier(0);
            });
            step(e + 1, full || e + 1 < nsteps, [&](int P, int mb) { return vwB[P][mb]; }, [&](int P) {
                __builtin_amdgcn_sched_barrier(0);
                load_vw(P, min(32 * (e + 3), nt32 - 32), vwB[P]);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        // step e of the straight-line form: its words in buffer e mod NVB,
        // which then takes step e + NVB's
        auto tri = [&](auto ec) {
            constexpr int e = decltype(ec)::value;
            uint32_t(&buf)[NPASS][MBP * VP] = vwS[e % NVB];
            step(e, true, [&](int P, int mb) { return buf[P][mb]; }, [&](int P) {
                if constexpr (e + NVB < kMaxWaveChunk / 32) {
                    __builtin_amdgcn_sched_barrier(0);
                    load_vw(P, 32 * (e + NVB), buf[P]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
        };
        if constexpr (SL) {
            // a full wave share: straight-line steps, so each wait for the
            // value words leaves the next steps' loads in flight
            tri(std::integral_constant<int, 0>{});
            tri(std::integral_constant<int, 1>{});
            tri(std::integral_constant<int, 2>{});
            tri(std::integral_constant<int, 3>{});
            tri(std::integral_constant<int, 4>{});
            tri(std::integral_constant<int, 5>{});
            tri(std::integral_constant<int, 6>{});
            tri(std::integral_constant<int, 7>{});
        } else if (!SLF && NPASS > 1 && nsteps == kMaxWaveChunk / 32) {
            // the same two steps ahead (A / B), straight-line
#pragma unroll
            for (int e = 0; e < kMaxWaveChunk / 32; e += 2) pair(e, true);
        } else {
            for (int e = 0; e < nsteps; e += 2) pair(e, false);
        }
    }
    float zsum[NPASS];
#pragma unroll
    for (int P = 0; P < NPASS; ++P) {
        float zt = za[P][0] + __builtin_amdgcn_ldexpf(za[P][1], 2) +
                   __builtin_amdgcn_ldexpf(za[P][2], 4) + __builtin_amdgcn_ldexpf(za[P][3], 6);
        zt = xor32_sum(xor16_sum(zt));
        zsum[P] = zt;
    }
    wave_lds_sync();
    // keep, for each channel row, the column of its own group; the wave's
    // output [h][D] overwrites its probabilities
    float *out = L.ls;
#pragma unroll
    for (int P = 0; P < NPASS; ++P) {
        if (r < G * GPP) {
            const int h = r / GPP, vg = P * GPP + r % GPP;
#pragma unroll
            for (int mb = 0; mb < MBP; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ch = P * CP + (4 * qd + i) * MBP + mb;
                    if (ch / 16 == vg)
                        out[h * D + ch] = __builtin_fmaf(outv[P][mb][i], 16777216.f, zsum[P]);
                }
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_out[h] = m_h[h];
        l_out[h] = l_h[h];
    }
}

// ------------------------------------------------------ fp16 residual
// Tokens [t0, t0 + nt) of the residual, 1 <= nt <= 64.  Logits: 16 lanes
// per token (D/16 channels each), four tokens per pass; P.V: the same lanes
// over the same passes, the four token phases summed at the end.  The loads
// of a batch of passes are all issued before their first use.
template <int D, int G, bool MASS>
__device__ __forceinline__ void residual_wave(const DecArgs &a, int unit, int t0,
                                              int nt, WaveLds<D, G> &L,
                                              float *m_out, float *l_out) {
    constexpr int CPL = D / 16;                   // channels per lane
    constexpr int PB = 8;                         // passes per load batch
    const CacheView &c = a.c;
    const int lane = threadIdx.x & 63;
    const int part = lane & 15, ph = lane >> 4;
    const uint16_t *qu = a.q + (size_t)unit * G * D;
    const uint16_t *kr = c.kres + (size_t)unit * c.res_unit();
    const uint16_t *vr = c.vres + (size_t)unit * c.res_unit();
    const uint16_t *kn = a.k_new ? a.k_new + (size_t)unit * D : nullptr;
    const uint16_t *vn = a.v_new ? a.v_new + (size_t)unit * D : nullptr;
    auto row_ptr = [&](const uint16_t *res, const uint16_t *nw, int slot) {
        return (nw && slot == a.new_slot) ? nw : res + (size_t)slot * D;
    };
    auto load_row = [&](const uint16_t *p, float *f) {
        if constexpr (CPL == 8) {
            unpack8h(*reinterpret_cast<const uint4 *>(p + CPL * part), f);
        } else {
            const uint2 x = *reinterpret_cast<const uint2 *>(p + CPL * part);
            const uint32_t w[2] = {x.x, x.y};
#pragma unroll
            for (int i = 0; i < 4; ++i) f[i] = h2f((uint16_t)(w[i >> 1] >> (16 * (i & 1))));
        }
    };

    float qv[G][CPL];
#pragma unroll
    for (int h = 0; h < G; ++h) load_row(qu + h * D, qv[h]);

    float mloc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) mloc[h] = -INFINITY;
    const int npass = (nt + 3) / 4;
    for (int p0 = 0; p0 < npass; p0 += PB) {
        float kf[PB][CPL];
#pragma unroll
        for (int b = 0; b < PB; ++b) {
            const int t = min((p0 + b) * 4 + ph, nt - 1);
            load_row(row_ptr(kr, kn, t0 + t), kf[b]);
        }
#pragma unroll
        for (int b = 0; b < PB; ++b) {
            const int t = (p0 + b) * 4 + ph;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < CPL; ++i) s += qv[h][i] * kf[b][i];
                s = row16_sum(s) * a.qscale;
                if (t < nt) {
                    mloc[h] = fmaxf(mloc[h], s);
                    if (part == 0) {
                        L.ls[h * kLsStride + t] = s;
                        if constexpr (MASS)       // the mass audit's logits
                            a.lg[((size_t)unit * G + h) * a.lg_stride + a.n_packed + t0 + t] = s;
                    }
                }
            }
        }
    }
    float m_h[G], l_h[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float m = mloc[h];
        m = xor32_max(xor16_max(m));
        m_h[h] = m;
        l_h[h] = 0.f;
    }
    wave_lds_sync();
    for (int t = lane; t < nt; t += 64)
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float p = __builtin_amdgcn_exp2f(L.ls[h * kLsStride + t] - m_h[h]);
            L.ls[h * kLsStride + t] = p;
            l_h[h] += p;
        }
#pragma unroll
    for (int h = 0; h < G; ++h) l_h[h] = wave_sum(l_h[h]);
    wave_lds_sync();

    float o[G][CPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < CPL; ++i) o[h][i] = 0.f;
    for (int p0 = 0; p0 < npass; p0 += PB) {
        float vf[PB][CPL];
#pragma unroll
        for (int b = 0; b < PB; ++b) {
            const int t = min((p0 + b) * 4 + ph, nt - 1);
            load_row(row_ptr(vr, vn, t0 + t), vf[b]);
        }
#pragma unroll
        for (int b = 0; b < PB; ++b) {
            const int t = (p0 + b) * 4 + ph;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float p = t < nt ? L.ls[h * kLsStride + min(t, nt - 1)] : 0.f;
#pragma unroll
                for (int i = 0; i < CPL; ++i) o[h][i] += p * vf[b][i];
            }
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            float v = o[h][i];
            v = xor32_sum(xor16_sum(v));
            o[h][i] = v;
        }
    wave_lds_sync();
    if (ph == 0)
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < CPL; ++i) L.ls[h * D + CPL * part + i] = o[h][i];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_out[h] = m_h[h];
        l_out[h] = l_h[h];
    }
}

// FULLV: value channel groups of 16 (D/16 scales per token).
// MASS: also store every token's logit for the persistence audit.
// W: waves per block, each with a chunk / W share of the split's tokens.
// KP, VP: 2-bit planes of the key / value codes (packed_wave).  Blocks per
// SIMD: 4 for the INT2 g = 1 kernel, 2 where the registers need it (g = 2
// and 8, 8-bit keys, 4-bit keys and values at g = 4, which at 3 would
// spill), else 3.
template <int D, int G, bool FULLV, bool ONE, bool MASS, int W = kWaves, int KP = 1,
          int VP = 1>
__global__ __launch_bounds__(W * 64, (G == 2 || G == 8 || KP == 4 || (G == 4 && KP == 2 && VP == 2)) ? 2 : (G == 1 && !ONE && KP == 1 && VP == 1) ? 4 : 3) void decode_kernel(DecArgs a) {
    // x = unit, y = split: with the round-robin dispatch of workgroups over
    // the 8 XCDs, every split of a unit (and its merge below) runs on the
    // XCD unit mod 8 when the unit count is a multiple of 8.
    const int unit = blockIdx.x;
    const int split = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const CacheView &c = a.c;

    __shared__ WaveLds<D, G> lds[W];
    __shared__ float red_ml[W][G][2];

    float m_w[G], l_w[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_w[h] = -INFINITY;
        l_w[h] = 0.f;
    }
    // The fp16 residual runs on waves res_wave0.. of split res_split: the
    // idle waves of the last packed split when they have room, else a split
    // of its own.
    const bool res_role = split == a.res_split && wave >= a.res_wave0;
    if (!res_role && split < a.n_chunks) {
        // a segment with per-unit counts: the grid covers the largest, and
        // this unit's waves past its own count have no tokens
        const int n_packed = c.n_unit ? min(c.n_unit[unit], a.n_packed) : a.n_packed;
        const int wchunk = a.chunk / W;
        const int t0 = split * a.chunk + wave * wchunk;
        const int nt = max(0, min(wchunk, n_packed - t0));
        // a full share (the last 32-token step may be partial) takes the
        // straight-line instance where it exists (SLF in packed_wave)
        constexpr bool SLF = FULLV && !ONE && KP < 4 &&
                             ((G * (D / 16) + 15) / 16 > 1 ||
                              (G == 1 && !MASS && KP == 1 && VP == 1));
        if constexpr (SLF) {
            if (nt > kMaxWaveChunk - 32)
                packed_wave<D, G, FULLV, ONE, MASS, KP, VP, true>(a, unit, t0, nt, lds[wave], m_w, l_w);
            else if (nt > 0)
                packed_wave<D, G, FULLV, ONE, MASS, KP, VP>(a, unit, t0, nt, lds[wave], m_w, l_w);
        } else if (nt > 0) {
            packed_wave<D, G, FULLV, ONE, MASS, KP, VP>(a, unit, t0, nt, lds[wave], m_w, l_w);
        }
    } else if (res_role) {
        const int nrw = W - a.res_wave0, rw = wave - a.res_wave0;
        const int per = (a.n_res + nrw - 1) / nrw;
        const int t0 = rw * per;
        const int nt = max(0, min(per, a.n_res - t0));
        if (nt > 0) residual_wave<D, G, MASS>(a, unit, t0, nt, lds[wave], m_w, l_w);
        // store the new token into its residual slot for later calls
        if (a.k_new && rw == 0 && lane < 2 * (D / 8)) {
            const int part = lane % (D / 8);
            const bool isv = lane >= D / 8;
            const uint16_t *src = (isv ? a.v_new : a.k_new) + (size_t)unit * D;
            uint16_t *dst = (isv ? c.vres : c.kres) + (size_t)unit * c.res_unit() +
                            (size_t)a.new_slot * D;
            reinterpret_cast<uint4 *>(dst)[part] = reinterpret_cast<const uint4 *>(src)[part];
        }
    }
    if (lane == 0)
#pragma unroll
        for (int h = 0; h < G; ++h) {
            red_ml[wave][h][0] = m_w[h];
            red_ml[wave][h][1] = l_w[h];
        }
    __syncthreads();

    // ----------------------------------------- merge the waves, store
    // Every thread reads its head's (max, sum) of all W waves at once (LDS
    // broadcasts, one wait) and takes them with selects, not branches: a
    // chain of dependent LDS reads here would add microseconds to every
    // block's tail.
    const size_t sbase = (size_t)unit * a.nsplit_total + a.split_off + split;
    for (int i = tid; i < G * D; i += (W * 64)) {
        const int h = i / D;
        float mw[W], lw[W], ow[W];
#pragma unroll
        for (int w = 0; w < W; ++w) {
            mw[w] = red_ml[w][h][0];
            lw[w] = red_ml[w][h][1];
            ow[w] = lds[w].ls[i];
        }
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) M = lw[w] > 0.f ? fmaxf(M, mw[w]) : M;
        float v = 0.f, L = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            // a wave without tokens wrote no output: its LDS is not read
            const bool ok = lw[w] > 0.f;
            const float e = ok ? __builtin_amdgcn_exp2f(mw[w] - M) : 0.f;
            v = __builtin_fmaf(ok ? ow[w] : 0.f, e, v);
            L = __builtin_fmaf(lw[w], e, L);
        }
        a.part_o[sbase * G * D + i] = v;
        if (i % D == 0) {
            a.part_ml[(sbase * G + h) * 2 + 0] = M;
            a.part_ml[(sbase * G + h) * 2 + 1] = L;
        }
    }
}

// Merge the splits of one (unit, head): o = sum_s 2^(m_s - M) o_s / L.
// Block (unit, head); thread (slice, channel) takes every SLICES-th split of
// one channel.  It loads a batch of up to NB splits' (max, sum, o) at once
// and folds it into a running (max, sum, o); the slices are then merged in
// LDS.  A workload with at most SLICES * NB splits per unit needs a single
// round trip to memory.
template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(
    const float *__restrict__ part_ml, const float *__restrict__ part_o,
    int nsplit, uint16_t *__restrict__ o, float *__restrict__ ml_out) {
    constexpr int SLICES = kThreads / D;
    constexpr int NB = 8;
    __shared__ float r_m[kThreads], r_l[kThreads], r_o[kThreads];
    const int unit = blockIdx.x;
    const int h = blockIdx.y;
    const int tid = threadIdx.x;
    const int ch = tid % D, slice = tid / D;
    const float *ml = part_ml + (size_t)unit * nsplit * G * 2 + h * 2;
    const float *po = part_o + (size_t)unit * nsplit * G * D + h * D + ch;

    constexpr int STEP = NB * SLICES;
    float m_run = -INFINITY, l_run = 0.f, o_run = 0.f;
    typedef float Batch[3][NB];                   // (max, sum, o) of NB splits
    auto load = [&](int s0, Batch &b) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int s = min(s0 + i * SLICES, nsplit - 1);
            b[0][i] = ml[(size_t)s * G * 2];
            b[1][i] = ml[(size_t)s * G * 2 + 1];
            b[2][i] = po[(size_t)s * G * D];
        }
    };
    // selects, not branches, so that the o loads are not held back behind
    // the (max, sum) ones
    auto fold = [&](int s0, const Batch &b) {
        float mx = m_run;
#pragma unroll
        for (int i = 0; i < NB; ++i)
            mx = (s0 + i * SLICES < nsplit && b[1][i] > 0.f) ? fmaxf(mx, b[0][i]) : mx;
        const float sc = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
        l_run *= sc;
        o_run *= sc;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const bool ok = s0 + i * SLICES < nsplit && b[1][i] > 0.f;
            const float w = ok ? __builtin_amdgcn_exp2f(b[0][i] - mx) : 0.f;
            l_run = __builtin_fmaf(ok ? b[1][i] : 0.f, w, l_run);
            o_run = __builtin_fmaf(ok ? b[2][i] : 0.f, w, o_run);
        }
        m_run = mx;
    };
    // the first two batches are requested together (up to 2 STEP splits in
    // one round trip), any further ones a batch at a time
    Batch b0, b1;
    load(slice, b0);
    const bool two = nsplit > STEP;               // uniform
    if (two) load(slice + STEP, b1);
    fold(slice, b0);
    if (two) fold(slice + STEP, b1);
    for (int s0 = slice + 2 * STEP; s0 < nsplit; s0 += STEP) {
        load(s0, b0);
        fold(s0, b0);
    }
    r_m[tid] = m_run;
    r_l[tid] = l_run;
    r_o[tid] = o_run;
    __syncthreads();
    if (slice == 0) {
        float M = -INFINITY;
        for (int k = 0; k < SLICES; ++k) M = fmaxf(M, r_m[k * D + ch]);
        float L = 0.f, acc = 0.f;
        for (int k = 0; k < SLICES; ++k) {
            if (r_l[k * D + ch] > 0.f) {
                const float w = __builtin_amdgcn_exp2f(r_m[k * D + ch] - M);
                L += r_l[k * D + ch] * w;
                acc += r_o[k * D + ch] * w;
            }
        }
        o[((size_t)unit * G + h) * D + ch] = f2h_bits(acc / L);
        if (ml_out && ch == 0) {          // the mass audit's normaliser
            ml_out[((size_t)unit * G + h) * 2 + 0] = M;
            ml_out[((size_t)unit * G + h) * 2 + 1] = L;
        }
    }
}

// Persistence audit: mass[unit][t] += sum over the unit's g heads of the
// attention weight 2^(logit - M) / L of cache token t, with the logits the
// decode kernels stored and each head's final (M, L) from the combine.
// One thread per token; every token is written once, so it is
// deterministic.
template <int G>
__global__ __launch_bounds__(kThreads) void decode_mass_kernel(
    const float *__restrict__ lg, int lg_stride, const float *__restrict__ ml,
    int n_tok, float *__restrict__ mass, int mass_stride) {
    const int unit = blockIdx.x;
    const int t = blockIdx.y * kThreads + threadIdx.x;
    if (t >= n_tok) return;
    float w = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float M = ml[((size_t)unit * G + h) * 2 + 0];
        const float L = ml[((size_t)unit * G + h) * 2 + 1];
        w += __builtin_amdgcn_exp2f(lg[((size_t)unit * G + h) * lg_stride + t] - M) / L;
    }
    mass[(size_t)unit * mass_stride + t] += w;
}

// Largest chunk whose blocks still fill half of the resident block slots
// (blocks per CU from the kernels' register and LDS use: 4 for g = 1, 3
// for g = 4, 2 for g = 2 and 8), never more than kMaxSplit - 1 packed
// splits per unit.  A 4-wave block's wave share is a power of two between
// max(kMinWaveChunk, Gk) and kMaxWaveChunk tokens, so it holds whole key
// groups and whole 32-token value steps; a 12-wave block's is a multiple of
// the key group (and of 16) up to kMaxWaveChunk, its last value step
// possibly partial.
int pick_chunk(int units, int n_packed, int n_res, int Gk, int g, bool mass) {
    const int per_cu = g == 1 ? 4 : g == 4 ? 3 : 2;
    const long want = 256L * per_cu / 2;
    const int minw = std::max(kMinWaveChunk, Gk);
    int ch4 = minw * kWaves;
    for (int w = kMaxWaveChunk; w > minw; w >>= 1) {
        const int ch = w * kWaves;
        const int next = ch / 2;
        if ((long)units * ((n_packed + ch - 1) / ch) >= want ||
            (n_packed + next - 1) / next > kMaxSplit - 1) {
            ch4 = ch;
            break;
        }
    }
    // g = 4: one 12-wave block per CU when such a grid fills the chip in one
    // round.  Three 4-wave blocks per CU all start together, and the
    // instruction arbiter's preference for older waves then makes the third
    // block of each CU finish ~35% after the first, so the call ends with
    // the CUs a third occupied; the waves of one block share one age.  The
    // call's time follows the tokens per CU, and longer wave shares cost less
    // per token, so:
    // - a power-of-two share whose grid fills 240-256 CUs (or 192 while the
    //   4-wave form would need splits of 512 tokens or fewer);
    // - else, when the 4-wave grid would give some CUs a third block, the
    //   finest share (a multiple of the key group and of 16) whose grid fits
    //   one round and fills at least 224 CUs;
    // - else the 4-wave form (at most two blocks per CU).
    // A residual that finds no idle waves in the last split adds a split per
    // unit, so it counts in the grid.
    if (g == 4 && !mass && units <= 256) {
        auto blocks12 = [&](long w) {
            const long ch = kBigWaves * w;
            const long sp = (n_packed + ch - 1) / ch;
            long extra = 0;
            if (n_res > 0) {
                const long used = sp > 0 ? (n_packed - (sp - 1) * ch + w - 1) / w : kBigWaves;
                if (kBigWaves - used < (n_res + 63) / 64) extra = 1;
            }
            return (long)units * (sp + extra);
        };
        for (int w = kMaxWaveChunk; w >= minw; w >>= 1) {
            const long big = blocks12(w);
            if (big <= 256 && (big >= 240 || (big >= 192 && ch4 <= 512)))
                return kBigWaves * w;
        }
        const long b4 = (long)units * ((n_packed + ch4 - 1) / ch4);
        if (b4 > 512) {
            const int step = std::max(16, Gk);
            const long per_unit = 256 / units;        // blocks per unit, one round
            long w = (n_packed + kBigWaves * per_unit - 1) / (kBigWaves * per_unit);
            w = std::max<long>((w + step - 1) / step * step, minw);
            for (; w <= kMaxWaveChunk; w += step) {
                const long big = blocks12(w);
                if (big <= 256) {
                    if (big >= 224) return (int)(kBigWaves * w);
                    break;
                }
            }
        }
    }
    return ch4;
}

// One launch of the decode kernel for the split plan in `a` (grid: units x
// a.nsplit splits, written at a.split_off of a.nsplit_total).
template <int D, int G>
void decode_kernel_launch(const DecArgs &a, int units, bool mass, hipStream_t stream) {
    const dim3 grid(units, a.nsplit);
    if (a.c.kp != 1 || a.c.vp != 1) {
        // a mixed-precision segment: 16-channel value groups, 4-wave blocks
        if (a.c.kp == 2 && a.c.vp == 2)
            decode_kernel<D, G, true, false, false, kWaves, 2, 2><<<grid, kThreads, 0, stream>>>(a);
        else if (a.c.kp == 4 && a.c.vp == 2)
            decode_kernel<D, G, true, false, false, kWaves, 4, 2><<<grid, kThreads, 0, stream>>>(a);
        else
            decode_kernel<D, G, true, false, false, kWaves, 2, 1><<<grid, kThreads, 0, stream>>>(a);
        return;
    }
    // one key batch per wave (64-token wave shares): the early-load form,
    // for g <= 2 (at g = 4 its registers would spill)
    const bool one = G <= 2 && a.chunk == kMinWaveChunk * kWaves;
    if constexpr (G == 4) {
        if (a.waves == kBigWaves) {
            if (a.c.Gv == 16)
                decode_kernel<D, G, true, false, false, kBigWaves><<<grid, kBigWaves * 64, 0, stream>>>(a);
            else
                decode_kernel<D, G, false, false, false, kBigWaves><<<grid, kBigWaves * 64, 0, stream>>>(a);
            return;
        }
    }
    if (mass) {
        if (a.c.Gv == 16) {
            if (one) decode_kernel<D, G, true, G <= 2, true><<<grid, kThreads, 0, stream>>>(a);
            else decode_kernel<D, G, true, false, true><<<grid, kThreads, 0, stream>>>(a);
        } else {
            if (one) decode_kernel<D, G, false, G <= 2, true><<<grid, kThreads, 0, stream>>>(a);
            else decode_kernel<D, G, false, false, true><<<grid, kThreads, 0, stream>>>(a);
        }
    } else if (a.c.Gv == 16) {
        if (one) decode_kernel<D, G, true, G <= 2, false><<<grid, kThreads, 0, stream>>>(a);
        else decode_kernel<D, G, true, false, false><<<grid, kThreads, 0, stream>>>(a);
    } else {
        if (one) decode_kernel<D, G, false, G <= 2, false><<<grid, kThreads, 0, stream>>>(a);
        else decode_kernel<D, G, false, false, false><<<grid, kThreads, 0, stream>>>(a);
    }
}

template <int D, int G>
hipError_t launch_decode_dg(const DecArgs &a, int units, float *ml_out,
                            const MassOut *mo, hipStream_t stream) {
    decode_kernel_launch<D, G>(a, units, mo != nullptr, stream);
    decode_combine_kernel<D, G><<<dim3(units, G), kThreads, 0, stream>>>(
        a.part_ml, a.part_o, a.nsplit_total, a.o, ml_out);
    if (mo) {
        const int n_tok = a.n_packed + a.n_res;
        decode_mass_kernel<G><<<dim3(units, (n_tok + kThreads - 1) / kThreads), kThreads, 0,
                                stream>>>(a.lg, a.lg_stride, ml_out, n_tok, mo->mass,
                                          mo->stride);
    }
    return hipGetLastError();
}

// Several packed segments (mixed precision) plus the residual: one decode
// launch per segment into consecutive split ranges, then one combine.
template <int D, int G>
hipError_t launch_decode_segs_dg(const DecArgs *as, int n_seg, int units,
                                 hipStream_t stream) {
    for (int s = 0; s < n_seg; ++s)
        if (as[s].nsplit > 0) decode_kernel_launch<D, G>(as[s], units, false, stream);
    decode_combine_kernel<D, G><<<dim3(units, G), kThreads, 0, stream>>>(
        as[0].part_ml, as[0].part_o, as[0].nsplit_total, as[0].o, nullptr);
    return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecArgs &a, int units, int g, float *ml_out,
                           const MassOut *mo, hipStream_t stream) {
    switch (g) {
    case 1: return launch_decode_dg<D, 1>(a, units, ml_out, mo, stream);
    case 2: return launch_decode_dg<D, 2>(a, units, ml_out, mo, stream);
    case 4: return launch_decode_dg<D, 4>(a, units, ml_out, mo, stream);
    case 8: return launch_decode_dg<D, 8>(a, units, ml_out, mo, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int D>
hipError_t launch_decode_segs_d(const DecArgs *as, int n_seg, int units, int g,
                                hipStream_t stream) {
    switch (g) {
    case 1: return launch_decode_segs_dg<D, 1>(as, n_seg, units, stream);
    case 2: return launch_decode_segs_dg<D, 2>(as, n_seg, units, stream);
    case 4: return launch_decode_segs_dg<D, 4>(as, n_seg, units, stream);
    case 8: return launch_decode_segs_dg<D, 8>(as, n_seg, units, stream);
    default: return hipErrorInvalidValue;
    }
}

size_t part_bytes(int units, int g, int D, int nsplit) {
    return (size_t)units * nsplit * g * (D + 2) * sizeof(float);
}

}  // namespace

size_t decode_ws_bytes(int units, int g, int D, int capacity) {
    const int min_chunk = kMinWaveChunk * kWaves;
    const int nsplit = std::min((capacity + min_chunk - 1) / min_chunk + 1, kMaxSplit);
    return part_bytes(units, g, D, nsplit);
}

// Mass-audit workspace: the decode partials, then the logits
// [units][g][lg_stride] and the final (M, L) [units][g][2], each region
// 256-byte aligned.
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static int lg_stride_of(int capacity, int nr) { return (capacity + nr + 3) & ~3; }

size_t decode_mass_ws_bytes(int units, int g, int D, int capacity, int nr) {
    return align256(decode_ws_bytes(units, g, D, capacity)) +
           align256((size_t)units * g * lg_stride_of(capacity, nr) * sizeof(float)) +
           (size_t)units * g * 2 * sizeof(float);
}

// ------------------------------------------------ allocation-free variant
// A file-scope device array holds the split partials of
// minikv_decode_attn_noalloc, for callers that cannot allocate.  Each GPU
// holds its own copy until the process ends; in host code `scratch` is only a
// stand-in for the symbol, so its device address is looked up once per device
// (with that device current) and only that address is ever handed to a
// kernel.  Every call on a GPU shares the array: calls that overlap on one
// GPU race.  Nothing in it needs clearing: every split writes its partial
// before the combine reads it.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

static std::mutex g_scratch_mu;
static void *g_scratch_ptr[64];

hipError_t decode_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

int decode_max_capacity(int g) {
    (void)g;
    return (kMaxSplit - 1) * kMaxWaveChunk * kWaves;
}

// The split plan of one call: chunk size, waves per block, packed splits,
// and where the residual runs.
struct Plan {
    int chunk, waves, n_chunks, nsplit, res_split, res_wave0;
};

// no_big: keep the 4-wave form (the mass audit and the 4- and 8-bit
// segments have no 12-wave form).
static Plan make_plan(int units, int g, int n_packed, int n_res, int Gk, bool no_big) {
    Plan p;
    p.chunk = pick_chunk(units, n_packed, n_res, Gk, g, no_big);
    p.waves = p.chunk % kBigWaves == 0 ? kBigWaves : kWaves;   // W = 4 chunks are 2^k
    p.n_chunks = (n_packed + p.chunk - 1) / p.chunk;
    p.nsplit = p.n_chunks;
    p.res_split = -1;
    p.res_wave0 = 0;
    if (n_res > 0) {
        // waves of 64 residual tokens at most; in the last packed split's
        // idle waves when there are enough of them
        const int W = p.waves;
        const int wchunk = p.chunk / W;
        const int need = (n_res + 63) / 64;
        const int used = p.n_chunks > 0
            ? (n_packed - (p.n_chunks - 1) * p.chunk + wchunk - 1) / wchunk : W;
        if (W - used >= need) {
            p.res_split = p.n_chunks - 1;
            p.res_wave0 = W - need;
        } else {
            p.res_split = p.n_chunks;
            p.nsplit = p.n_chunks + 1;
        }
    }
    return p;
}

size_t decode_plan_ws_bytes(int units, int g, int D, int n_packed, int n_res, int Gk,
                            bool mass) {
    const Plan p = make_plan(units, g, n_packed, n_res, Gk, mass);
    if (p.nsplit > kMaxSplit) return 0;
    return part_bytes(units, g, D, p.nsplit);
}

hipError_t launch_decode(const uint16_t *q, uint16_t *o, int units, int g,
                         int n_packed, int n_res, const CacheView &c,
                         const uint16_t *k_new, const uint16_t *v_new,
                         void *ws, size_t ws_bytes, hipStream_t stream,
                         const MassOut *mo) {
    DecArgs a;
    a.q = q;
    a.o = o;
    a.c = c;
    a.n_packed = n_packed;
    a.n_res = n_res;
    const Plan p = make_plan(units, g, n_packed, n_res, c.Gk, mo != nullptr);
    a.chunk = p.chunk;
    a.waves = p.waves;
    a.n_chunks = p.n_chunks;
    a.nsplit = p.nsplit;
    a.res_split = p.res_split;
    a.res_wave0 = p.res_wave0;
    a.split_off = 0;
    a.nsplit_total = p.nsplit;
    a.qscale = kLog2e / sqrtf((float)c.D);
    a.k_new = k_new;
    a.v_new = v_new;
    a.new_slot = n_res - 1;
    // the entry points check the plan against the workspace before any HIP
    // call; this guard is never taken after that validation
    if (part_bytes(units, g, c.D, a.nsplit) > ws_bytes || a.nsplit > kMaxSplit)
        return hipErrorInvalidValue;
    a.part_ml = static_cast<float *>(ws);
    a.part_o = a.part_ml + (size_t)units * a.nsplit * g * 2;
    a.lg = nullptr;
    a.lg_stride = 0;
    float *ml_out = nullptr;
    if (mo) {
        if (decode_mass_ws_bytes(units, g, c.D, c.cap, c.nr) > ws_bytes)
            return hipErrorInvalidValue;
        char *base = static_cast<char *>(ws) + align256(decode_ws_bytes(units, g, c.D, c.cap));
        a.lg_stride = lg_stride_of(c.cap, c.nr);
        a.lg = reinterpret_cast<float *>(base);
        ml_out = reinterpret_cast<float *>(
            base + align256((size_t)units * g * a.lg_stride * sizeof(float)));
    }
    return c.D == 128 ? launch_decode_d<128>(a, units, g, ml_out, mo, stream)
                      : launch_decode_d<64>(a, units, g, ml_out, mo, stream);
}

// Split plans of a mixed-precision decode: segment s covers n_bound[s]
// packed tokens per unit (its largest per-unit count when it has per-unit
// counts); the residual runs with the last segment.  Returns the total
// number of splits, or -1 if a segment needs more than kMaxSplit.
static int plan_segments(int units, int g, const CacheView *segs, const int *n_bound,
                         int n_seg, int n_res, Plan *plans) {
    int total = 0;
    for (int s = 0; s < n_seg; ++s) {
        const bool planes = segs[s].kp != 1 || segs[s].vp != 1;
        plans[s] = make_plan(units, g, n_bound[s], s == n_seg - 1 ? n_res : 0, segs[s].Gk,
                             planes);
        if (plans[s].nsplit > kMaxSplit) return -1;
        total += plans[s].nsplit;
    }
    return total;
}

size_t decode_segs_ws_bytes(int units, int g, int D, const int *caps, int n_seg) {
    int total = 1;                                // the residual's own split
    for (int s = 0; s < n_seg; ++s)
        total += std::min((caps[s] + kMinWaveChunk * kWaves - 1) / (kMinWaveChunk * kWaves),
                          kMaxSplit);
    return part_bytes(units, g, D, total);
}

size_t decode_segs_plan_ws_bytes(int units, int g, int D, const CacheView *segs,
                                 const int *n_bound, int n_seg, int n_res) {
    Plan plans[kMaxSegments];
    const int total = plan_segments(units, g, segs, n_bound, n_seg, n_res, plans);
    return total < 0 ? 0 : part_bytes(units, g, D, total);
}

hipError_t launch_decode_segs(const uint16_t *q, uint16_t *o, int units, int g,
                              const CacheView *segs, const int *n_bound, int n_seg,
                              int n_res, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (n_seg < 1 || n_seg > kMaxSegments) return hipErrorInvalidValue;
    Plan plans[kMaxSegments];
    const int total = plan_segments(units, g, segs, n_bound, n_seg, n_res, plans);
    const int D = segs[0].D;
    // checked by the entry point before any HIP call
    if (total < 0 || part_bytes(units, g, D, total) > ws_bytes) return hipErrorInvalidValue;
    DecArgs as[kMaxSegments];
    int off = 0;
    for (int s = 0; s < n_seg; ++s) {
        DecArgs &a = as[s];
        const Plan &p = plans[s];
        a.q = q;
        a.o = o;
        a.c = segs[s];
        a.n_packed = n_bound[s];
        a.n_res = s == n_seg - 1 ? n_res : 0;
        a.chunk = p.chunk;
        a.waves = p.waves;
            a.n_chunks = p.n_chunks;
        a.nsplit = p.nsplit;
        a.res_split = p.res_split;
        a.res_wave0 = p.res_wave0;
        a.split_off = off;
        a.nsplit_total = total;
        a.qscale = kLog2e / sqrtf((float)D);
        a.k_new = nullptr;
        a.v_new = nullptr;
        a.new_slot = -1;
        a.part_ml = static_cast<float *>(ws);
        a.part_o = a.part_ml + (size_t)units * total * g * 2;
        a.lg = nullptr;
        a.lg_stride = 0;
        off += p.nsplit;
    }
    return D == 128 ? launch_decode_segs_d<128>(as, n_seg, units, g, stream)
                    : launch_decode_segs_d<64>(as, n_seg, units, g, stream);
}

}  // namespace minikv
