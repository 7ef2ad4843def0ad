// Internal host-side launchers of libminikv's kernels.  Arguments are
// validated by abi.cpp before any of these is called; each launcher only
// computes a grid and enqueues kernels on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace minikv {

// Device view of one packed segment of a layer's cache plus the layer's
// fp16 residual (layout in include/minikv.h).  Codes of kbits / vbits bits
// are stored as kp = kbits/2 and vp = vbits/2 planes of 2-bit codes, each
// plane in the INT2 word layout, plane-major within a unit.  n_unit
// (nullable) gives each unit's own count of packed tokens.
struct CacheView {
    int32_t *kq;
    uint16_t *ks, *kz;
    int32_t *vq;
    uint16_t *vs, *vz;
    uint16_t *kres, *vres;
    int cap, nr, D, Gk, Gv;
    int kp = 1, vp = 1;
    const int32_t *n_unit = nullptr;
    __host__ __device__ size_t kplane() const { return (size_t)cap * (D / 16); }
    __host__ __device__ size_t vplane() const { return (size_t)(cap / 16) * D; }
    __host__ __device__ size_t kq_unit() const { return kp * kplane(); }
    __host__ __device__ size_t km_unit() const { return (size_t)(cap / Gk) * D; }
    __host__ __device__ size_t vq_unit() const { return vp * vplane(); }
    __host__ __device__ size_t vm_unit() const { return (size_t)cap * (D / Gv); }
    __host__ __device__ size_t res_unit() const { return (size_t)nr * D; }
};

// Source rows for packing: row p of unit u is src[u*src_unit + r*D ...]
// with r = sel ? sel[u*sel_unit + p] : p.
// A selected index outside [0, n_rows) is clamped into it, so a bad index
// never reads outside the unit's rows.
struct PackSrc {
    const uint16_t *k, *v;
    size_t src_unit;        // elements between units
    const int32_t *sel;     // nullable: identity
    size_t sel_unit;
    int n_rows;             // source rows per unit
};

// Quantise n_tok tokens (multiple of Gk) of every unit into the packed
// region starting at token dst_off (multiple of Gk), at the segment's
// kbits / vbits, then copy the next n_tail source rows into residual slots
// tail_off .. tail_off + n_tail - 1.  With c.n_unit set, unit u packs only
// its own n_unit[u] <= n_tok tokens (n_tail must then be 0).
hipError_t launch_pack(const PackSrc &src, int units, int n_tok, int n_tail,
                       int dst_off, const CacheView &c, hipStream_t stream,
                       int tail_off = 0);

// comp[u][0 .. n - m) = the indices of [0, n) not in sel[u][0 .. m)
// (ascending sel, ascending result).
hipError_t launch_complement(const int32_t *sel, int units, int n, int m,
                             int32_t *comp, hipStream_t stream);

// Copy k_new/v_new [units][D] into residual slot `slot`.
hipError_t launch_append_copy(const uint16_t *k_new, const uint16_t *v_new,
                              int units, int slot, const CacheView &c,
                              hipStream_t stream);

// Decode attention: q, o [units*g][D].  Caches up to decode_max_capacity(g)
// packed tokens per unit.
size_t decode_ws_bytes(int units, int g, int D, int capacity);
// Workspace bytes the call's split plan needs (<= decode_ws_bytes of any
// capacity >= n_packed), or 0 if the plan is not possible (too many splits).
size_t decode_plan_ws_bytes(int units, int g, int D, int n_packed, int n_res,
                            int Gk, bool mass);
size_t decode_mass_ws_bytes(int units, int g, int D, int capacity, int nr);
int decode_max_capacity(int g);
// Size of the device array that holds the split partials of the
// allocation-free decode entry point, and its address on the current device
// (looked up once per device).
constexpr size_t kDecodeScratchBytes = 16u << 20;
hipError_t decode_scratch(void **out);
// Persistence audit output: mass[unit * stride + t] += the attention weight
// of cache token t summed over the unit's g heads.
struct MassOut {
    float *mass;
    int stride;
};
// k_new/v_new [units][D] (nullable): a token appended in the same launch; it
// is residual slot n_res - 1 and is stored there by the kernel.  mo
// (nullable) asks for the mass audit; ws must then hold
// decode_mass_ws_bytes.
hipError_t launch_decode(const uint16_t *q, uint16_t *o, int units, int g,
                         int n_packed, int n_res, const CacheView &c,
                         const uint16_t *k_new, const uint16_t *v_new,
                         void *ws, size_t ws_bytes, hipStream_t stream,
                         const MassOut *mo = nullptr);

// Mixed-precision decode over n_seg <= kMaxSegments packed segments of the
// same layer (each its own bit widths, capacity and, optionally, per-unit
// counts; n_bound[s] = the segment's largest per-unit count) plus the fp16
// residual (n_res tokens, in the last segment's view): one softmax over the
// union.  Keys and values of 4- and 8-bit segments need Gv = 16.
constexpr int kMaxSegments = 3;
size_t decode_segs_ws_bytes(int units, int g, int D, const int *caps, int n_seg);
size_t decode_segs_plan_ws_bytes(int units, int g, int D, const CacheView *segs,
                                 const int *n_bound, int n_seg, int n_res);
hipError_t launch_decode_segs(const uint16_t *q, uint16_t *o, int units, int g,
                              const CacheView *segs, const int *n_bound, int n_seg,
                              int n_res, void *ws, size_t ws_bytes, hipStream_t stream);

// The fused prefill tail: the selection runs in pass 2's epilogue (the
// last workgroup of each unit); counters: [B * Hkv] device words.
struct FusedSelect {
    uint32_t *counters;
    int32_t *sel;
    int n_hh, n_recent;
};

// Prefill, both passes.  significance: col gets DiffKV's per-key
// significance (max over the group's heads of the head's column sum, over
// n - j) instead of the column sum over the group's heads.  fs (nullable):
// also select, fused into pass 2.
hipError_t launch_prefill(const uint16_t *q, const uint16_t *k,
                          const uint16_t *v, uint16_t *o, float *lse,
                          float *col, int B, int Hq, int Hkv, int n, int D,
                          hipStream_t stream, bool significance = false,
                          const FusedSelect *fs = nullptr);

// DiffKV tiers per unit from significance scores (see minikv_tier_diffkv).
hipError_t launch_tier(const float *score, int units, int n, float alpha_hi,
                       float alpha_lo, int Gk, int32_t *idx_hi, int32_t *idx_lo,
                       int32_t *n_hi, int32_t *n_lo, hipStream_t stream);

// Top-k + recent window per unit.
hipError_t launch_select(const float *col, int units, int n, int n_hh,
                         int n_recent, int32_t *sel, hipStream_t stream);

}  // namespace minikv
