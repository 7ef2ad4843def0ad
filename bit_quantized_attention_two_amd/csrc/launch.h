// Internal host-side launchers of libminikv's kernels.  Arguments are
// validated by abi.cpp before any of these is called; each launcher only
// computes a grid and enqueues kernels on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace minikv {

// Device view of one layer's compressed cache (layout in include/minikv.h).
struct CacheView {
    int32_t *kq;
    uint16_t *ks, *kz;
    int32_t *vq;
    uint16_t *vs, *vz;
    uint16_t *kres, *vres;
    int cap, nr, D, Gk, Gv;
    __host__ __device__ size_t kq_unit() const { return (size_t)cap * (D / 16); }
    __host__ __device__ size_t km_unit() const { return (size_t)(cap / Gk) * D; }
    __host__ __device__ size_t vq_unit() const { return (size_t)(cap / 16) * D; }
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
// region starting at token dst_off (multiple of Gk), then copy the next
// n_tail source rows into residual slots 0..n_tail-1.
hipError_t launch_pack(const PackSrc &src, int units, int n_tok, int n_tail,
                       int dst_off, const CacheView &c, hipStream_t stream);

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

// Prefill, both passes.
hipError_t launch_prefill(const uint16_t *q, const uint16_t *k,
                          const uint16_t *v, uint16_t *o, float *lse,
                          float *col, int B, int Hq, int Hkv, int n, int D,
                          hipStream_t stream);

// Top-k + recent window per unit.
hipError_t launch_select(const float *col, int units, int n, int n_hh,
                         int n_recent, int32_t *sel, hipStream_t stream);

}  // namespace minikv
