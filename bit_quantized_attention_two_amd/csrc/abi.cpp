// C ABI of libminikv: argument validation, sizing helpers and launches.
//
// Every entry point validates its arguments in plain host code first; only
// then does it touch HIP (device check, launches).  Errors are reported as a
// status code plus a thread-local message, with no launch and no change to
// the caller's host-side counters.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/minikv.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int32_t ok() {
    g_err[0] = '\0';
    return MINIKV_OK;
}

bool aligned16(const void *p) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

bool pow2_16_128(int32_t x) {
    return x == 16 || x == 32 || x == 64 || x == 128;
}

// Shape checks shared by every call.
int32_t check_dims(const minikv_dims *d) {
    if (!d) return fail(MINIKV_EINVAL, "dims is NULL");
    if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1)
        return fail(MINIKV_EINVAL, "batch/heads must be >= 1");
    if (d->n_q_heads % d->n_kv_heads)
        return fail(MINIKV_EINVAL, "n_q_heads %% n_kv_heads != 0");
    const int g = d->n_q_heads / d->n_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8)
        return fail(MINIKV_EUNSUPPORTED, "GQA group size %d not in {1,2,4,8}", g);
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(MINIKV_EUNSUPPORTED, "head_dim %d not in {64,128}", d->head_dim);
    if (!pow2_16_128(d->group_k))
        return fail(MINIKV_EUNSUPPORTED, "group_k %d not in {16,32,64,128}", d->group_k);
    if (!pow2_16_128(d->group_v) || d->head_dim % d->group_v)
        return fail(MINIKV_EUNSUPPORTED, "group_v %d must be in {16,32,64,128} and divide head_dim",
                    d->group_v);
    if (d->residual_cap < d->group_k || d->residual_cap > 256 ||
        d->residual_cap % d->group_k)
        return fail(MINIKV_EINVAL, "residual_cap %d must be a multiple of group_k in [group_k, 256]",
                    d->residual_cap);
    const long long bh = (long long)d->batch * d->n_q_heads;
    if (bh > 65535) return fail(MINIKV_EUNSUPPORTED, "batch * n_q_heads too large");
    return MINIKV_OK;
}

int32_t check_len(const minikv_dims *d, int32_t n) {
    if (n < 0) return fail(MINIKV_EINVAL, "n < 0");
    const long long elems = (long long)d->batch * d->n_q_heads * n * d->head_dim;
    if (elems > (1LL << 40)) return fail(MINIKV_EINVAL, "tensor too large");
    if (n > (1 << 24)) return fail(MINIKV_EUNSUPPORTED, "n > 2^24");
    return MINIKV_OK;
}

#define CHECK(expr)                          \
    do {                                     \
        int32_t _s = (expr);                 \
        if (_s != MINIKV_OK) return _s;      \
    } while (0)

#define CHECK_PTR(p, name)                                                     \
    do {                                                                       \
        if (!(p)) return fail(MINIKV_EINVAL, "%s is NULL", name);              \
        if (!aligned16(p)) return fail(MINIKV_EINVAL, "%s not 16-byte aligned", name); \
    } while (0)

int32_t check_cache(const minikv_dims *d, const minikv_layer_cache *c) {
    if (!c) return fail(MINIKV_EINVAL, "cache is NULL");
    CHECK_PTR(c->kq, "cache.kq");
    CHECK_PTR(c->k_scale, "cache.k_scale");
    CHECK_PTR(c->k_zero, "cache.k_zero");
    CHECK_PTR(c->vq, "cache.vq");
    CHECK_PTR(c->v_scale, "cache.v_scale");
    CHECK_PTR(c->v_zero, "cache.v_zero");
    CHECK_PTR(c->k_res, "cache.k_res");
    CHECK_PTR(c->v_res, "cache.v_res");
    if (c->capacity < 0 || c->capacity % d->group_k)
        return fail(MINIKV_EINVAL, "capacity %d must be a non-negative multiple of group_k",
                    c->capacity);
    if (c->n_packed < 0 || c->n_packed > c->capacity || c->n_packed % d->group_k)
        return fail(MINIKV_EINVAL, "n_packed %d inconsistent", c->n_packed);
    if (c->n_res < 0 || c->n_res >= d->residual_cap)
        return fail(MINIKV_EINVAL, "n_res %d inconsistent", c->n_res);
    return MINIKV_OK;
}

minikv::CacheView view_of(const minikv_dims *d, const minikv_layer_cache *c) {
    minikv::CacheView v;
    v.kq = c->kq;
    v.ks = c->k_scale;
    v.kz = c->k_zero;
    v.vq = c->vq;
    v.vs = c->v_scale;
    v.vz = c->v_zero;
    v.kres = c->k_res;
    v.vres = c->v_res;
    v.cap = c->capacity;
    v.nr = d->residual_cap;
    v.D = d->head_dim;
    v.Gk = d->group_k;
    v.Gv = d->group_v;
    return v;
}

// First HIP call of every compute entry point: the current device must be a
// gfx950.  Cached per device id.
std::mutex g_dev_mu;
int g_dev_ok[64];   // 0 unknown, 1 ok, -1 unsupported

int32_t check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(MINIKV_EHIP, "hipGetDevice failed");
    if (dev < 0 || dev >= 64) return fail(MINIKV_EUNSUPPORTED, "device id %d", dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_ok[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(MINIKV_EHIP, "hipGetDeviceProperties failed");
        g_dev_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    if (g_dev_ok[dev] != 1)
        return fail(MINIKV_EUNSUPPORTED, "device %d is not gfx950", dev);
    return MINIKV_OK;
}

int32_t hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess)
        return fail(MINIKV_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int32_t minikv_version(void) { return 100; }   // 0.1.0

const char *minikv_status_str(int32_t s) {
    switch (s) {
    case MINIKV_OK: return "MINIKV_OK";
    case MINIKV_EINVAL: return "MINIKV_EINVAL";
    case MINIKV_EUNSUPPORTED: return "MINIKV_EUNSUPPORTED";
    case MINIKV_ECAPACITY: return "MINIKV_ECAPACITY";
    case MINIKV_EHIP: return "MINIKV_EHIP";
    default: return "MINIKV_UNKNOWN";
    }
}

const char *minikv_last_error(void) { return g_err; }

int32_t minikv_pyramid_budgets(int32_t n, int32_t n_layers, int32_t hh_num,
                               int32_t hh_den, int32_t rw_num, int32_t rw_den,
                               int32_t depth, int32_t pyramid, int32_t *k_out,
                               int32_t *r_out) {
    if (!k_out || !r_out) return fail(MINIKV_EINVAL, "output pointer is NULL");
    if (n < 0 || n_layers < 1 || hh_num < 0 || hh_den <= 0 || rw_num < 0 ||
        rw_den <= 0 || (pyramid && depth < 1))
        return fail(MINIKV_EINVAL, "bad budget arguments");
    const long long r = (long long)n * rw_num / rw_den;
    const long long k = (long long)n * hh_num / hh_den;
    if (r > n) return fail(MINIKV_EINVAL, "recent window exceeds n");
    for (int l = 0; l < n_layers; ++l) {
        long long kl = k;
        if (pyramid && n_layers > 1) {
            const long long kmin = k / depth;
            const long long kmax = 2 * k - kmin;
            kl = kmin + (kmax - kmin) * (n_layers - 1 - l) / (n_layers - 1);
        }
        if (kl > n - r) kl = n - r;
        k_out[l] = (int32_t)kl;
    }
    *r_out = (int32_t)r;
    return ok();
}

int32_t minikv_cache_bytes_closed_form(int32_t n_layers, int32_t n_heads,
                                       int32_t head_dim, int32_t lprompt,
                                       int32_t lgen, int32_t budget_num,
                                       int32_t budget_den, int32_t bits,
                                       int32_t group, uint64_t *minikv_bytes,
                                       uint64_t *full_bytes) {
    if (!minikv_bytes || !full_bytes) return fail(MINIKV_EINVAL, "output pointer is NULL");
    if (n_layers < 1 || n_heads < 1 || head_dim < 1 || lprompt < 0 || lgen < 0 ||
        budget_num < 0 || budget_den <= 0 || bits < 1 || group < 1)
        return fail(MINIKV_EINVAL, "bad cache-size arguments");
    // bytes = 2 (K,V) * L * H * D * tokens * (bits + 32/group) / 8, with
    // tokens = lprompt * budget + lgen; evaluated exactly in integers.
    const unsigned long long elems = 2ull * n_layers * n_heads * head_dim;
    const unsigned long long tok_num =
        (unsigned long long)lprompt * budget_num + (unsigned long long)lgen * budget_den;
    const unsigned long long bits_num = (unsigned long long)bits * group + 32ull;
    const unsigned long long den = (unsigned long long)budget_den * group * 8ull;
    *minikv_bytes = elems * tok_num * bits_num / den;
    *full_bytes = elems * (unsigned long long)(lprompt + lgen) * 2ull;
    return ok();
}

int32_t minikv_cache_layout(const minikv_dims *d, int32_t capacity,
                            size_t out[8]) {
    CHECK(check_dims(d));
    if (!out) return fail(MINIKV_EINVAL, "out is NULL");
    if (capacity < 0 || capacity % d->group_k)
        return fail(MINIKV_EINVAL, "capacity must be a non-negative multiple of group_k");
    const size_t units = (size_t)d->batch * d->n_kv_heads;
    const size_t D = d->head_dim;
    out[0] = units * (capacity / 16) * D * 4;
    out[1] = units * (capacity / d->group_k) * D * 2;
    out[2] = out[1];
    out[3] = units * capacity * (D / 16) * 4;
    out[4] = units * capacity * (D / d->group_v) * 2;
    out[5] = out[4];
    out[6] = units * d->residual_cap * D * 2;
    out[7] = out[6];
    return ok();
}

int32_t minikv_prefill_ws_bytes(const minikv_dims *d, int32_t n,
                                int32_t lse_given, size_t *out) {
    CHECK(check_dims(d));
    CHECK(check_len(d, n));
    if (!out) return fail(MINIKV_EINVAL, "out is NULL");
    const size_t lse_bytes = (size_t)d->batch * d->n_q_heads * n * sizeof(float);
    *out = lse_given ? 0 : ((lse_bytes + 255) / 256) * 256;
    return ok();
}

int32_t minikv_decode_ws_bytes(const minikv_dims *d, int32_t capacity,
                               size_t *out) {
    CHECK(check_dims(d));
    if (!out) return fail(MINIKV_EINVAL, "out is NULL");
    if (capacity < 0) return fail(MINIKV_EINVAL, "capacity < 0");
    *out = minikv::decode_ws_bytes(d->batch * d->n_kv_heads,
                                   d->n_q_heads / d->n_kv_heads, d->head_dim,
                                   capacity);
    return ok();
}

int32_t minikv_decode_mass_ws_bytes(const minikv_dims *d, int32_t capacity,
                                    size_t *out) {
    CHECK(check_dims(d));
    if (!out) return fail(MINIKV_EINVAL, "out is NULL");
    if (capacity < 0) return fail(MINIKV_EINVAL, "capacity < 0");
    *out = minikv::decode_mass_ws_bytes(d->batch * d->n_kv_heads,
                                        d->n_q_heads / d->n_kv_heads, d->head_dim,
                                        capacity, d->residual_cap);
    return ok();
}

int32_t minikv_prefill_attn(const minikv_dims *d, int32_t n, const void *q,
                            const void *k, const void *v, void *o, float *lse,
                            float *col, void *stream) {
    CHECK(check_dims(d));
    CHECK(check_len(d, n));
    if (n == 0) return ok();
    CHECK_PTR(q, "q");
    CHECK_PTR(k, "k");
    CHECK_PTR(v, "v");
    CHECK_PTR(o, "o");
    CHECK_PTR(lse, "lse");
    CHECK_PTR(col, "col");
    CHECK(check_device());
    return hip_status(
        minikv::launch_prefill(static_cast<const uint16_t *>(q),
                               static_cast<const uint16_t *>(k),
                               static_cast<const uint16_t *>(v),
                               static_cast<uint16_t *>(o), lse, col, d->batch,
                               d->n_q_heads, d->n_kv_heads, n, d->head_dim,
                               static_cast<hipStream_t>(stream)),
        "prefill launch");
}

static int32_t check_select_args(const minikv_dims *d, int32_t n, int32_t n_hh,
                                 int32_t n_recent) {
    if (n_recent < 0 || n_recent > n)
        return fail(MINIKV_EINVAL, "need 0 <= n_recent <= n");
    if (n_hh < 0 || n_hh > n - n_recent)
        return fail(MINIKV_EINVAL, "need 0 <= n_hh <= n - n_recent");
    (void)d;
    return MINIKV_OK;
}

int32_t minikv_select(const minikv_dims *d, int32_t n, const float *col,
                      int32_t n_hh, int32_t n_recent, int32_t *sel,
                      void *stream) {
    CHECK(check_dims(d));
    CHECK(check_len(d, n));
    CHECK(check_select_args(d, n, n_hh, n_recent));
    if (n_hh + n_recent == 0) return ok();
    CHECK_PTR(col, "col");
    CHECK_PTR(sel, "sel");
    CHECK(check_device());
    return hip_status(minikv::launch_select(col, d->batch * d->n_kv_heads, n, n_hh,
                                            n_recent, sel,
                                            static_cast<hipStream_t>(stream)),
                      "select launch");
}

int32_t minikv_prefill_select(const minikv_dims *d, int32_t n, const void *q,
                              const void *k, const void *v, void *o, float *col,
                              float *lse, int32_t n_hh, int32_t n_recent,
                              int32_t *sel, void *ws, size_t ws_bytes,
                              void *stream) {
    CHECK(check_dims(d));
    CHECK(check_len(d, n));
    CHECK(check_select_args(d, n, n_hh, n_recent));
    if (n == 0) return ok();
    CHECK_PTR(q, "q");
    CHECK_PTR(k, "k");
    CHECK_PTR(v, "v");
    CHECK_PTR(o, "o");
    CHECK_PTR(col, "col");
    if (n_hh + n_recent > 0) CHECK_PTR(sel, "sel");
    float *lse_buf = lse;
    if (lse) {
        CHECK_PTR(lse, "lse");
    } else {
        size_t need = 0;
        minikv_prefill_ws_bytes(d, n, 0, &need);
        CHECK_PTR(ws, "ws");
        if (ws_bytes < need)
            return fail(MINIKV_EINVAL, "workspace too small: %zu < %zu", ws_bytes, need);
        lse_buf = static_cast<float *>(ws);
    }
    CHECK(check_device());
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = minikv::launch_prefill(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), static_cast<uint16_t *>(o), lse_buf, col,
        d->batch, d->n_q_heads, d->n_kv_heads, n, d->head_dim, s);
    if (e != hipSuccess) return hip_status(e, "prefill launch");
    if (n_hh + n_recent > 0)
        e = minikv::launch_select(col, d->batch * d->n_kv_heads, n, n_hh, n_recent,
                                  sel, s);
    return hip_status(e, "select launch");
}

int32_t minikv_pack(const minikv_dims *d, int32_t n, const void *k,
                    const void *v, const int32_t *sel, int32_t n_sel,
                    minikv_layer_cache *c, void *stream) {
    CHECK(check_dims(d));
    CHECK(check_len(d, n));
    CHECK(check_cache(d, c));
    if (n_sel < 0 || n_sel > n) return fail(MINIKV_EINVAL, "need 0 <= n_sel <= n");
    const int32_t n_tok = (n_sel / d->group_k) * d->group_k;
    const int32_t n_tail = n_sel - n_tok;
    if (n_tok > c->capacity)
        return fail(MINIKV_ECAPACITY, "%d packed tokens exceed capacity %d", n_tok,
                    c->capacity);
    if (n_tail >= d->residual_cap)
        return fail(MINIKV_ECAPACITY, "residual tail %d >= residual_cap", n_tail);
    if (n_sel > 0) {
        CHECK_PTR(k, "k");
        CHECK_PTR(v, "v");
        CHECK_PTR(sel, "sel");
        CHECK(check_device());
        minikv::PackSrc src;
        src.k = static_cast<const uint16_t *>(k);
        src.v = static_cast<const uint16_t *>(v);
        src.src_unit = (size_t)n * d->head_dim;
        src.sel = sel;
        src.sel_unit = (size_t)n_sel;
        src.n_rows = n;
        hipError_t e = minikv::launch_pack(src, d->batch * d->n_kv_heads, n_tok,
                                           n_tail, 0, view_of(d, c),
                                           static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_status(e, "pack launch");
    }
    c->n_packed = n_tok;
    c->n_res = n_tail;
    return ok();
}

int32_t minikv_append(const minikv_dims *d, minikv_layer_cache *c,
                      const void *k_new, const void *v_new, void *stream) {
    CHECK(check_dims(d));
    CHECK(check_cache(d, c));
    CHECK_PTR(k_new, "k_new");
    CHECK_PTR(v_new, "v_new");
    const bool flush = c->n_res + 1 == d->residual_cap;
    if (flush && c->n_packed + d->residual_cap > c->capacity)
        return fail(MINIKV_ECAPACITY, "flush of %d tokens exceeds capacity %d",
                    d->residual_cap, c->capacity);
    CHECK(check_device());
    const minikv::CacheView cv = view_of(d, c);
    const int units = d->batch * d->n_kv_heads;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = minikv::launch_append_copy(static_cast<const uint16_t *>(k_new),
                                              static_cast<const uint16_t *>(v_new),
                                              units, c->n_res, cv, s);
    if (e != hipSuccess) return hip_status(e, "append launch");
    if (flush) {
        minikv::PackSrc src;
        src.k = c->k_res;
        src.v = c->v_res;
        src.src_unit = cv.res_unit();
        src.sel = nullptr;
        src.sel_unit = 0;
        src.n_rows = d->residual_cap;
        e = minikv::launch_pack(src, units, d->residual_cap, 0, c->n_packed, cv, s);
        if (e != hipSuccess) return hip_status(e, "flush launch");
        c->n_packed += d->residual_cap;
        c->n_res = 0;
    } else {
        c->n_res += 1;
    }
    return ok();
}

static int32_t check_decode(const minikv_dims *d, const minikv_layer_cache *c,
                            const void *q, const void *o, const void *ws,
                            size_t ws_bytes) {
    CHECK_PTR(q, "q");
    CHECK_PTR(o, "o");
    CHECK_PTR(ws, "ws");
    const int units = d->batch * d->n_kv_heads;
    const int g = d->n_q_heads / d->n_kv_heads;
    if (c->capacity > minikv::decode_max_capacity(g))
        return fail(MINIKV_EUNSUPPORTED, "capacity %d above the decode limit %d",
                    c->capacity, minikv::decode_max_capacity(g));
    const size_t need = minikv::decode_ws_bytes(units, g, d->head_dim, c->capacity);
    if (ws_bytes < need)
        return fail(MINIKV_EINVAL, "workspace too small: %zu < %zu", ws_bytes, need);
    return MINIKV_OK;
}

// The launch's own split plan, checked on the host before any HIP call (it
// always fits a workspace sized for the capacity; checked all the same).
static int32_t check_decode_plan(const minikv_dims *d, int32_t n_packed,
                                 int32_t n_res, size_t ws_bytes, bool mass) {
    const int units = d->batch * d->n_kv_heads;
    const int g = d->n_q_heads / d->n_kv_heads;
    const size_t need = minikv::decode_plan_ws_bytes(units, g, d->head_dim, n_packed,
                                                     n_res, d->group_k, mass);
    if (need == 0 || need > ws_bytes)
        return fail(MINIKV_EINVAL, "decode split plan does not fit the workspace (%zu > %zu)",
                    need, ws_bytes);
    return MINIKV_OK;
}

int32_t minikv_decode_attn(const minikv_dims *d, const minikv_layer_cache *c,
                           const void *q, void *o, void *ws, size_t ws_bytes,
                           void *stream) {
    CHECK(check_dims(d));
    CHECK(check_cache(d, c));
    CHECK(check_decode(d, c, q, o, ws, ws_bytes));
    if (c->n_packed + c->n_res == 0) return fail(MINIKV_EINVAL, "cache holds no token");
    CHECK(check_decode_plan(d, c->n_packed, c->n_res, ws_bytes, false));
    CHECK(check_device());
    const int units = d->batch * d->n_kv_heads;
    const int g = d->n_q_heads / d->n_kv_heads;
    return hip_status(minikv::launch_decode(static_cast<const uint16_t *>(q),
                                            static_cast<uint16_t *>(o), units, g,
                                            c->n_packed, c->n_res, view_of(d, c),
                                            nullptr, nullptr, ws, ws_bytes,
                                            static_cast<hipStream_t>(stream)),
                      "decode launch");
}

int32_t minikv_decode_attn_noalloc(const minikv_dims *d, const minikv_layer_cache *c,
                                   const void *q, void *o, void *stream) {
    CHECK(check_dims(d));
    CHECK(check_cache(d, c));
    CHECK_PTR(q, "q");
    CHECK_PTR(o, "o");
    const int g = d->n_q_heads / d->n_kv_heads;
    if (c->capacity > minikv::decode_max_capacity(g))
        return fail(MINIKV_EUNSUPPORTED, "capacity %d above the decode limit %d",
                    c->capacity, minikv::decode_max_capacity(g));
    if (c->n_packed + c->n_res == 0) return fail(MINIKV_EINVAL, "cache holds no token");
    const int units = d->batch * d->n_kv_heads;
    const size_t need = minikv::decode_plan_ws_bytes(units, g, d->head_dim, c->n_packed,
                                                     c->n_res, d->group_k, false);
    if (need == 0 || need > minikv::kDecodeScratchBytes)
        return fail(MINIKV_ECAPACITY,
                    "split partials of this call (%zu bytes) exceed the %zu-byte "
                    "scratch array; use minikv_decode_attn with a workspace",
                    need, minikv::kDecodeScratchBytes);
    CHECK(check_device());
    void *ws = nullptr;
    CHECK(hip_status(minikv::decode_scratch(&ws), "scratch address"));
    return hip_status(minikv::launch_decode(static_cast<const uint16_t *>(q),
                                            static_cast<uint16_t *>(o), units, g,
                                            c->n_packed, c->n_res, view_of(d, c),
                                            nullptr, nullptr, ws,
                                            minikv::kDecodeScratchBytes,
                                            static_cast<hipStream_t>(stream)),
                      "decode launch");
}

int32_t minikv_append_decode(const minikv_dims *d, minikv_layer_cache *c,
                             const void *k_new, const void *v_new, const void *q,
                             void *o, void *ws, size_t ws_bytes, void *stream) {
    CHECK(check_dims(d));
    CHECK(check_cache(d, c));
    CHECK_PTR(k_new, "k_new");
    CHECK_PTR(v_new, "v_new");
    CHECK(check_decode(d, c, q, o, ws, ws_bytes));
    const bool flush = c->n_res + 1 == d->residual_cap;
    if (flush) {
        // the residual is packed first: the separate calls, in order
        if (c->n_packed + d->residual_cap > c->capacity)
            return fail(MINIKV_ECAPACITY, "flush of %d tokens exceeds capacity %d",
                        d->residual_cap, c->capacity);
        CHECK(check_decode_plan(d, c->n_packed + d->residual_cap, 0, ws_bytes, false));
        CHECK(minikv_append(d, c, k_new, v_new, stream));
        return minikv_decode_attn(d, c, q, o, ws, ws_bytes, stream);
    }
    CHECK(check_decode_plan(d, c->n_packed, c->n_res + 1, ws_bytes, false));
    CHECK(check_device());
    const int units = d->batch * d->n_kv_heads;
    const int g = d->n_q_heads / d->n_kv_heads;
    const int32_t st = hip_status(
        minikv::launch_decode(static_cast<const uint16_t *>(q), static_cast<uint16_t *>(o),
                              units, g, c->n_packed, c->n_res + 1, view_of(d, c),
                              static_cast<const uint16_t *>(k_new),
                              static_cast<const uint16_t *>(v_new), ws, ws_bytes,
                              static_cast<hipStream_t>(stream)),
        "append+decode launch");
    if (st == MINIKV_OK) c->n_res += 1;
    return st;
}

int32_t minikv_decode_attn_mass(const minikv_dims *d, const minikv_layer_cache *c,
                                const void *q, void *o, float *mass,
                                int32_t mass_stride, void *ws, size_t ws_bytes,
                                void *stream) {
    CHECK(check_dims(d));
    CHECK(check_cache(d, c));
    CHECK(check_decode(d, c, q, o, ws, ws_bytes));
    CHECK_PTR(mass, "mass");
    if (c->n_packed + c->n_res == 0) return fail(MINIKV_EINVAL, "cache holds no token");
    if (mass_stride < c->n_packed + c->n_res)
        return fail(MINIKV_EINVAL, "mass_stride %d < %d cached tokens", mass_stride,
                    c->n_packed + c->n_res);
    const int units = d->batch * d->n_kv_heads;
    const int g = d->n_q_heads / d->n_kv_heads;
    const size_t need = minikv::decode_mass_ws_bytes(units, g, d->head_dim, c->capacity,
                                                     d->residual_cap);
    if (ws_bytes < need)
        return fail(MINIKV_EINVAL, "workspace too small: %zu < %zu", ws_bytes, need);
    CHECK(check_decode_plan(d, c->n_packed, c->n_res, ws_bytes, true));
    CHECK(check_device());
    const minikv::MassOut mo{mass, mass_stride};
    return hip_status(minikv::launch_decode(static_cast<const uint16_t *>(q),
                                            static_cast<uint16_t *>(o), units, g,
                                            c->n_packed, c->n_res, view_of(d, c),
                                            nullptr, nullptr, ws, ws_bytes,
                                            static_cast<hipStream_t>(stream), &mo),
                      "decode+mass launch");
}

}  // extern "C"

// ================================================= mixed-precision caches

namespace {

bool bits_pair_ok(int kb, int vb) {
    return (kb == 2 && vb == 2) || (kb == 4 && vb == 4) || (kb == 4 && vb == 2) ||
           (kb == 8 && vb == 4);
}

int32_t check_segment(const minikv_dims *d, const minikv_segment *s, int i) {
    if (!bits_pair_ok(s->key_bits, s->value_bits))
        return fail(MINIKV_EUNSUPPORTED, "segment %d: key/value bits %d/%d not supported", i,
                    s->key_bits, s->value_bits);
    CHECK_PTR(s->kq, "segment.kq");
    CHECK_PTR(s->k_scale, "segment.k_scale");
    CHECK_PTR(s->k_zero, "segment.k_zero");
    CHECK_PTR(s->vq, "segment.vq");
    CHECK_PTR(s->v_scale, "segment.v_scale");
    CHECK_PTR(s->v_zero, "segment.v_zero");
    if (s->capacity < 0 || s->capacity % d->group_k || s->capacity % 16)
        return fail(MINIKV_EINVAL, "segment %d: capacity %d must be a non-negative multiple of "
                    "group_k and 16", i, s->capacity);
    if (s->n_packed < 0 || s->n_packed > s->capacity || s->n_packed % d->group_k)
        return fail(MINIKV_EINVAL, "segment %d: n_packed %d inconsistent", i, s->n_packed);
    if (s->n_unit && (reinterpret_cast<uintptr_t>(s->n_unit) & 3u))
        return fail(MINIKV_EINVAL, "segment %d: n_unit not 4-byte aligned", i);
    return MINIKV_OK;
}

int32_t check_mixed(const minikv_dims *d, const minikv_mixed_cache *c) {
    if (!c) return fail(MINIKV_EINVAL, "cache is NULL");
    if (d->group_v != 16)
        return fail(MINIKV_EUNSUPPORTED, "mixed-precision caches need group_v 16");
    if (c->n_seg < 1 || c->n_seg > MINIKV_MAX_SEGMENTS)
        return fail(MINIKV_EINVAL, "n_seg %d not in [1, %d]", c->n_seg, MINIKV_MAX_SEGMENTS);
    for (int i = 0; i < c->n_seg; ++i) CHECK(check_segment(d, &c->seg[i], i));
    if (c->flush_seg < 0 || c->flush_seg >= c->n_seg || c->seg[c->flush_seg].n_unit)
        return fail(MINIKV_EINVAL, "flush_seg %d must name a segment without n_unit",
                    c->flush_seg);
    CHECK_PTR(c->k_res, "cache.k_res");
    CHECK_PTR(c->v_res, "cache.v_res");
    if (c->n_res < 0 || c->n_res >= d->residual_cap)
        return fail(MINIKV_EINVAL, "n_res %d inconsistent", c->n_res);
    return MINIKV_OK;
}

minikv::CacheView seg_view(const minikv_dims *d, const minikv_mixed_cache *c, int i) {
    const minikv_segment &s = c->seg[i];
    minikv::CacheView v;
    v.kq = s.kq;
    v.ks = s.k_scale;
    v.kz = s.k_zero;
    v.vq = s.vq;
    v.vs = s.v_scale;
    v.vz = s.v_zero;
    v.kres = c->k_res;
    v.vres = c->v_res;
    v.cap = s.capacity;
    v.nr = d->residual_cap;
    v.D = d->head_dim;
    v.Gk = d->group_k;
    v.Gv = d->group_v;
    v.kp = s.key_bits / 2;
    v.vp = s.value_bits / 2;
    v.n_unit = s.n_unit;
    return v;
}

}  // namespace

extern "C" {

int32_t minikv_segment_layout(const minikv_dims *d, int32_t key_bits, int32_t value_bits,
                              int32_t capacity, size_t out[6]) {
    CHECK(check_dims(d));
    if (!out) return fail(MINIKV_EINVAL, "out is NULL");
    if (!bits_pair_ok(key_bits, value_bits))
        return fail(MINIKV_EINVAL, "key/value bits %d/%d not supported", key_bits, value_bits);
    if (capacity < 0 || capacity % d->group_k || capacity % 16)
        return fail(MINIKV_EINVAL, "capacity must be a non-negative multiple of group_k and 16");
    const size_t units = (size_t)d->batch * d->n_kv_heads;
    const size_t D = d->head_dim;
    out[0] = units * (key_bits / 2) * capacity * (D / 16) * 4;
    out[1] = units * (capacity / d->group_k) * D * 2;
    out[2] = out[1];
    out[3] = units * (value_bits / 2) * (capacity / 16) * D * 4;
    out[4] = units * capacity * (D / d->group_v) * 2;
    out[5] = out[4];
    return ok();
}

int32_t minikv_mikv_ws_bytes(const minikv_dims *d, int32_t n, int32_t n_sel, size_t *out) {
    CHECK(check_dims(d));
    CHECK(check_len(d, n));
    if (!out) return fail(MINIKV_EINVAL, "out is NULL");
    if (n_sel < 0 || n_sel > n) return fail(MINIKV_EINVAL, "need 0 <= n_sel <= n");
    const size_t b = (size_t)d->batch * d->n_kv_heads * (n - n_sel) * sizeof(int32_t);
    *out = (b + 255) / 256 * 256;
    return ok();
}

int32_t minikv_pack_mikv(const minikv_dims *d, int32_t n, const void *k, const void *v,
                         const int32_t *sel, int32_t n_sel, minikv_mixed_cache *c,
                         void *ws, size_t ws_bytes, void *stream) {
    CHECK(check_dims(d));
    CHECK(check_len(d, n));
    CHECK(check_mixed(d, c));
    if (c->n_seg != 2 || c->flush_seg != 0 || c->seg[0].n_unit || c->seg[1].n_unit)
        return fail(MINIKV_EINVAL, "MiKV pack needs two segments without n_unit, flush_seg 0");
    if (n_sel < 0 || n_sel > n) return fail(MINIKV_EINVAL, "need 0 <= n_sel <= n");
    const int Gk = d->group_k;
    const int hi_tok = n_sel / Gk * Gk, hi_tail = n_sel - hi_tok;
    const int lo_tok = (n - n_sel) / Gk * Gk, lo_tail = (n - n_sel) - lo_tok;
    if (hi_tok > c->seg[0].capacity || lo_tok > c->seg[1].capacity)
        return fail(MINIKV_ECAPACITY, "segment capacity %d / %d < %d / %d packed tokens",
                    c->seg[0].capacity, c->seg[1].capacity, hi_tok, lo_tok);
    if (hi_tail + lo_tail >= d->residual_cap)
        return fail(MINIKV_ECAPACITY, "residual tails %d >= residual_cap", hi_tail + lo_tail);
    size_t need = 0;
    minikv_mikv_ws_bytes(d, n, n_sel, &need);
    if (n > 0) {
        CHECK_PTR(k, "k");
        CHECK_PTR(v, "v");
        if (n_sel > 0) CHECK_PTR(sel, "sel");
        if (n_sel < n) {
            CHECK_PTR(ws, "ws");
            if (ws_bytes < need)
                return fail(MINIKV_EINVAL, "workspace too small: %zu < %zu", ws_bytes, need);
        }
        CHECK(check_device());
        hipStream_t s = static_cast<hipStream_t>(stream);
        const int units = d->batch * d->n_kv_heads;
        minikv::PackSrc src;
        src.k = static_cast<const uint16_t *>(k);
        src.v = static_cast<const uint16_t *>(v);
        src.src_unit = (size_t)n * d->head_dim;
        src.n_rows = n;
        hipError_t e = hipSuccess;
        if (n_sel > 0) {
            src.sel = sel;
            src.sel_unit = (size_t)n_sel;
            e = minikv::launch_pack(src, units, hi_tok, hi_tail, 0, seg_view(d, c, 0), s, 0);
            if (e != hipSuccess) return hip_status(e, "pack launch");
        }
        if (n_sel < n) {
            int32_t *comp = static_cast<int32_t *>(ws);
            e = minikv::launch_complement(sel, units, n, n_sel, comp, s);
            if (e != hipSuccess) return hip_status(e, "complement launch");
            src.sel = comp;
            src.sel_unit = (size_t)(n - n_sel);
            e = minikv::launch_pack(src, units, lo_tok, lo_tail, 0, seg_view(d, c, 1), s,
                                    hi_tail);
            if (e != hipSuccess) return hip_status(e, "pack launch");
        }
    }
    c->seg[0].n_packed = hi_tok;
    c->seg[1].n_packed = lo_tok;
    c->n_res = hi_tail + lo_tail;
    return ok();
}

int32_t minikv_append_mixed(const minikv_dims *d, minikv_mixed_cache *c, const void *k_new,
                            const void *v_new, void *stream) {
    CHECK(check_dims(d));
    CHECK(check_mixed(d, c));
    CHECK_PTR(k_new, "k_new");
    CHECK_PTR(v_new, "v_new");
    minikv_segment &fs = c->seg[c->flush_seg];
    const bool flush = c->n_res + 1 == d->residual_cap;
    if (flush && fs.n_packed + d->residual_cap > fs.capacity)
        return fail(MINIKV_ECAPACITY, "flush of %d tokens exceeds capacity %d",
                    d->residual_cap, fs.capacity);
    CHECK(check_device());
    const minikv::CacheView cv = seg_view(d, c, c->flush_seg);
    const int units = d->batch * d->n_kv_heads;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = minikv::launch_append_copy(static_cast<const uint16_t *>(k_new),
                                              static_cast<const uint16_t *>(v_new), units,
                                              c->n_res, cv, s);
    if (e != hipSuccess) return hip_status(e, "append launch");
    if (flush) {
        minikv::PackSrc src;
        src.k = c->k_res;
        src.v = c->v_res;
        src.src_unit = cv.res_unit();
        src.sel = nullptr;
        src.sel_unit = 0;
        src.n_rows = d->residual_cap;
        e = minikv::launch_pack(src, units, d->residual_cap, 0, fs.n_packed, cv, s);
        if (e != hipSuccess) return hip_status(e, "flush launch");
        fs.n_packed += d->residual_cap;
        c->n_res = 0;
    } else {
        c->n_res += 1;
    }
    return ok();
}

int32_t minikv_decode_mixed_ws_bytes(const minikv_dims *d, const minikv_mixed_cache *c,
                                     size_t *out) {
    CHECK(check_dims(d));
    CHECK(check_mixed(d, c));
    if (!out) return fail(MINIKV_EINVAL, "out is NULL");
    int caps[MINIKV_MAX_SEGMENTS];
    for (int i = 0; i < c->n_seg; ++i) caps[i] = c->seg[i].capacity;
    *out = minikv::decode_segs_ws_bytes(d->batch * d->n_kv_heads, d->n_q_heads / d->n_kv_heads,
                                        d->head_dim, caps, c->n_seg);
    return ok();
}

int32_t minikv_decode_mixed(const minikv_dims *d, const minikv_mixed_cache *c, const void *q,
                            void *o, void *ws, size_t ws_bytes, void *stream) {
    CHECK(check_dims(d));
    CHECK(check_mixed(d, c));
    CHECK_PTR(q, "q");
    CHECK_PTR(o, "o");
    CHECK_PTR(ws, "ws");
    const int units = d->batch * d->n_kv_heads;
    const int g = d->n_q_heads / d->n_kv_heads;
    int tokens = c->n_res;
    minikv::CacheView views[MINIKV_MAX_SEGMENTS];
    int bound[MINIKV_MAX_SEGMENTS];
    for (int i = 0; i < c->n_seg; ++i) {
        if (c->seg[i].capacity > minikv::decode_max_capacity(g))
            return fail(MINIKV_EUNSUPPORTED, "segment %d capacity above the decode limit", i);
        views[i] = seg_view(d, c, i);
        bound[i] = c->seg[i].n_packed;
        tokens += bound[i];
    }
    if (tokens == 0) return fail(MINIKV_EINVAL, "cache holds no token");
    size_t need = 0;
    minikv_decode_mixed_ws_bytes(d, c, &need);
    const size_t plan = minikv::decode_segs_plan_ws_bytes(units, g, d->head_dim, views, bound,
                                                          c->n_seg, c->n_res);
    if (ws_bytes < need || plan == 0 || plan > ws_bytes)
        return fail(MINIKV_EINVAL, "workspace too small: %zu < %zu", ws_bytes, need);
    CHECK(check_device());
    return hip_status(minikv::launch_decode_segs(static_cast<const uint16_t *>(q),
                                                 static_cast<uint16_t *>(o), units, g, views,
                                                 bound, c->n_seg, c->n_res, ws, ws_bytes,
                                                 static_cast<hipStream_t>(stream)),
                      "mixed decode launch");
}

int32_t minikv_diffkv_ws_bytes(const minikv_dims *d, int32_t n, int32_t lse_given,
                               size_t *out) {
    return minikv_prefill_ws_bytes(d, n, lse_given, out);
}

int32_t minikv_prefill_diffkv(const minikv_dims *d, int32_t n, const void *q, const void *k,
                              const void *v, void *o, float *score, float *lse, void *ws,
                              size_t ws_bytes, void *stream) {
    CHECK(check_dims(d));
    CHECK(check_len(d, n));
    if (n == 0) return ok();
    CHECK_PTR(q, "q");
    CHECK_PTR(k, "k");
    CHECK_PTR(v, "v");
    CHECK_PTR(o, "o");
    CHECK_PTR(score, "score");
    float *lse_buf = lse;
    if (lse) {
        CHECK_PTR(lse, "lse");
    } else {
        size_t need = 0;
        minikv_prefill_ws_bytes(d, n, 0, &need);
        CHECK_PTR(ws, "ws");
        if (ws_bytes < need)
            return fail(MINIKV_EINVAL, "workspace too small: %zu < %zu", ws_bytes, need);
        lse_buf = static_cast<float *>(ws);
    }
    CHECK(check_device());
    return hip_status(
        minikv::launch_prefill(static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                               static_cast<const uint16_t *>(v), static_cast<uint16_t *>(o),
                               lse_buf, score, d->batch, d->n_q_heads, d->n_kv_heads, n,
                               d->head_dim, static_cast<hipStream_t>(stream), true),
        "diffkv prefill launch");
}

int32_t minikv_tier_diffkv(const minikv_dims *d, int32_t n, const float *score, float alpha_hi,
                           float alpha_lo, int32_t *idx_hi, int32_t *idx_lo, int32_t *n_hi,
                           int32_t *n_lo, void *stream) {
    CHECK(check_dims(d));
    CHECK(check_len(d, n));
    if (!(alpha_lo <= alpha_hi))
        return fail(MINIKV_EINVAL, "need alpha_lo <= alpha_hi");
    if (n == 0) return ok();
    CHECK_PTR(score, "score");
    CHECK_PTR(idx_hi, "idx_hi");
    CHECK_PTR(idx_lo, "idx_lo");
    CHECK_PTR(n_hi, "n_hi");
    CHECK_PTR(n_lo, "n_lo");
    CHECK(check_device());
    return hip_status(minikv::launch_tier(score, d->batch * d->n_kv_heads, n, alpha_hi, alpha_lo,
                                          d->group_k, idx_hi, idx_lo, n_hi, n_lo,
                                          static_cast<hipStream_t>(stream)),
                      "tier launch");
}

int32_t minikv_pack_diffkv(const minikv_dims *d, int32_t n, const void *k, const void *v,
                           const int32_t *idx_hi, const int32_t *idx_lo, int32_t *n_hi,
                           int32_t *n_lo, minikv_mixed_cache *c, void *stream) {
    CHECK(check_dims(d));
    CHECK(check_len(d, n));
    if (!c) return fail(MINIKV_EINVAL, "cache is NULL");
    if (c->n_seg != 3 || c->flush_seg != 2)
        return fail(MINIKV_EINVAL, "DiffKV pack needs three segments, flush_seg 2");
    const int want[3][2] = {{8, 4}, {4, 2}, {8, 4}};
    for (int i = 0; i < 3; ++i)
        if (c->seg[i].key_bits != want[i][0] || c->seg[i].value_bits != want[i][1])
            return fail(MINIKV_EINVAL, "DiffKV segment %d must be K%dV%d", i, want[i][0],
                        want[i][1]);
    const int bound = n / d->group_k * d->group_k;
    if (c->seg[0].capacity < bound || c->seg[1].capacity < bound)
        return fail(MINIKV_ECAPACITY, "tier segments need capacity >= %d", bound);
    // the new state, validated as a whole before anything is launched
    minikv_mixed_cache next = *c;
    next.seg[0].n_unit = n_hi;
    next.seg[1].n_unit = n_lo;
    next.seg[0].n_packed = bound;
    next.seg[1].n_packed = bound;
    next.seg[2].n_unit = nullptr;
    next.seg[2].n_packed = 0;
    next.n_res = 0;
    CHECK(check_mixed(d, &next));
    if (n > 0) {
        CHECK_PTR(k, "k");
        CHECK_PTR(v, "v");
        CHECK_PTR(idx_hi, "idx_hi");
        CHECK_PTR(idx_lo, "idx_lo");
        CHECK_PTR(n_hi, "n_hi");
        CHECK_PTR(n_lo, "n_lo");
        CHECK(check_device());
        hipStream_t s = static_cast<hipStream_t>(stream);
        const int units = d->batch * d->n_kv_heads;
        minikv::PackSrc src;
        src.k = static_cast<const uint16_t *>(k);
        src.v = static_cast<const uint16_t *>(v);
        src.src_unit = (size_t)n * d->head_dim;
        src.n_rows = n;
        src.sel_unit = (size_t)n;
        for (int i = 0; i < 2; ++i) {
            src.sel = i == 0 ? idx_hi : idx_lo;
            const hipError_t e =
                minikv::launch_pack(src, units, bound, 0, 0, seg_view(d, &next, i), s, 0);
            if (e != hipSuccess) return hip_status(e, "pack launch");
        }
    }
    *c = next;
    return ok();
}

}  // extern "C"

// ============================================== fused prefill tail

namespace {

size_t tail_counter_off(const minikv_dims *d, int32_t n, int32_t lse_given) {
    size_t lse = 0;
    minikv_prefill_ws_bytes(d, n, lse_given, &lse);
    return (lse + 255) / 256 * 256;
}

}  // namespace

extern "C" {

int32_t minikv_prefill_tail_ws_bytes(const minikv_dims *d, int32_t n, int32_t lse_given,
                                     size_t *out) {
    CHECK(check_dims(d));
    CHECK(check_len(d, n));
    if (!out) return fail(MINIKV_EINVAL, "out is NULL");
    const size_t cnt = (size_t)d->batch * d->n_kv_heads * sizeof(uint32_t);
    *out = tail_counter_off(d, n, lse_given) + (cnt + 255) / 256 * 256;
    return ok();
}

int32_t minikv_prefill_select_pack(const minikv_dims *d, int32_t n, const void *q,
                                   const void *k, const void *v, void *o, float *col,
                                   float *lse, int32_t n_hh, int32_t n_recent, int32_t *sel,
                                   minikv_layer_cache *c, int32_t fuse_select, void *ws,
                                   size_t ws_bytes, void *stream) {
    CHECK(check_dims(d));
    CHECK(check_len(d, n));
    CHECK(check_select_args(d, n, n_hh, n_recent));
    CHECK(check_cache(d, c));
    if (fuse_select != 0 && fuse_select != 1)
        return fail(MINIKV_EINVAL, "fuse_select must be 0 or 1");
    const int32_t n_sel = n_hh + n_recent;
    const int32_t n_tok = (n_sel / d->group_k) * d->group_k;
    const int32_t n_tail = n_sel - n_tok;
    if (n_tok > c->capacity)
        return fail(MINIKV_ECAPACITY, "%d packed tokens exceed capacity %d", n_tok,
                    c->capacity);
    if (n_tail >= d->residual_cap)
        return fail(MINIKV_ECAPACITY, "residual tail %d >= residual_cap", n_tail);
    if (n == 0) {
        c->n_packed = c->n_res = 0;
        return ok();
    }
    CHECK_PTR(q, "q");
    CHECK_PTR(k, "k");
    CHECK_PTR(v, "v");
    CHECK_PTR(o, "o");
    CHECK_PTR(col, "col");
    if (n_sel > 0) CHECK_PTR(sel, "sel");
    if (lse) CHECK_PTR(lse, "lse");
    size_t need = 0;
    minikv_prefill_tail_ws_bytes(d, n, lse != nullptr, &need);
    CHECK_PTR(ws, "ws");
    if (ws_bytes < need)
        return fail(MINIKV_EINVAL, "workspace too small: %zu < %zu", ws_bytes, need);
    CHECK(check_device());
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *lse_buf = lse ? lse : static_cast<float *>(ws);
    uint32_t *cnt = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) +
                                                 tail_counter_off(d, n, lse != nullptr));
    const bool fuse = n_sel > 0 && fuse_select == 1;
    const minikv::FusedSelect fs{cnt, sel, n_hh, n_recent};
    hipError_t e = minikv::launch_prefill(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), static_cast<uint16_t *>(o), lse_buf, col, d->batch,
        d->n_q_heads, d->n_kv_heads, n, d->head_dim, s, false, fuse ? &fs : nullptr);
    if (e != hipSuccess) return hip_status(e, "prefill launch");
    if (n_sel > 0 && !fuse) {
        e = minikv::launch_select(col, d->batch * d->n_kv_heads, n, n_hh, n_recent, sel, s);
        if (e != hipSuccess) return hip_status(e, "select launch");
    }
    if (n_sel > 0) {
        minikv::PackSrc src;
        src.k = static_cast<const uint16_t *>(k);
        src.v = static_cast<const uint16_t *>(v);
        src.src_unit = (size_t)n * d->head_dim;
        src.sel = sel;
        src.sel_unit = (size_t)n_sel;
        src.n_rows = n;
        e = minikv::launch_pack(src, d->batch * d->n_kv_heads, n_tok, n_tail, 0, view_of(d, c),
                                s);
        if (e != hipSuccess) return hip_status(e, "pack launch");
    }
    c->n_packed = n_tok;
    c->n_res = n_tail;
    return ok();
}

}  // extern "C"
