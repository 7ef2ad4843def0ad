// Stand-ins for the HIP runtime and the library's kernel launchers, for the
// sanitizer build of the C ABI's host code (abi.cpp) on a machine without a
// GPU.  The HIP calls report "no device"; a launcher reaching here means the
// entry point got past its validation, which the driver counts.  The sizing
// helpers mirror the library's formulas closely enough for the validation
// paths the driver exercises.
#include <hip/hip_runtime.h>

#include "../../bit_quantized_attention_two_amd/csrc/launch.h"

int g_launches = 0;

extern "C" hipError_t hipGetDevice(int *d) {
    if (d) *d = 0;
    return hipErrorNoDevice;
}
extern "C" hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600 *, int) {
    return hipErrorNoDevice;
}
extern "C" const char *hipGetErrorString(hipError_t) { return "stub"; }

namespace minikv {
hipError_t launch_pack(const PackSrc &, int, int, int, int, const CacheView &, hipStream_t, int) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_complement(const int32_t *, int, int, int, int32_t *, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_append_copy(const uint16_t *, const uint16_t *, int, int, const CacheView &,
                              hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_decode(const uint16_t *, uint16_t *, int, int, int, int, const CacheView &,
                         const uint16_t *, const uint16_t *, void *, size_t, hipStream_t,
                         const MassOut *) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_decode_segs(const uint16_t *, uint16_t *, int, int, const CacheView *,
                              const int *, int, int, void *, size_t, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_prefill(const uint16_t *, const uint16_t *, const uint16_t *, uint16_t *,
                          float *, float *, int, int, int, int, int, hipStream_t, bool,
                          const FusedSelect *) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_select(const float *, int, int, int, int, int32_t *, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_tier(const float *, int, int, float, float, int, int32_t *, int32_t *,
                       int32_t *, int32_t *, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t decode_scratch(void **out) {
    *out = nullptr;
    return hipErrorNoDevice;
}
static size_t parts(int units, int g, int D, int splits) {
    return (size_t)units * splits * g * (D + 2) * sizeof(float);
}
size_t decode_ws_bytes(int units, int g, int D, int capacity) {
    return parts(units, g, D, capacity / 256 + 2);
}
size_t decode_mass_ws_bytes(int units, int g, int D, int capacity, int nr) {
    return decode_ws_bytes(units, g, D, capacity) + (size_t)units * g * (capacity + nr + 2) * 4;
}
int decode_max_capacity(int) { return 511 * 1024; }
size_t decode_plan_ws_bytes(int units, int g, int D, int n_packed, int, int, bool) {
    return parts(units, g, D, n_packed / 256 + 2);
}
size_t decode_segs_ws_bytes(int units, int g, int D, const int *caps, int n_seg) {
    int s = 1;
    for (int i = 0; i < n_seg; ++i) s += caps[i] / 256 + 1;
    return parts(units, g, D, s);
}
size_t decode_segs_plan_ws_bytes(int units, int g, int D, const CacheView *, const int *n,
                                 int n_seg, int) {
    int s = 1;
    for (int i = 0; i < n_seg; ++i) s += n[i] / 256 + 1;
    return parts(units, g, D, s);
}
}  // namespace minikv
