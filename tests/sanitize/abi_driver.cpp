// Sanitizer driver for the C ABI's host code: every host helper with valid
// and invalid arguments, and every compute entry point with arguments its
// validation must reject (and a few it must accept, reaching the stubbed
// launchers or the stubbed device check).  Exit status 0 iff every status
// code is the expected one; AddressSanitizer / UBSan abort on any error.
#include <cstdio>
#include <cstring>
#include <vector>

#include "minikv.h"

extern int g_launches;
static int g_fail = 0;

#define EXPECT(expr, want)                                                        \
    do {                                                                          \
        const int32_t _s = (expr);                                                \
        if (_s != (want)) {                                                       \
            std::printf("line %d: %s = %d, want %d (%s)\n", __LINE__, #expr, _s,  \
                        (int)(want), minikv_last_error());                        \
            ++g_fail;                                                             \
        }                                                                         \
    } while (0)

int main() {
    void *fake = reinterpret_cast<void *>(0x1000);
    void *odd = reinterpret_cast<void *>(0x1001);
    minikv_dims d{1, 4, 2, 128, 16, 16, 128};
    minikv_dims bad{1, 6, 4, 128, 16, 16, 128};
    minikv_dims badD{1, 4, 4, 96, 16, 16, 128};

    // host helpers
    std::vector<int32_t> k(40);
    int32_t r = 0;
    EXPECT(minikv_pyramid_budgets(4096, 32, 1, 4, 1, 4, 7, 1, k.data(), &r), MINIKV_OK);
    EXPECT(minikv_pyramid_budgets(8192, 40, 1, 4, 1, 4, 7, 0, k.data(), &r), MINIKV_OK);
    EXPECT(minikv_pyramid_budgets(-1, 32, 1, 4, 1, 4, 7, 1, k.data(), &r), MINIKV_EINVAL);
    EXPECT(minikv_pyramid_budgets(10, 0, 1, 4, 1, 4, 7, 1, k.data(), &r), MINIKV_EINVAL);
    EXPECT(minikv_pyramid_budgets(10, 2, 1, 4, 1, 4, 7, 1, nullptr, &r), MINIKV_EINVAL);
    uint64_t a = 0, b = 0;
    EXPECT(minikv_cache_bytes_closed_form(32, 32, 128, 4096, 512, 1, 2, 2, 16, &a, &b), MINIKV_OK);
    if (a != 335544320ull || b != 2415919104ull) { std::printf("closed form %llu %llu\n", (unsigned long long)a, (unsigned long long)b); ++g_fail; }
    EXPECT(minikv_cache_bytes_closed_form(0, 32, 128, 4096, 512, 1, 2, 2, 16, &a, &b), MINIKV_EINVAL);
    size_t lay[8], seg[6], sz = 0;
    EXPECT(minikv_cache_layout(&d, 4096, lay), MINIKV_OK);
    EXPECT(minikv_cache_layout(&d, 4095, lay), MINIKV_EINVAL);
    EXPECT(minikv_cache_layout(&bad, 4096, lay), MINIKV_EINVAL);
    EXPECT(minikv_cache_layout(&badD, 4096, lay), MINIKV_EUNSUPPORTED);
    EXPECT(minikv_cache_layout(nullptr, 4096, lay), MINIKV_EINVAL);
    EXPECT(minikv_segment_layout(&d, 8, 4, 4096, seg), MINIKV_OK);
    EXPECT(minikv_segment_layout(&d, 8, 8, 4096, seg), MINIKV_EINVAL);
    EXPECT(minikv_prefill_ws_bytes(&d, 131072, 0, &sz), MINIKV_OK);
    EXPECT(minikv_prefill_ws_bytes(&d, -5, 0, &sz), MINIKV_EINVAL);
    EXPECT(minikv_prefill_tail_ws_bytes(&d, 4096, 0, &sz), MINIKV_OK);
    EXPECT(minikv_decode_ws_bytes(&d, 4096, &sz), MINIKV_OK);
    EXPECT(minikv_decode_mass_ws_bytes(&d, 4096, &sz), MINIKV_OK);
    EXPECT(minikv_mikv_ws_bytes(&d, 1000, 500, &sz), MINIKV_OK);
    EXPECT(minikv_mikv_ws_bytes(&d, 1000, 1001, &sz), MINIKV_EINVAL);
    EXPECT(minikv_diffkv_ws_bytes(&d, 1000, 0, &sz), MINIKV_OK);
    if (std::strcmp(minikv_status_str(MINIKV_ECAPACITY), "MINIKV_ECAPACITY")) ++g_fail;
    if (minikv_version() != 100) ++g_fail;

    // compute entry points: rejected before any HIP call
    EXPECT(minikv_prefill_attn(&d, 100, nullptr, fake, fake, fake, (float *)fake, (float *)fake, nullptr), MINIKV_EINVAL);
    EXPECT(minikv_prefill_attn(&d, 100, odd, fake, fake, fake, (float *)fake, (float *)fake, nullptr), MINIKV_EINVAL);
    EXPECT(minikv_prefill_attn(&d, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), MINIKV_OK);
    EXPECT(minikv_select(&d, 10, (float *)fake, 8, 3, (int32_t *)fake, nullptr), MINIKV_EINVAL);
    EXPECT(minikv_prefill_select(&d, 64, fake, fake, fake, fake, (float *)fake, nullptr, 8, 8, (int32_t *)fake, fake, 16, nullptr), MINIKV_EINVAL);
    minikv_layer_cache c{(int32_t *)fake, (uint16_t *)fake, (uint16_t *)fake, (int32_t *)fake, (uint16_t *)fake, (uint16_t *)fake, (uint16_t *)fake, (uint16_t *)fake, 64, 48, 127};
    EXPECT(minikv_append(&d, &c, fake, fake, nullptr), MINIKV_ECAPACITY);
    if (c.n_packed != 48 || c.n_res != 127) ++g_fail;
    EXPECT(minikv_pack(&d, 200, fake, fake, (int32_t *)fake, 100, &c, nullptr), MINIKV_ECAPACITY);
    minikv_layer_cache empty = c;
    empty.n_packed = 0;
    empty.n_res = 0;
    EXPECT(minikv_decode_attn(&d, &empty, fake, fake, fake, 1 << 20, nullptr), MINIKV_EINVAL);
    EXPECT(minikv_decode_attn_noalloc(&d, &empty, fake, fake, nullptr), MINIKV_EINVAL);
    minikv_layer_cache one = c;
    one.n_packed = 16;
    one.n_res = 0;
    EXPECT(minikv_decode_attn(&d, &one, fake, fake, fake, 8, nullptr), MINIKV_EINVAL);
    EXPECT(minikv_decode_attn_mass(&d, &one, fake, fake, nullptr, 100, fake, 1 << 20, nullptr), MINIKV_EINVAL);
    EXPECT(minikv_prefill_select_pack(&d, 300, fake, fake, fake, fake, (float *)fake, nullptr, 75, 75, (int32_t *)fake, &one, 1, fake, 1 << 20, nullptr), MINIKV_ECAPACITY);
    EXPECT(minikv_prefill_select_pack(&d, 300, fake, fake, fake, fake, (float *)fake, nullptr, 8, 8, (int32_t *)fake, &one, 2, fake, 1 << 20, nullptr), MINIKV_EINVAL);
    // valid arguments reach the (stubbed) device check: EHIP
    EXPECT(minikv_decode_attn(&d, &one, fake, fake, fake, 1 << 20, nullptr), MINIKV_EHIP);
    EXPECT(minikv_prefill_attn(&d, 100, fake, fake, fake, fake, (float *)fake, (float *)fake, nullptr), MINIKV_EHIP);

    // mixed caches
    minikv_mixed_cache mc;
    std::memset(&mc, 0, sizeof(mc));
    for (int i = 0; i < 2; ++i) {
        minikv_segment &s = mc.seg[i];
        s.kq = (int32_t *)fake; s.k_scale = (uint16_t *)fake; s.k_zero = (uint16_t *)fake;
        s.vq = (int32_t *)fake; s.v_scale = (uint16_t *)fake; s.v_zero = (uint16_t *)fake;
        s.key_bits = i ? 2 : 4; s.value_bits = i ? 2 : 4; s.capacity = 256; s.n_packed = 0;
        s.n_unit = nullptr;
    }
    mc.n_seg = 2;
    mc.flush_seg = 0;
    mc.k_res = (uint16_t *)fake;
    mc.v_res = (uint16_t *)fake;
    mc.n_res = 0;
    EXPECT(minikv_decode_mixed_ws_bytes(&d, &mc, &sz), MINIKV_OK);
    EXPECT(minikv_decode_mixed(&d, &mc, fake, fake, fake, 1 << 20, nullptr), MINIKV_EINVAL);
    EXPECT(minikv_pack_mikv(&d, 1000, fake, fake, (int32_t *)fake, 500, &mc, fake, 1 << 20, nullptr), MINIKV_ECAPACITY);
    mc.seg[0].key_bits = 8; mc.seg[0].value_bits = 8;
    EXPECT(minikv_decode_mixed(&d, &mc, fake, fake, fake, 1 << 20, nullptr), MINIKV_EUNSUPPORTED);
    mc.seg[0].key_bits = 4; mc.seg[0].value_bits = 4;
    mc.n_seg = 4;
    EXPECT(minikv_decode_mixed(&d, &mc, fake, fake, fake, 1 << 20, nullptr), MINIKV_EINVAL);
    mc.n_seg = 2;
    EXPECT(minikv_pack_diffkv(&d, 1000, fake, fake, (int32_t *)fake, (int32_t *)fake, (int32_t *)fake, (int32_t *)fake, &mc, nullptr), MINIKV_EINVAL);
    EXPECT(minikv_tier_diffkv(&d, 1000, (float *)fake, 0.5f, 1.0f, (int32_t *)fake, (int32_t *)fake, (int32_t *)fake, (int32_t *)fake, nullptr), MINIKV_EINVAL);
    minikv_dims d32{1, 4, 2, 128, 16, 32, 128};
    EXPECT(minikv_decode_mixed(&d32, &mc, fake, fake, fake, 1 << 20, nullptr), MINIKV_EUNSUPPORTED);

    if (g_launches != 0) { std::printf("%d launches reached\n", g_launches); ++g_fail; }
    std::printf("%s: %d failures\n", g_fail ? "FAIL" : "ok", g_fail);
    return g_fail ? 1 : 0;
}
