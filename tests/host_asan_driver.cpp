// Host-side checks of libspecverify's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (test infrastructure, CPU only).  sv_api.cpp is
// linked against stub launchers: every call below is either refused by the
// host validation (the stubs must not run) or passes it and reaches a stub,
// which declines the launch (SV_ERR_LAUNCH).  Buffers are sized exactly, so a
// read or write past them is reported by the sanitizer.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <vector>

#include "libspecverify.h"
#include "sv_launch.h"

static int g_launches = 0;
static int g_failures = 0;

#define EXPECT(cond)                                                           \
    do {                                                                       \
        if (!(cond)) {                                                         \
            std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);     \
            ++g_failures;                                                      \
        }                                                                      \
    } while (0)

namespace sv {
static hipError_t declined() {
    ++g_launches;
    return hipErrorNotSupported;
}
hipError_t launch_budget(const float*, const int32_t*, int, int, const float*, int, int, int32_t*,
                         int32_t*, float*, int32_t*, void*, const PackTargets*, hipStream_t) {
    return declined();
}
hipError_t launch_allocate(const float*, const int32_t*, int, int, const int32_t*, int32_t*,
                           int32_t*, float*, int32_t*, void*, const PackTargets*, hipStream_t) {
    return declined();
}
size_t budget_workspace_bytes(int n_req, int k_max) {
    return 16 + (size_t)n_req * (size_t)k_max * 8;
}
hipError_t launch_uniform_k(const float*, const int32_t*, int, int, const float*, int, int,
                            int32_t*, int32_t*, double*, int32_t*, hipStream_t) {
    return declined();
}
hipError_t launch_pack(const int32_t*, const int32_t*, const int32_t*, int, int, int32_t*,
                       int32_t*, int32_t*, int32_t*, int32_t*, hipStream_t) {
    return declined();
}
size_t verify_workspace_bytes(int n_req, int k_max) {
    return (size_t)n_req * (size_t)(2 * k_max + 1) * 128 + 64;
}
hipError_t launch_verify(const VerifyArgs&, hipStream_t) { return declined(); }
hipError_t launch_accept_stats(const int32_t*, const int32_t*, int, int, uint64_t*, uint64_t*,
                               uint64_t*, hipStream_t) {
    return declined();
}
hipError_t launch_calibrate_update(float*, const float*, const float*, const float*,
                                   const int32_t*, const int32_t*, int, int, float, int32_t*,
                                   hipStream_t) {
    return declined();
}
hipError_t launch_calibrate_predict(const float*, const float*, const float*, const float*, int,
                                    int, float*, hipStream_t) {
    return declined();
}
hipError_t launch_philox_uniforms(uint64_t, uint64_t, int, int, float*, float*, hipStream_t) {
    return declined();
}
}  // namespace sv

int main() {
    // status strings, every code and an unknown one
    for (int s = 0; s <= 9; ++s) EXPECT(sv_status_str((sv_status)s) != nullptr);
    EXPECT(sv_status_str((sv_status)99) != nullptr);

    // cost shaping on exactly sized host buffers
    {
        const int raw_len = 129, out_len = 121, g = 16;  // ceil_16(120) = 128: 129 entries
        std::vector<float> raw(raw_len), out(out_len);
        for (int t = 0; t < raw_len; ++t) raw[t] = 1.0f + 0.01f * (float)((t * 37) % 11);
        EXPECT(sv_cost_table_prepare(raw.data(), raw_len, g, out.data(), out_len) == SV_OK);
        float run = raw[0];
        for (int t = 0; t < out_len; ++t) {
            const int padded = (t + g - 1) / g * g;
            run = raw[0];
            for (int u = 0; u <= padded; ++u) run = std::fmax(run, raw[u]);
            EXPECT(out[t] == run);
        }
        EXPECT(sv_cost_table_prepare(raw.data(), raw_len - 1, g, out.data(), out_len) ==
               SV_ERR_SHAPE);
        EXPECT(sv_cost_table_prepare(raw.data(), raw_len, 0, out.data(), out_len) == SV_ERR_SHAPE);
        raw[5] = std::numeric_limits<float>::quiet_NaN();
        EXPECT(sv_cost_table_prepare(raw.data(), raw_len, g, out.data(), out_len) == SV_ERR_VALUE);
        raw[5] = -1.0f;
        EXPECT(sv_cost_table_prepare(raw.data(), raw_len, g, out.data(), out_len) == SV_ERR_VALUE);
        EXPECT(sv_cost_table_prepare(nullptr, raw_len, g, out.data(), out_len) == SV_ERR_NULL);
        std::vector<float> one(1, 2.0f), o1(1);
        EXPECT(sv_cost_table_prepare(one.data(), 1, 1, o1.data(), 1) == SV_OK && o1[0] == 2.0f);
    }

    // stand-ins for device pointers: never dereferenced on the host
    alignas(16) static float fake[64];
    void* F = fake;
    const float* cf = fake;
    float* mf = fake;
    const int32_t* ci = reinterpret_cast<const int32_t*>(fake);
    int32_t* mi = reinterpret_cast<int32_t*>(fake);

    // workspace sizes and their limits
    EXPECT(sv_budget_workspace_bytes(-1, 3) == 0 && sv_budget_workspace_bytes(2, 65) == 0);
    EXPECT(sv_budget_workspace_bytes(8192, 2) == 0 && sv_budget_workspace_bytes(4, 3) > 0);
    EXPECT(sv_verify_workspace_bytes(1, 65) == 0 && sv_verify_workspace_bytes(-2, 1) == 0);
    EXPECT(sv_verify_workspace_bytes(SV_MAX_VERIFY_SLOTS / 15 + 1, 7) == 0);

    int before = g_launches;
    // budget: refusals launch nothing
    EXPECT(sv_budget_select(cf, ci, 4, 3, cf, 10, 0, 4, mi, mi, mf, mi, F, 1024, nullptr) ==
           SV_ERR_SHAPE);  // cost shorter than t_base + n k + 1
    EXPECT(sv_budget_select(cf, ci, 4, 3, nullptr, 64, 0, 4, mi, mi, mf, mi, F, 1024, nullptr) ==
           SV_ERR_NULL);
    EXPECT(sv_budget_select(cf, ci, 4, 3, cf, 64, -1, 4, mi, mi, mf, mi, F, 1024, nullptr) ==
           SV_ERR_VALUE);
    EXPECT(sv_budget_select(cf, ci, 4, 3, cf, 64, 0, 4, mi, mi, mf, mi, F, 8, nullptr) ==
           SV_ERR_WORKSPACE);
    EXPECT(sv_budget_select(cf, ci, 4, 65, cf, 4096, 0, 4, mi, mi, mf, mi, F, 1 << 20,
                            nullptr) == SV_ERR_SHAPE);
    EXPECT(sv_budget_select_pack(cf, ci, 4, 3, cf, 64, 0, 4, ci, ci, mi, mi, mf, nullptr, mi, mi,
                                 mi, mi, F, 1024, nullptr) == SV_ERR_NULL);
    EXPECT(sv_budget_allocate(cf, ci, 4, 3, nullptr, mi, mi, mf, mi, F, 1024, nullptr) ==
           SV_ERR_NULL);
    EXPECT(sv_uniform_k_select(cf, ci, 4, 3, cf, 12, 0, 4, mi, mi, nullptr, mi, nullptr) ==
           SV_ERR_SHAPE);
    EXPECT(sv_pack_varlen(ci, ci, ci, 4, 3, nullptr, mi, mi, mi, mi, nullptr) == SV_ERR_NULL);
    EXPECT(sv_pack_varlen(ci, ci, ci, -1, 3, mi, mi, mi, mi, mi, nullptr) == SV_ERR_SHAPE);
    EXPECT(g_launches == before);
    // ... and valid ones reach the (declining) launchers
    EXPECT(sv_budget_select(cf, ci, 4, 3, cf, 64, 0, 4, mi, mi, mf, mi, F, 1024, nullptr) ==
           SV_ERR_LAUNCH);
    EXPECT(sv_pack_varlen(ci, ci, ci, 4, 3, mi, mi, mi, mi, mi, nullptr) == SV_ERR_LAUNCH);
    EXPECT(sv_uniform_k_select(cf, ci, 4, 3, cf, 64, 0, 4, mi, mi, nullptr, mi, nullptr) ==
           SV_ERR_LAUNCH);
    EXPECT(g_launches == before + 3);

    // verify: refusals
    before = g_launches;
    auto verify = [&](int64_t tld, int64_t trows, int64_t dld, int dt, int vocab, int n, int k,
                      int mode, float temp, void* ws, size_t wsb) {
        return sv_verify(F, tld, trows, F, dld, (sv_dtype)dt, vocab, ci, ci, n, k, (sv_mode)mode,
                         temp, 1, 2, mi, mi, mf, mf, mf, nullptr, nullptr, mi, ws, wsb, nullptr);
    };
    const size_t wsb = 1 << 20;
    EXPECT(verify(32, 16, 32, 7, 32, 4, 3, 0, 1.0f, F, wsb) == SV_ERR_DTYPE);
    EXPECT(verify(32, 16, 32, SV_F32, 32, 4, 3, 5, 1.0f, F, wsb) == SV_ERR_VALUE);
    EXPECT(verify(32, 16, 32, SV_F32, 32, 4, 3, 0, 0.0f, F, wsb) == SV_ERR_VALUE);
    EXPECT(verify(32, 16, 32, SV_F32, 32, 4, 3, 0, std::nanf(""), F, wsb) == SV_ERR_VALUE);
    EXPECT(verify(32, 16, 32, SV_F32, 32, 4, 3, 0, 1e-39f, F, wsb) == SV_ERR_VALUE);
    EXPECT(verify(16, 16, 32, SV_F32, 32, 4, 3, 0, 1.0f, F, wsb) == SV_ERR_SHAPE);
    EXPECT(verify(32, -1, 32, SV_F32, 32, 4, 3, 0, 1.0f, F, wsb) == SV_ERR_SHAPE);
    EXPECT(verify(32, 16, 32, SV_F32, 0, 4, 3, 0, 1.0f, F, wsb) == SV_ERR_SHAPE);
    EXPECT(verify(32, 16, 32, SV_F32, 32, 4, 65, 0, 1.0f, F, wsb) == SV_ERR_SHAPE);
    EXPECT(verify(32, 16, 32, SV_F32, 32, SV_MAX_VERIFY_SLOTS, 3, 0, 1.0f, F, wsb) ==
           SV_ERR_SHAPE);
    EXPECT(verify(32, 16, 32, SV_F32, 32, 4, 3, 0, 1.0f, F, 64) == SV_ERR_WORKSPACE);
    EXPECT(verify(32, 16, 32, SV_F32, 32, 4, 3, 0, 1.0f, nullptr, wsb) == SV_ERR_WORKSPACE);
    EXPECT(sv_verify_stages(F, 32, 16, F, 32, SV_F32, 32, ci, ci, 4, 3, SV_STOCHASTIC, 1.0f, 0,
                            0, mi, mi, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, F,
                            wsb, 4, nullptr) == SV_ERR_VALUE);
    EXPECT(verify(32, 16, 32, SV_F32, 32, 0, 3, 0, 1.0f, nullptr, 0) == SV_OK);  // empty batch
    EXPECT(g_launches == before);
    EXPECT(verify(32, 16, 32, SV_BF16, 32, 4, 3, 1, 0.0f, F, wsb) == SV_ERR_LAUNCH);  // greedy
    EXPECT(g_launches == before + 1);

    // the rest of the calls: refusals, then one that passes
    before = g_launches;
    EXPECT(sv_accept_stats(ci, ci, 4, 65, nullptr, nullptr, nullptr, nullptr) == SV_ERR_SHAPE);
    EXPECT(sv_calibrate_update(mf, cf, cf, cf, ci, ci, 4, 3, -1.0f, mi, nullptr) == SV_ERR_VALUE);
    EXPECT(sv_calibrate_predict(nullptr, cf, cf, cf, 4, 3, mf, nullptr) == SV_ERR_NULL);
    EXPECT(sv_philox_uniforms(0, 0, -1, 2, mf, mf, nullptr) == SV_ERR_SHAPE);
    EXPECT(g_launches == before);
    EXPECT(sv_philox_uniforms(0, 0, 3, 2, mf, mf, nullptr) == SV_ERR_LAUNCH);

    if (g_failures) {
        std::fprintf(stderr, "%d check(s) failed\n", g_failures);
        return 1;
    }
    std::printf("host checks passed (%d launches reached the stubs)\n", g_launches);
    return 0;
}
