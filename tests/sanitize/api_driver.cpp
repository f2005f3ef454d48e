// Host-side run of the C ABI under AddressSanitizer and UndefinedBehavior-
// Sanitizer: every validation path, the status strings and the act-order
// permutation (pure host code).  Built as plain C++ (no device code): the
// kernel launchers are stubs that are never reached, because without a GPU
// every call that passes validation stops at the device check.  The limit
// queries return values large enough that no limit is hit here; the limits
// themselves are tested against the real library.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "mnb.h"
#include "mnb_acc4.hpp"
#include "mnb_internal.hpp"
#include "mnb_gidx.hpp"

namespace mnb {
int64_t gemv_max_k(bool, bool) { return int64_t(1) << 30; }
int64_t acc4_gemv_max_k() { return int64_t(1) << 30; }
int64_t gemm_mfma_max_k() { return int64_t(1) << 30; }
int64_t gemm_small_max_k() { return int64_t(1) << 30; }
int set_prefill_rows(int) { return 0; }
size_t gemm_small_workspace(const Layout&, int64_t) { return 0; }
hipError_t launch_repack(const Layout&, const uint8_t*, const void*, const uint8_t*, const int32_t*, void*,
                         hipStream_t) { std::abort(); }
hipError_t launch_permute_columns(const void*, const int32_t*, int64_t, int64_t, int, void*, hipStream_t)
{ std::abort(); }
hipError_t launch_unpack_debug(const Layout&, const void*, uint8_t*, float*, hipStream_t) { std::abort(); }
hipError_t launch_gemv(const Layout&, const WeightView&, const WeightView*, const void*, const int32_t*, bool,
                       const Bias&, void*, hipStream_t, const char**) { std::abort(); }
hipError_t launch_gemm_small(const Layout&, const WeightView&, const void*, int64_t, const Bias&, void*, void*,
                             hipStream_t, const char**) { std::abort(); }
hipError_t launch_gemm_mfma(const Layout&, const WeightView&, const void*, int64_t, const Bias&, void*,
                            hipStream_t, const char**) { std::abort(); }
hipError_t launch_acc4_gemv(const Layout&, const WeightView&, const float*, const float*, float*, _Float16*,
                            float*, hipStream_t, const char**) { std::abort(); }
hipError_t launch_acc4_quantize(const float*, int64_t, int64_t, _Float16*, float*, hipStream_t) { std::abort(); }
hipError_t launch_gemm_small_f32(const Layout&, const WeightView&, const void*, int64_t, const float*,
                                 const float*, float*, void*, hipStream_t, const char**, int, int64_t) { std::abort(); }
hipError_t launch_gemm_mfma_f32(const Layout&, const WeightView&, const void*, int64_t, const float*,
                                const float*, float*, hipStream_t, const char**, int, int64_t) { std::abort(); }
hipError_t launch_split_f32_rows(const float*, int64_t, int64_t, _Float16*, float*, hipStream_t) { std::abort(); }
hipError_t noalloc_scratch(int, void**) { std::abort(); }
int64_t gidx_max_m() { return int64_t(65535) * 64; }
hipError_t launch_gemm_gidx(const Layout&, const WeightView&, const void*, int64_t, bool, const int32_t*,
                            const Bias&, void*, hipStream_t, const char**) { std::abort(); }
}  // namespace mnb

static int failures = 0;

static void expect(mnb_status got, mnb_status want, const char* what)
{
    if (got != want) {
        std::printf("FAIL %s: status %d, expected %d (%s)\n", what, (int)got, (int)want, mnb_last_error());
        ++failures;
    }
}

static mnb_weight_desc desc(int64_t n, int64_t k, int g, int zp, int sdt)
{
    mnb_weight_desc d;
    std::memset(&d, 0, sizeof(d));
    d.n = n;
    d.k = k;
    d.group_size = g;
    d.has_zero_points = zp;
    d.scale_dtype = sdt;
    return d;
}

int main()
{
    const mnb_status OK = MNB_OK, INV = MNB_ERR_INVALID_ARGUMENT, UNS = MNB_ERR_UNSUPPORTED,
                     DEV = MNB_ERR_DEVICE;
    // aligned stand-ins for device pointers; never dereferenced
    void* fake = reinterpret_cast<void*>(uintptr_t(1) << 40);
    char* fakec = static_cast<char*>(fake);
    mnb_weight_desc d = desc(300, 512, 32, 1, MNB_F16);

    // descriptors
    expect(mnb_gemv(nullptr, fake, fake, MNB_F16, fake, nullptr), INV, "null descriptor");
    mnb_weight_desc bad = desc(-1, 512, 32, 1, MNB_F16);
    expect(mnb_gemv(&bad, fake, fake, MNB_F16, fake, nullptr), INV, "negative N");
    bad = desc(64, 0, 32, 1, MNB_F16);
    expect(mnb_gemv(&bad, fake, fake, MNB_F16, fake, nullptr), INV, "K = 0");
    bad = desc(64, 512, 24, 1, MNB_F16);
    expect(mnb_gemv(&bad, fake, fake, MNB_F16, fake, nullptr), INV, "group not a power of two");
    bad = desc(64, 512, 256, 1, MNB_F16);
    expect(mnb_gemv(&bad, fake, fake, MNB_F16, fake, nullptr), UNS, "group 256");
    bad = desc(64, 500, 32, 1, MNB_F16);
    expect(mnb_gemv(&bad, fake, fake, MNB_F16, fake, nullptr), UNS, "K not a multiple of the group");
    bad = desc(64, 512, 32, 2, MNB_F16);
    expect(mnb_gemv(&bad, fake, fake, MNB_F16, fake, nullptr), INV, "has_zero_points = 2");
    bad = desc(64, 512, 32, 1, 7);
    expect(mnb_gemv(&bad, fake, fake, MNB_F16, fake, nullptr), INV, "scale dtype");
    bad = desc(int64_t(1) << 40, 512, 32, 1, MNB_F16);
    expect(mnb_gemv(&bad, fake, fake, MNB_F16, fake, nullptr), INV, "N beyond 32 bits");
    if (mnb_repacked_bytes(&d) == 0) {
        std::printf("FAIL repacked_bytes\n");
        ++failures;
    }
    mnb_layout lay;
    expect(mnb_repacked_layout(&d, &lay), OK, "layout");
    expect(mnb_repacked_layout(&d, nullptr), INV, "layout NULL");

    // pointers, dtypes and sizes
    expect(mnb_gemv(&d, fakec + 8, fake, MNB_F16, fake, nullptr), INV, "misaligned weight");
    expect(mnb_gemv(&d, fake, fakec + 4, MNB_F16, fake, nullptr), INV, "misaligned activation");
    expect(mnb_gemv(&d, fake, fake, 5, fake, nullptr), INV, "activation dtype");
    expect(mnb_gemv(&d, fake, fake, MNB_F16, fake, nullptr), DEV, "valid decode call without a device");
    expect(mnb_gemv_gate_up_swiglu(&d, fake, nullptr, fake, MNB_F16, fake, nullptr), INV, "gate/up NULL");
    expect(mnb_gemm(&d, fake, fake, -1, MNB_F16, fake, nullptr, 0, nullptr), INV, "negative M");
    expect(mnb_gemm(&d, fake, fake, 0, MNB_F16, fake, nullptr, 0, nullptr), OK, "M = 0");
    const size_t wsf = mnb_gemm_workspace_bytes_for(&d, 8, MNB_F32);
    if (wsf != 256 + (4 * 8 * 512 + 255) / 256 * 256) {
        std::printf("FAIL fp32 workspace size %zu\n", wsf);
        ++failures;
    }
    expect(mnb_gemm(&d, fake, fake, 8, MNB_F32, fake, nullptr, 0, nullptr), INV, "fp32 GEMM without workspace");
    expect(mnb_gemm(&d, fake, fake, 8, MNB_F32, fake, fake, wsf - 1, nullptr), INV, "fp32 GEMM workspace too small");
    expect(mnb_gemm(&d, fake, fake, 8, MNB_F32, fake, fake, wsf, nullptr), DEV, "valid fp32 GEMM without a device");
    expect(mnb_gemm(&d, fake, fake, 64, MNB_F16, fake, nullptr, 0, nullptr), DEV, "valid GEMM without a device");
    expect(mnb_gemm_bias(&d, fake, fake, 4, MNB_F16, fake, -1, MNB_BIAS_FUSED, fake, nullptr, 0, nullptr), INV,
           "negative bias stride");
    expect(mnb_gemm_bias(&d, fake, fake, 4, MNB_F16, fake, 0, 9, fake, nullptr, 0, nullptr), INV, "bias mode");
    expect(mnb_gemm_bias(&d, fake, fake, 4, MNB_F16, fakec + 1, 0, MNB_BIAS_FUSED, fake, nullptr, 0, nullptr), INV,
           "misaligned bias");
    const size_t ws4 = mnb_gemm_accuracy4_workspace_bytes(&d, 40);
    expect(mnb_gemm_accuracy4(&d, fake, static_cast<const float*>(fake), 40, nullptr, static_cast<float*>(fake),
                              fake, ws4 - 1, nullptr), INV, "int8 workspace too small");
    expect(mnb_gemm_accuracy4(&d, fake, static_cast<const float*>(fake), 40, nullptr, static_cast<float*>(fake),
                              nullptr, ws4, nullptr), INV, "int8 workspace NULL");
    expect(mnb_gemm_accuracy4(&d, fake, static_cast<const float*>(fake), 1, nullptr, static_cast<float*>(fake),
                              nullptr, 0, nullptr), DEV, "valid int8 decode without a device");
    // the no-allocation form: validation, then the size limit, then the device
    const float* fa = static_cast<const float*>(fake);
    float* fy = static_cast<float*>(fake);
    expect(mnb_gemm_accuracy4_noalloc(&d, fake, fa, -1, nullptr, fy, nullptr), INV, "no-alloc negative M");
    expect(mnb_gemm_accuracy4_noalloc(&d, fake, fa, 0, nullptr, fy, nullptr), MNB_OK, "no-alloc M = 0");
    expect(mnb_gemm_accuracy4_noalloc(&d, fake, fa, 1 << 20, nullptr, fy, nullptr), UNS, "no-alloc beyond scratch");
    expect(mnb_gemm_accuracy4_noalloc(&d, fake, fa, 40, nullptr, fy, nullptr), DEV, "no-alloc without a device");
    expect(mnb_gemm_accuracy4_noalloc(&d, fake, fa, 1, nullptr, fy, nullptr), DEV, "no-alloc decode without a device");
    const size_t wsa = mnb_gemm_act_order_workspace_bytes(&d, 40, MNB_F16);
    expect(mnb_gemm_act_order(&d, fake, fake, 40, MNB_F16, nullptr, fake, fake, wsa, nullptr), INV, "perm NULL");
    expect(mnb_gemm_act_order(&d, fake, fake, 40, MNB_F16, static_cast<const int32_t*>(fake), fake, fake, wsa - 1,
                              nullptr), INV, "act-order workspace too small");
    // any g_idx: validation, then the device
    const int32_t* fg = static_cast<const int32_t*>(fake);
    expect(mnb_gemm_group_indices(&d, fake, fake, 40, MNB_F16, nullptr, nullptr, 0, MNB_BIAS_FUSED, fake, nullptr),
           INV, "group indices NULL");
    expect(mnb_gemm_group_indices(&d, fake, fake, 40, MNB_F16, fg, nullptr, -1, MNB_BIAS_FUSED, fake, nullptr), INV,
           "group indices negative bias stride");
    expect(mnb_gemm_group_indices(&d, fake, fake, 40, MNB_F16, fg, nullptr, 0, 7, fake, nullptr), INV,
           "group indices bias mode");
    expect(mnb_gemm_group_indices(&d, fake, fake, 40, MNB_F32, fg, nullptr, 0, MNB_BIAS_FUSED, fakec + 2, nullptr),
           INV, "group indices misaligned fp32 output");
    expect(mnb_gemm_group_indices(&d, fake, fake, 40, MNB_F16, reinterpret_cast<const int32_t*>(fakec + 4), nullptr,
                                  0, MNB_BIAS_FUSED, fake, nullptr), INV, "group indices misaligned g_idx");
    expect(mnb_gemm_group_indices(&d, fake, fakec + 8, 40, MNB_F16, fg, nullptr, 0, MNB_BIAS_FUSED, fake, nullptr),
           INV, "group indices misaligned activation");
    expect(mnb_gemm_group_indices(&d, fake, fake, int64_t(65535) * 64 + 1, MNB_F16, fg, nullptr, 0, MNB_BIAS_FUSED,
                                  fake, nullptr), UNS, "group indices M beyond the grid");
    expect(mnb_gemm_group_indices(&d, fake, fake, 0, MNB_F16, nullptr, nullptr, 0, MNB_BIAS_FUSED, fake, nullptr),
           MNB_OK, "group indices M = 0");
    expect(mnb_gemm_group_indices(&d, fake, fake, 40, MNB_F32, fg, fake, 512, MNB_BIAS_FUSED, fake, nullptr), DEV,
           "valid group-indices call without a device");
    expect(mnb_unpack_debug(&d, fakec + 16, nullptr, nullptr, nullptr), INV, "unpack misaligned");
    for (int s = -1; s < 6; ++s)
        if (std::strlen(mnb_status_string(s)) == 0) {
            std::printf("FAIL status string %d\n", s);
            ++failures;
        }

    // act order on the host: random group assignments, checked as a stable
    // sort of k by group; then the refusals
    unsigned seed = 12345u;
    for (int round = 0; round < 20; ++round) {
        const int g = 16 << (round % 4);
        const int64_t K = int64_t(g) * (1 + round * 3);
        mnb_weight_desc da = desc(40, K, g, 1, MNB_F16);
        std::vector<int32_t> gidx(K), perm(K);
        for (int64_t k = 0; k < K; ++k) gidx[k] = int32_t(k / g);
        for (int64_t k = K - 1; k > 0; --k) {  // Fisher-Yates with an LCG
            seed = seed * 1664525u + 1013904223u;
            const int64_t j = int64_t(seed % uint32_t(k + 1));
            std::swap(gidx[k], gidx[j]);
        }
        expect(mnb_act_order_permutation(&da, gidx.data(), perm.data()), OK, "permutation");
        std::vector<char> seen(K, 0);
        for (int64_t i = 0; i < K; ++i) {
            const int32_t k = perm[i];
            if (k < 0 || k >= K || seen[k] || gidx[k] != i / g || (i % g && perm[i - 1] > k)) {
                std::printf("FAIL permutation entry %lld\n", (long long)i);
                ++failures;
                break;
            }
            seen[k] = 1;
        }
        gidx[0] = int32_t(K / g);   // a group out of range
        expect(mnb_act_order_permutation(&da, gidx.data(), perm.data()), INV, "g_idx out of range");
        if (K / g > 1) {
            for (int64_t k = 0; k < K; ++k) gidx[k] = int32_t(k / g);
            gidx[0] = 1;             // group 0 one short, group 1 one over
            expect(mnb_act_order_permutation(&da, gidx.data(), perm.data()), UNS, "uneven groups");
        }
    }
    std::printf("%s: %d failures\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
