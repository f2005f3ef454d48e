// mnb_api.cpp -- the C ABI of include/mnb.h: host-side validation, shape-class
// dispatch and launches on the caller's stream.
//
// Validation follows the attribute and operand checks of
// onnx-runtime-ep-cuda 0.1.0-dev.3, src/kernels/matmul_nbits.rs
// (MatMulNBitsFactory::create, run, run_f16 and the require_* helpers): every
// check runs on the host before any HIP call, and an unsupported request is
// refused with a reason instead of being computed some other way.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mnb.h"
#include "mnb_acc4.hpp"
#include "mnb_internal.hpp"
#include "mnb_gidx.hpp"

using mnb::Layout;

namespace {

thread_local std::string g_error;
thread_local const char* g_variant = "";

mnb_status fail(mnb_status s, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_error = std::string("mnb: ") + buf;
    return s;
}

mnb_status ok(const char* variant)
{
    g_error.clear();
    g_variant = variant ? variant : "";
    return MNB_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

mnb_status check_desc(const mnb_weight_desc* w, Layout* L)
{
    if (!w) return fail(MNB_ERR_INVALID_ARGUMENT, "weight descriptor is NULL");
    if (w->n < 0) return fail(MNB_ERR_INVALID_ARGUMENT, "N must be >= 0 (got %lld)", (long long)w->n);
    if (w->k <= 0) return fail(MNB_ERR_INVALID_ARGUMENT, "K must be > 0 (got %lld)", (long long)w->k);
    const int g = w->group_size;
    if (g < 16 || (g & (g - 1)) != 0)
        return fail(MNB_ERR_INVALID_ARGUMENT, "block_size must be a power of 2 and >= 16 (got %d)", g);
    if (g > 128)
        return fail(MNB_ERR_UNSUPPORTED, "block_size %d not supported (16, 32, 64 or 128)", g);
    if (w->k % g != 0)
        return fail(MNB_ERR_UNSUPPORTED, "K=%lld is not a multiple of block_size %d",
                    (long long)w->k, g);
    if (w->has_zero_points != 0 && w->has_zero_points != 1)
        return fail(MNB_ERR_INVALID_ARGUMENT, "has_zero_points must be 0 or 1 (got %d)",
                    w->has_zero_points);
    if (w->scale_dtype != MNB_F16 && w->scale_dtype != MNB_F32)
        return fail(MNB_ERR_INVALID_ARGUMENT, "scale_dtype must be MNB_F16 or MNB_F32 (got %d)",
                    w->scale_dtype);
    if (w->reserved != 0) return fail(MNB_ERR_INVALID_ARGUMENT, "reserved field must be 0");
    if (w->n > INT32_MAX || w->k > INT32_MAX)
        return fail(MNB_ERR_INVALID_ARGUMENT, "N and K must fit in 32 bits");
    *L = mnb::make_layout(w->n, w->k, g, w->has_zero_points != 0, w->scale_dtype == MNB_F16);
    if (L->total < 0 || L->total > (int64_t(1) << 46))
        return fail(MNB_ERR_INVALID_ARGUMENT, "repacked size overflows");
    return MNB_OK;
}

mnb_status check_act_dtype(int32_t a_dtype)
{
    if (a_dtype != MNB_F16 && a_dtype != MNB_F32)
        return fail(MNB_ERR_INVALID_ARGUMENT, "a_dtype must be MNB_F16 or MNB_F32 (got %d)", a_dtype);
    return MNB_OK;
}

mnb_status check_ptr(const void* p, uintptr_t align, const char* name)
{
    if (!p) return fail(MNB_ERR_INVALID_ARGUMENT, "%s is NULL", name);
    if (!aligned(p, align))
        return fail(MNB_ERR_INVALID_ARGUMENT, "%s must be %u-byte aligned", name, (unsigned)align);
    return MNB_OK;
}

// A gfx950 device must be current.  The architecture is looked up once per
// device (a property query is not free); later calls cost one hipGetDevice.
mnb_status check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return fail(MNB_ERR_DEVICE, "no HIP device available");
    }
    static std::mutex mu;
    static signed char is_gfx950[64] = {0};  // 0 unknown, 1 yes, -1 no
    if (dev >= 64) return fail(MNB_ERR_DEVICE, "device index %d out of range", dev);
    if (is_gfx950[dev] == 0) {
        std::lock_guard<std::mutex> lock(mu);
        if (is_gfx950[dev] == 0) {
            hipDeviceProp_t prop;
            if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
                (void)hipGetLastError();
                return fail(MNB_ERR_DEVICE, "cannot query device %d", dev);
            }
            is_gfx950[dev] = std::string(prop.gcnArchName).rfind("gfx950", 0) == 0 ? 1 : -1;
        }
    }
    if (is_gfx950[dev] < 0) return fail(MNB_ERR_DEVICE, "device %d is not gfx950", dev);
    return MNB_OK;
}

mnb_status launched(hipError_t e, const char* variant)
{
    if (e != hipSuccess) return fail(MNB_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
    return ok(variant);
}

#define MNB_TRY(x)                           \
    do {                                     \
        const mnb_status s_ = (x);           \
        if (s_ != MNB_OK) return s_;         \
    } while (0)

}  // namespace

extern "C" {

size_t mnb_repacked_bytes(const mnb_weight_desc* w)
{
    Layout L;
    if (check_desc(w, &L) != MNB_OK) return 0;
    g_error.clear();
    return (size_t)L.total;
}

mnb_status mnb_repacked_layout(const mnb_weight_desc* w, mnb_layout* out)
{
    Layout L;
    MNB_TRY(check_desc(w, &L));
    if (!out) return fail(MNB_ERR_INVALID_ARGUMENT, "out is NULL");
    out->tiles = L.T;
    out->chunks = L.C;
    out->groups_per_chunk = L.Q;
    out->codes_offset = L.codes_off;
    out->codes_bytes = L.codes_bytes;
    out->scales_offset = L.scales_off;
    out->scales_bytes = L.scales_bytes;
    out->zero_points_offset = L.zp_off;
    out->zero_points_bytes = L.zp_bytes;
    out->range_flags_offset = L.flags_off;
    out->range_flags_bytes = L.flags_bytes;
    out->total_bytes = L.total;
    g_error.clear();
    return MNB_OK;
}

static mnb_status repack_common(const mnb_weight_desc* w, const uint8_t* packed, const void* scales,
                                const uint8_t* zero_points, const int32_t* perm, void* repacked,
                                void* stream)
{
    Layout L;
    MNB_TRY(check_desc(w, &L));
    MNB_TRY(check_ptr(repacked, 256, "repacked"));
    if (L.N == 0) return ok("repack");
    MNB_TRY(check_ptr(packed, 16, "packed"));
    MNB_TRY(check_ptr(scales, 16, "scales"));
    if (w->has_zero_points) {
        MNB_TRY(check_ptr(zero_points, 16, "zero_points"));
    } else if (zero_points) {
        return fail(MNB_ERR_INVALID_ARGUMENT, "zero_points given but has_zero_points is 0");
    }
    MNB_TRY(check_device());
    if (perm) MNB_TRY(check_ptr(perm, 4, "perm"));
    return launched(mnb::launch_repack(L, packed, scales, zero_points, perm, repacked,
                                       static_cast<hipStream_t>(stream)),
                    "repack");
}

mnb_status mnb_repack(const mnb_weight_desc* w, const uint8_t* packed, const void* scales,
                      const uint8_t* zero_points, void* repacked, void* stream)
{
    return repack_common(w, packed, scales, zero_points, nullptr, repacked, stream);
}

mnb_status mnb_act_order_permutation(const mnb_weight_desc* w, const int32_t* g_idx, int32_t* perm)
{
    Layout L;
    MNB_TRY(check_desc(w, &L));
    if (L.K == 0) return ok("act_order_permutation");
    if (!g_idx) return fail(MNB_ERR_INVALID_ARGUMENT, "g_idx is NULL");
    if (!perm) return fail(MNB_ERR_INVALID_ARGUMENT, "perm is NULL");
    std::vector<int64_t> next(L.kb, 0);
    for (int64_t k = 0; k < L.K; ++k) {
        const int32_t grp = g_idx[k];
        if (grp < 0 || grp >= L.kb)
            return fail(MNB_ERR_INVALID_ARGUMENT, "g_idx[%lld]=%d is outside 0..%lld", (long long)k, (int)grp,
                        (long long)(L.kb - 1));
        ++next[grp];
    }
    for (int64_t b = 0; b < L.kb; ++b)
        if (next[b] != L.g)
            return fail(MNB_ERR_UNSUPPORTED, "group %lld has %lld members; the repacked layout needs %d per group",
                        (long long)b, (long long)next[b], (int)L.g);
    // stable: the members of each group in increasing k
    for (int64_t b = 0; b < L.kb; ++b) next[b] = b * L.g;
    for (int64_t k = 0; k < L.K; ++k) perm[next[g_idx[k]]++] = (int32_t)k;
    return ok("act_order_permutation");
}

mnb_status mnb_repack_act_order(const mnb_weight_desc* w, const uint8_t* packed, const void* scales,
                                const uint8_t* zero_points, const int32_t* perm, void* repacked,
                                void* stream)
{
    if (!perm) return fail(MNB_ERR_INVALID_ARGUMENT, "perm is NULL");
    return repack_common(w, packed, scales, zero_points, perm, repacked, stream);
}

static mnb_status gemv_common(const mnb_weight_desc* w, const void* gate, const void* up,
                              const void* a, int32_t a_dtype, const mnb::Bias& bias, void* y,
                              void* stream, const int32_t* perm = nullptr)
{
    Layout L;
    MNB_TRY(check_desc(w, &L));
    MNB_TRY(check_act_dtype(a_dtype));
    const bool f16 = a_dtype == MNB_F16;
    if (L.K > mnb::gemv_max_k(f16, perm != nullptr))
        return fail(MNB_ERR_UNSUPPORTED, "K=%lld exceeds the decode GEMV limit %lld for %s activations",
                    (long long)L.K, (long long)mnb::gemv_max_k(f16, perm != nullptr), f16 ? "fp16" : "fp32");
    if (L.N == 0) return ok("noop");
    MNB_TRY(check_ptr(gate, 256, up ? "gate_repacked" : "repacked"));
    if (up) MNB_TRY(check_ptr(up, 256, "up_repacked"));
    MNB_TRY(check_ptr(a, 16, "a"));
    MNB_TRY(check_ptr(y, f16 ? 2 : 4, "y"));
    if (bias.ptr) MNB_TRY(check_ptr(bias.ptr, f16 ? 2 : 4, "bias"));
    MNB_TRY(check_device());
    const char* variant = "";
    const mnb::WeightView gv = mnb::view_of(L, gate);
    mnb::WeightView uv;
    if (up) uv = mnb::view_of(L, up);
    return launched(mnb::launch_gemv(L, gv, up ? &uv : nullptr, a, perm, f16, bias, y,
                                     static_cast<hipStream_t>(stream), &variant),
                    variant);
}

mnb_status mnb_gemv(const mnb_weight_desc* w, const void* repacked, const void* a, int32_t a_dtype,
                    void* y, void* stream)
{
    return gemv_common(w, repacked, nullptr, a, a_dtype, mnb::Bias(), y, stream);
}

mnb_status mnb_gemv_gate_up_swiglu(const mnb_weight_desc* w, const void* gate_repacked,
                                   const void* up_repacked, const void* a, int32_t a_dtype,
                                   void* y, void* stream)
{
    if (!up_repacked) return fail(MNB_ERR_INVALID_ARGUMENT, "up_repacked is NULL");
    return gemv_common(w, gate_repacked, up_repacked, a, a_dtype, mnb::Bias(), y, stream);
}

// Up to kSliceMaxM fp16 rows (M for fp16 and int8 activations, 2M for fp32
// ones) run the small-M kernel, once per slice of at most 16 rows: above 16
// rows the prefill GEMM's grid covers too few CUs at these heights
// (N = 14336, K = 4096: 35-40 us at M = 17..32 against 16.3-17.4 us in two
// slices, about 25 us in three).  More rows run the prefill GEMM.
constexpr int64_t kSliceMaxM = 48;

static size_t workspace_for(const Layout& L, int64_t m)
{
    if (m >= 2 && m <= kSliceMaxM) return mnb::gemm_small_workspace(L, m < 16 ? m : 16);
    return 0;
}

// fp32 activations with M > 1: the row scales (fp32 [M]) at offset 0, then
// at the next 256-byte boundary the (hi, lo) fp16 row pairs [2M, K], then the
// workspace of the GEMM that runs on those 2M rows.
static size_t f32_scale_bytes(int64_t m) { return (size_t)((4 * m + 255) / 256 * 256); }
static size_t f32_rows_bytes(const Layout& L, int64_t m) { return (size_t)((4 * m * L.K + 255) / 256 * 256); }

static size_t workspace_for(const Layout& L, int64_t m, int32_t a_dtype)
{
    if (a_dtype == MNB_F32 && m > 1) return f32_scale_bytes(m) + f32_rows_bytes(L, m) + workspace_for(L, 2 * m);
    return workspace_for(L, m);
}

size_t mnb_gemm_workspace_bytes(const mnb_weight_desc* w, int64_t m)
{
    return mnb_gemm_workspace_bytes_for(w, m, MNB_F16);
}

size_t mnb_gemm_workspace_bytes_for(const mnb_weight_desc* w, int64_t m, int32_t a_dtype)
{
    Layout L;
    if (check_desc(w, &L) != MNB_OK) return 0;
    if (check_act_dtype(a_dtype) != MNB_OK) return 0;
    if (m < 0) {
        fail(MNB_ERR_INVALID_ARGUMENT, "M must be >= 0");
        return 0;
    }
    if (m > INT64_MAX / 8 / L.K) {
        fail(MNB_ERR_INVALID_ARGUMENT, "M*K overflows");
        return 0;
    }
    g_error.clear();
    return workspace_for(L, m, a_dtype);
}


// Both GEMMs have 32-bit buffer offsets.
static mnb_status check_gemm_k(const Layout& L, int64_t rows)
{
    if (rows >= 2 && rows <= kSliceMaxM && L.K > mnb::gemm_small_max_k())
        return fail(MNB_ERR_UNSUPPORTED, "K=%lld exceeds the small-M GEMM limit %lld (2 <= rows <= %lld)",
                    (long long)L.K, (long long)mnb::gemm_small_max_k(), (long long)kSliceMaxM);
    if (rows > kSliceMaxM && L.K > mnb::gemm_mfma_max_k())
        return fail(MNB_ERR_UNSUPPORTED, "K=%lld exceeds the prefill GEMM limit %lld (rows > %lld)", (long long)L.K,
                    (long long)mnb::gemm_mfma_max_k(), (long long)kSliceMaxM);
    return MNB_OK;
}

// fp32 activations, M > 1: each row split into a (hi, lo) pair of fp16 rows
// scaled by a power of two, then the fp16 GEMM on the 2M rows with an epilogue
// that adds each pair and scales it back.
static mnb_status gemm_f32_rows(const mnb_weight_desc* w, const Layout& L, const void* repacked, const void* a,
                                int64_t m, const mnb::Bias& bias, void* y, void* workspace,
                                size_t workspace_bytes, void* stream)
{
    if (m > INT64_MAX / 8 / L.K) return fail(MNB_ERR_INVALID_ARGUMENT, "M*K overflows");
    if (2 * m > INT32_MAX) return fail(MNB_ERR_INVALID_ARGUMENT, "2M must fit in 32 bits");
    if (L.N == 0) return ok("noop");
    MNB_TRY(check_gemm_k(L, 2 * m));
    const size_t need = workspace_for(L, m, MNB_F32);
    if (workspace_bytes < need)
        return fail(MNB_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes given, %zu needed (fp32 activations, "
                    "mnb_gemm_workspace_bytes_for)", workspace_bytes, need);
    MNB_TRY(check_ptr(workspace, 256, "workspace"));
    MNB_TRY(check_ptr(repacked, 256, "repacked"));
    MNB_TRY(check_ptr(a, 16, "a"));
    MNB_TRY(check_ptr(y, 4, "y"));
    if (bias.ptr) MNB_TRY(check_ptr(bias.ptr, 4, "bias"));
    MNB_TRY(check_device());
    const mnb::WeightView v = mnb::view_of(L, repacked);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* rs = reinterpret_cast<float*>(ws);
    _Float16* hl = reinterpret_cast<_Float16*>(ws + f32_scale_bytes(m));
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = mnb::launch_split_f32_rows(static_cast<const float*>(a), m, L.K, hl, rs, s);
    if (e != hipSuccess) return launched(e, "f32_split");
    const char* variant = "";
    const float* b = static_cast<const float*>(bias.ptr);
    if (2 * m <= kSliceMaxM) {
        // slices of 8 rows: their 16 (hi, lo) fp16 rows, row scales, outputs
        // and per-row bias
        e = hipSuccess;
        for (int64_t r0 = 0; r0 < m && e == hipSuccess; r0 += 8) {
            const int64_t rows = m - r0 < 8 ? m - r0 : 8;
            e = mnb::launch_gemm_small_f32(L, v, hl + 2 * r0 * L.K, 2 * rows, rs + r0, b ? b + r0 * bias.row_stride : b,
                                           static_cast<float*>(y) + r0 * L.N,
                                           ws + f32_scale_bytes(m) + f32_rows_bytes(L, m), s, &variant, 1,
                                           bias.row_stride);
        }
    } else
        e = mnb::launch_gemm_mfma_f32(L, v, hl, 2 * m, rs, b, static_cast<float*>(y), s, &variant, 1, bias.row_stride);
    return launched(e, variant);
}

static mnb_status gemm_common(const mnb_weight_desc* w, const void* repacked, const void* a, int64_t m,
                              int32_t a_dtype, const mnb::Bias& bias, void* y, void* workspace,
                              size_t workspace_bytes, void* stream)
{
    Layout L;
    MNB_TRY(check_desc(w, &L));
    MNB_TRY(check_act_dtype(a_dtype));
    if (m < 0) return fail(MNB_ERR_INVALID_ARGUMENT, "M must be >= 0 (got %lld)", (long long)m);
    if (m > INT32_MAX) return fail(MNB_ERR_INVALID_ARGUMENT, "M must fit in 32 bits");
    if (m == 1) return gemv_common(w, repacked, nullptr, a, a_dtype, bias, y, stream);
    if (m > 1 && a_dtype == MNB_F32) return gemm_f32_rows(w, L, repacked, a, m, bias, y, workspace, workspace_bytes, stream);
    const size_t need = workspace_for(L, m);
    if (m == 0 || L.N == 0) return ok("noop");
    MNB_TRY(check_gemm_k(L, m));
    if (workspace_bytes < need)
        return fail(MNB_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes given, %zu needed",
                    workspace_bytes, need);
    if (need > 0) MNB_TRY(check_ptr(workspace, 16, "workspace"));
    MNB_TRY(check_ptr(repacked, 256, "repacked"));
    MNB_TRY(check_ptr(a, 16, "a"));
    MNB_TRY(check_ptr(y, 2, "y"));
    if (bias.ptr) MNB_TRY(check_ptr(bias.ptr, 2, "bias"));
    MNB_TRY(check_device());
    const mnb::WeightView v = mnb::view_of(L, repacked);
    const char* variant = "";
    hipError_t e;
    if (m <= kSliceMaxM) {
        // 16-row slices of A, Y and a per-row bias, one small-M launch each
        // (the small-M kernel needs no workspace)
        e = hipSuccess;
        for (int64_t r0 = 0; r0 < m && e == hipSuccess; r0 += 16) {
            mnb::Bias b = bias;
            if (b.ptr && b.row_stride) b.ptr = static_cast<const uint16_t*>(b.ptr) + r0 * b.row_stride;
            e = mnb::launch_gemm_small(L, v, static_cast<const uint16_t*>(a) + r0 * L.K, m - r0 < 16 ? m - r0 : 16, b,
                                       static_cast<uint16_t*>(y) + r0 * L.N, workspace,
                                       static_cast<hipStream_t>(stream), &variant);
        }
    } else {
        e = mnb::launch_gemm_mfma(L, v, a, m, bias, y, static_cast<hipStream_t>(stream), &variant);
    }
    return launched(e, variant);
}

mnb_status mnb_gemm(const mnb_weight_desc* w, const void* repacked, const void* a, int64_t m,
                    int32_t a_dtype, void* y, void* workspace, size_t workspace_bytes, void* stream)
{
    return gemm_common(w, repacked, a, m, a_dtype, mnb::Bias(), y, workspace, workspace_bytes, stream);
}

mnb_status mnb_gemm_bias(const mnb_weight_desc* w, const void* repacked, const void* a, int64_t m,
                         int32_t a_dtype, const void* bias, int64_t bias_row_stride,
                         int32_t bias_mode, void* y, void* workspace, size_t workspace_bytes,
                         void* stream)
{
    if (bias_mode != MNB_BIAS_FUSED && bias_mode != MNB_BIAS_AFTER_ROUND)
        return fail(MNB_ERR_INVALID_ARGUMENT, "bias_mode must be MNB_BIAS_FUSED or MNB_BIAS_AFTER_ROUND (got %d)",
                    (int)bias_mode);
    if (bias_row_stride < 0)
        return fail(MNB_ERR_INVALID_ARGUMENT, "bias_row_stride must be >= 0 (got %lld)",
                    (long long)bias_row_stride);
    if (bias && m > 1 && w && bias_row_stride > (INT64_MAX / 4 - w->n) / (m - 1))
        return fail(MNB_ERR_INVALID_ARGUMENT, "bias extent (M-1)*%lld + N overflows", (long long)bias_row_stride);
    mnb::Bias b;
    b.ptr = bias;
    b.row_stride = bias_row_stride;
    b.after_round = bias_mode == MNB_BIAS_AFTER_ROUND ? 1 : 0;
    return gemm_common(w, repacked, a, m, a_dtype, b, y, workspace, workspace_bytes, stream);
}

static size_t act_order_a_bytes(const Layout& L, int64_t m, int32_t a_dtype)
{
    const int64_t elem = a_dtype == MNB_F32 ? 4 : 2;
    return (size_t)(((m * L.K * elem) + 255) / 256 * 256);
}

size_t mnb_gemm_act_order_workspace_bytes(const mnb_weight_desc* w, int64_t m, int32_t a_dtype)
{
    Layout L;
    if (check_desc(w, &L) != MNB_OK) return 0;
    if (m < 0 || check_act_dtype(a_dtype) != MNB_OK) return 0;
    if (L.K > 0 && m > INT64_MAX / 16 / L.K) {
        fail(MNB_ERR_INVALID_ARGUMENT, "M*K overflows");
        return 0;
    }
    g_error.clear();
    return act_order_a_bytes(L, m, a_dtype) + workspace_for(L, m, a_dtype);
}

mnb_status mnb_gemm_act_order(const mnb_weight_desc* w, const void* repacked, const void* a, int64_t m,
                              int32_t a_dtype, const int32_t* perm, void* y, void* workspace,
                              size_t workspace_bytes, void* stream)
{
    Layout L;
    MNB_TRY(check_desc(w, &L));
    MNB_TRY(check_act_dtype(a_dtype));
    if (m < 0) return fail(MNB_ERR_INVALID_ARGUMENT, "M must be >= 0 (got %lld)", (long long)m);
    if (m == 0 || L.N == 0) return ok("noop");
    if (m > INT32_MAX) return fail(MNB_ERR_INVALID_ARGUMENT, "M must fit in 32 bits");
    if (L.K > 0 && m > INT64_MAX / 16 / L.K) return fail(MNB_ERR_INVALID_ARGUMENT, "M*K overflows");
    MNB_TRY(check_gemm_k(L, a_dtype == MNB_F32 ? 2 * m : m));
    const size_t a_bytes = act_order_a_bytes(L, m, a_dtype);
    const size_t need = a_bytes + workspace_for(L, m, a_dtype);
    if (workspace_bytes < need)
        return fail(MNB_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes given, %zu needed",
                    workspace_bytes, need);
    MNB_TRY(check_ptr(workspace, 256, "workspace"));
    if (!perm) return fail(MNB_ERR_INVALID_ARGUMENT, "perm is NULL");
    MNB_TRY(check_ptr(perm, 4, "perm"));
    MNB_TRY(check_ptr(a, 16, "a"));
    // decode: the GEMV gathers A's columns itself while it stages them,
    // when the two copies fit in its LDS and perm is 16-byte aligned
    if (m == 1 && L.K <= mnb::gemv_max_k(a_dtype == MNB_F16, true) &&
        reinterpret_cast<uintptr_t>(perm) % 16 == 0)
        return gemv_common(w, repacked, nullptr, a, a_dtype, mnb::Bias(), y, stream, perm);
    MNB_TRY(check_device());
    // A's columns in the repacked order, then the ordinary call on them
    const hipError_t e = mnb::launch_permute_columns(a, perm, m, L.K, a_dtype == MNB_F32 ? 4 : 2, workspace,
                                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return launched(e, "act_order_permute");
    return gemm_common(w, repacked, workspace, m, a_dtype, mnb::Bias(), y,
                       static_cast<unsigned char*>(workspace) + a_bytes, workspace_bytes - a_bytes, stream);
}

mnb_status mnb_gemm_group_indices(const mnb_weight_desc* w, const void* repacked, const void* a, int64_t m,
                                  int32_t a_dtype, const int32_t* g_idx, const void* bias,
                                  int64_t bias_row_stride, int32_t bias_mode, void* y, void* stream)
{
    Layout L;
    MNB_TRY(check_desc(w, &L));
    MNB_TRY(check_act_dtype(a_dtype));
    if (bias_mode != MNB_BIAS_FUSED && bias_mode != MNB_BIAS_AFTER_ROUND)
        return fail(MNB_ERR_INVALID_ARGUMENT, "bias_mode must be MNB_BIAS_FUSED or MNB_BIAS_AFTER_ROUND (got %d)",
                    (int)bias_mode);
    if (bias_row_stride < 0)
        return fail(MNB_ERR_INVALID_ARGUMENT, "bias_row_stride must be >= 0 (got %lld)",
                    (long long)bias_row_stride);
    if (m < 0) return fail(MNB_ERR_INVALID_ARGUMENT, "M must be >= 0 (got %lld)", (long long)m);
    if (m > mnb::gidx_max_m())
        return fail(MNB_ERR_UNSUPPORTED, "M must be at most %lld (got %lld)", (long long)mnb::gidx_max_m(),
                    (long long)m);
    if (bias && m > 1 && bias_row_stride > (INT64_MAX / 4 - L.N) / (m - 1))
        return fail(MNB_ERR_INVALID_ARGUMENT, "bias extent (M-1)*%lld + N overflows", (long long)bias_row_stride);
    if (L.K > INT32_MAX - mnb::kChunkK) return fail(MNB_ERR_UNSUPPORTED, "K too large for the group-index kernel");
    if (m == 0 || L.N == 0) return ok("noop");
    if (L.K > 0 && !g_idx) return fail(MNB_ERR_INVALID_ARGUMENT, "g_idx is NULL");
    MNB_TRY(check_ptr(repacked, 256, "repacked"));
    const uintptr_t elem = a_dtype == MNB_F32 ? 4 : 2;
    MNB_TRY(check_ptr(a, 16, "a"));
    MNB_TRY(check_ptr(y, elem, "y"));
    if (g_idx) MNB_TRY(check_ptr(g_idx, 16, "g_idx"));
    if (bias) MNB_TRY(check_ptr(bias, elem, "bias"));
    MNB_TRY(check_device());
    mnb::Bias b;
    b.ptr = bias;
    b.row_stride = bias_row_stride;
    b.after_round = bias_mode == MNB_BIAS_AFTER_ROUND ? 1 : 0;
    const char* variant = "";
    const hipError_t e = mnb::launch_gemm_gidx(L, mnb::view_of(L, repacked), a, m, a_dtype == MNB_F16, g_idx, b, y,
                                               static_cast<hipStream_t>(stream), &variant);
    return launched(e, variant);
}

// int8 activations (accuracy_level 4): the workspace holds the activation
// scales (fp32 [M]) at offset 0 and the codes (fp16 integers [M, K]) at the
// next 256-byte boundary, then the small-M GEMM's own workspace.
static size_t acc4_scale_bytes(int64_t m) { return (size_t)((4 * m + 255) / 256 * 256); }
static size_t acc4_codes_bytes(const Layout& L, int64_t m) { return (size_t)((2 * m * L.K + 255) / 256 * 256); }

size_t mnb_gemm_accuracy4_workspace_bytes(const mnb_weight_desc* w, int64_t m)
{
    Layout L;
    if (check_desc(w, &L) != MNB_OK) return 0;
    if (m < 0 || (L.K > 0 && m > INT64_MAX / 4 / L.K)) return 0;
    g_error.clear();
    return acc4_scale_bytes(m) + acc4_codes_bytes(L, m) + workspace_for(L, m);
}

static mnb_status accuracy4_common(const mnb_weight_desc* w, const void* repacked, const float* a, int64_t m,
                                   const float* bias, float* y, void* workspace, size_t workspace_bytes,
                                   void* stream)
{
    Layout L;
    MNB_TRY(check_desc(w, &L));
    if (m < 0) return fail(MNB_ERR_INVALID_ARGUMENT, "M must be >= 0 (got %lld)", (long long)m);
    if (m > INT32_MAX) return fail(MNB_ERR_INVALID_ARGUMENT, "M must fit in 32 bits");
    if (m == 0 || L.N == 0) return ok("noop");
    if (m > INT64_MAX / 4 / L.K) return fail(MNB_ERR_INVALID_ARGUMENT, "M*K overflows");
    if (m == 1 && L.K > mnb::acc4_gemv_max_k())
        return fail(MNB_ERR_UNSUPPORTED, "K=%lld exceeds the int8-activation decode limit %lld",
                    (long long)L.K, (long long)mnb::acc4_gemv_max_k());
    MNB_TRY(check_gemm_k(L, m));
    const size_t need = acc4_scale_bytes(m) + acc4_codes_bytes(L, m) + workspace_for(L, m);
    // the decode GEMV needs no workspace; given one, it receives the codes
    if ((m > 1 || workspace) && workspace_bytes < need)
        return fail(MNB_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes given, %zu needed",
                    workspace_bytes, need);
    if (m > 1 || workspace) MNB_TRY(check_ptr(workspace, 256, "workspace"));
    MNB_TRY(check_ptr(repacked, 256, "repacked"));
    MNB_TRY(check_ptr(a, 16, "a"));
    MNB_TRY(check_ptr(y, 4, "y"));
    if (bias) MNB_TRY(check_ptr(bias, 4, "bias"));
    MNB_TRY(check_device());
    const mnb::WeightView v = mnb::view_of(L, repacked);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* sc = reinterpret_cast<float*>(ws);
    _Float16* q = ws ? reinterpret_cast<_Float16*>(ws + acc4_scale_bytes(m)) : nullptr;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const char* variant = "";
    if (m == 1) return launched(mnb::launch_acc4_gemv(L, v, a, bias, y, q, sc, s, &variant), variant);
    hipError_t e = mnb::launch_acc4_quantize(a, m, L.K, q, sc, s);
    if (e != hipSuccess) return launched(e, "accuracy4_quantize");
    if (m <= kSliceMaxM) {
        // slices of 16 rows: their codes, row scales and outputs
        for (int64_t r0 = 0; r0 < m && e == hipSuccess; r0 += 16)
            e = mnb::launch_gemm_small_f32(L, v, q + r0 * L.K, m - r0 < 16 ? m - r0 : 16, sc + r0, bias, y + r0 * L.N,
                                           ws + acc4_scale_bytes(m) + acc4_codes_bytes(L, m), s, &variant);
    } else
        e = mnb::launch_gemm_mfma_f32(L, v, q, m, sc, bias, y, s, &variant);
    return launched(e, variant);
}

mnb_status mnb_gemm_accuracy4(const mnb_weight_desc* w, const void* repacked, const float* a, int64_t m,
                              const float* bias, float* y, void* workspace, size_t workspace_bytes,
                              void* stream)
{
    return accuracy4_common(w, repacked, a, m, bias, y, workspace, workspace_bytes, stream);
}

}  // extern "C"

extern "C" {

mnb_status mnb_gemm_accuracy4_noalloc(const mnb_weight_desc* w, const void* repacked, const float* a, int64_t m,
                                      const float* bias, float* y, void* stream)
{
    Layout L;
    MNB_TRY(check_desc(w, &L));
    if (m < 0) return fail(MNB_ERR_INVALID_ARGUMENT, "M must be >= 0 (got %lld)", (long long)m);
    if (m == 0 || L.N == 0) return ok("noop");
    if (m > INT32_MAX) return fail(MNB_ERR_INVALID_ARGUMENT, "M must fit in 32 bits");
    if (m > INT64_MAX / 4 / L.K) return fail(MNB_ERR_INVALID_ARGUMENT, "M*K overflows");
    // the decode GEMV keeps the codes on chip and needs no workspace
    if (m == 1) return accuracy4_common(w, repacked, a, m, bias, y, nullptr, 0, stream);
    const size_t need = acc4_scale_bytes(m) + acc4_codes_bytes(L, m) + workspace_for(L, m);
    if (need > (size_t)MNB_NOALLOC_SCRATCH_BYTES)
        return fail(MNB_ERR_UNSUPPORTED, "the request needs %zu bytes of workspace; the no-allocation form holds %zu",
                    need, (size_t)MNB_NOALLOC_SCRATCH_BYTES);
    MNB_TRY(check_device());
    int dev = -1;
    (void)hipGetDevice(&dev);
    void* ws = nullptr;
    const hipError_t e = mnb::noalloc_scratch(dev, &ws);
    if (e != hipSuccess) return fail(MNB_ERR_DEVICE, "cannot locate the scratch array on device %d: %s", dev,
                                     hipGetErrorString(e));
    return accuracy4_common(w, repacked, a, m, bias, y, ws, (size_t)MNB_NOALLOC_SCRATCH_BYTES, stream);
}

mnb_status mnb_unpack_debug(const mnb_weight_desc* w, const void* repacked, uint8_t* codes,
                            float* w_f32, void* stream)
{
    Layout L;
    MNB_TRY(check_desc(w, &L));
    MNB_TRY(check_ptr(repacked, 256, "repacked"));
    if (L.N == 0 || (!codes && !w_f32)) return ok("unpack_debug");
    if (w_f32) MNB_TRY(check_ptr(w_f32, 4, "w_f32"));
    MNB_TRY(check_device());
    return launched(mnb::launch_unpack_debug(L, repacked, codes, w_f32,
                                             static_cast<hipStream_t>(stream)),
                    "unpack_debug");
}

int32_t mnb_debug_prefill_rows(int32_t rows) { return mnb::set_prefill_rows(rows); }

// Any value is accepted (an int at the boundary, not the enum type): unknown
// ones give MNB_ERR_UNKNOWN.
const char* mnb_status_string(int32_t status)
{
    switch (status) {
    case MNB_OK: return "MNB_OK";
    case MNB_ERR_INVALID_ARGUMENT: return "MNB_ERR_INVALID_ARGUMENT";
    case MNB_ERR_UNSUPPORTED: return "MNB_ERR_UNSUPPORTED";
    case MNB_ERR_DEVICE: return "MNB_ERR_DEVICE";
    }
    return "MNB_ERR_UNKNOWN";
}

const char* mnb_last_error(void) { return g_error.c_str(); }

const char* mnb_last_variant(void) { return g_variant; }

}  // extern "C"
