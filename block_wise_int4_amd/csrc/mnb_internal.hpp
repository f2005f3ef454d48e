// mnb_internal.hpp -- kernel launchers behind the C ABI (library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mnb_layout.hpp"

namespace mnb {

// Pointers to the three sections of one repacked weight.
struct WeightView {
    const uint8_t* codes;
    const void* scales;
    const uint8_t* zp;  // nullptr without zero points
};

inline WeightView view_of(const Layout& L, const void* repacked)
{
    const uint8_t* b = static_cast<const uint8_t*>(repacked);
    return WeightView{b + L.codes_off, b + L.scales_off, L.has_zp ? b + L.zp_off : nullptr};
}

// perm: NULL, or the act-order permutation of k (the codes of ONNX position
// perm[k] go to position k; scales and zero points keep their groups).
hipError_t launch_repack(const Layout& L, const uint8_t* packed, const void* scales,
                         const uint8_t* zp, const int32_t* perm, void* repacked, hipStream_t stream);
// out[m, k] = a[m, perm[k]] for an [M, K] matrix of elem_bytes (2 or 4)
// elements; K a multiple of 16, out 16-byte aligned; an index outside
// 0..K-1 reads column 0.
hipError_t launch_permute_columns(const void* a, const int32_t* perm, int64_t M, int64_t K,
                                  int elem_bytes, void* out, hipStream_t stream);
hipError_t launch_unpack_debug(const Layout& L, const void* repacked, uint8_t* codes, float* w,
                               hipStream_t stream);

// Largest K the decode GEMV stages in LDS, per activation dtype; act order
// stages a second, gathered copy.
int64_t gemv_max_k(bool f16_act, bool act_order = false);
// Optional bias of the output, element (m, n) at ptr[m * row_stride + n], in
// the output's dtype; after_round selects fp16(fp16(acc) + b) over
// fp16(acc + b).
struct Bias {
    const void* ptr = nullptr;
    int64_t row_stride = 0;
    int after_round = 0;
};

// y = a . dequant(B)^T (up == nullptr) or silu(a . Bg^T) * (a . Bu^T).
// perm (act order, up == nullptr only): NULL, or device int32 [K], 16-byte
// aligned, K a multiple of 4: the product takes a[perm[k]] at column k.
hipError_t launch_gemv(const Layout& L, const WeightView& gate, const WeightView* up,
                       const void* a, const int32_t* perm, bool f16_act, const Bias& bias, void* y,
                       hipStream_t stream, const char** variant);

// 2 <= M <= 16, fp16 activations, K up to gemm_small_max_k().
int64_t gemm_small_max_k();
size_t gemm_small_workspace(const Layout& L, int64_t m);
hipError_t launch_gemm_small(const Layout& L, const WeightView& w, const void* a, int64_t m,
                             const Bias& bias, void* y, void* ws, hipStream_t stream, const char** variant);

// M > 16, fp16 activations, K up to gemm_mfma_max_k().
int64_t gemm_mfma_max_k();
// Tile height of the prefill GEMM where the group size offers several: 64,
// 96 or 128 for every later call, 0 to choose per call; returns the
// previous value (-1: invalid).
int set_prefill_rows(int rows);
hipError_t launch_gemm_mfma(const Layout& L, const WeightView& w, const void* a, int64_t m,
                            const Bias& bias, void* y, hipStream_t stream, const char** variant);

// Device address of the no-allocation scratch array on device `dev` (which
// must be current), MNB_NOALLOC_SCRATCH_BYTES bytes; looked up on the first
// call per device, then cached.
hipError_t noalloc_scratch(int dev, void** out);

}  // namespace mnb
