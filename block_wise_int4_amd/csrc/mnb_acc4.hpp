// mnb_acc4.hpp -- host-side declarations of the int8-activation kernels
// (accuracy_level 4): fp32 activations, fp32 outputs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mnb_internal.hpp"
#include "mnb_layout.hpp"

namespace mnb {

// Largest K the M=1 kernel holds as int8 records in LDS.
int64_t acc4_gemv_max_k();

// M = 1: quantizes a [K] in every workgroup and computes y [N]; bias [N] or
// NULL.  q_out [K] (the codes as fp16 integers, k order) and s_out [1] may be
// NULL; otherwise the first workgroup writes the row's codes and scale there.
hipError_t launch_acc4_gemv(const Layout& L, const WeightView& w, const float* a, const float* bias,
                            float* y, _Float16* q_out, float* s_out, hipStream_t stream,
                            const char** variant);

// Rows of a [M, K] (K a multiple of 16, a 16-byte aligned) to their codes,
// written as fp16 integers q [M, K], and scales s [M].
hipError_t launch_acc4_quantize(const float* a, int64_t M, int64_t K, _Float16* q, float* s,
                                hipStream_t stream);

// The fp16 GEMMs on such codes (exact integers, so every group dot is exact
// in their fp32 accumulators) with an fp32 output: y[m, n] = row_scale[m] *
// acc[m, n] (+ bias[n]); a16 [M, K] fp16.  With pair_rows, a16 holds 2M rows
// (m counts them), the (hi, lo) parts of fp32 activations from
// launch_split_f32_rows, and y[r, n] = row_scale[r] * (acc[2r, n] + acc[2r +
// 1, n]) (+ bias[r * bias_stride + n]).
hipError_t launch_gemm_small_f32(const Layout& L, const WeightView& w, const void* a16, int64_t m,
                                 const float* row_scale, const float* bias, float* y, void* ws,
                                 hipStream_t stream, const char** variant, int pair_rows = 0,
                                 int64_t bias_stride = 0);
hipError_t launch_gemm_mfma_f32(const Layout& L, const WeightView& w, const void* a16, int64_t m,
                                const float* row_scale, const float* bias, float* y, hipStream_t stream,
                                const char** variant, int pair_rows = 0, int64_t bias_stride = 0);

// fp32 activations a [M, K] (K a multiple of 16, 16-byte aligned) as fp16 row
// pairs hl [2M, K] (row 2m = hi, 2m + 1 = lo of row m, scaled by 2^-e_m) and
// row_scale [M] = 2^e_m.
hipError_t launch_split_f32_rows(const float* a, int64_t M, int64_t K, _Float16* hl, float* row_scale,
                                 hipStream_t stream);

}  // namespace mnb
