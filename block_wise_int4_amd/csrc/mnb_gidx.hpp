// mnb_gidx.hpp -- launcher of the group-index route (library-internal).
#pragma once

#include "mnb_internal.hpp"

namespace mnb {

// Any group-index input: y[m, n] = sum_k a[m, k] (code[n, k] - zp[n, G]) scale[n, G]
// with G = g_idx[k] (a k whose G is outside 0..kb-1 adds nothing), from a plain
// repack; 1 <= M <= gidx_max_m(), a and g_idx 16-byte aligned, fp32 sums.
int64_t gidx_max_m();
hipError_t launch_gemm_gidx(const Layout& L, const WeightView& w, const void* a, int64_t m, bool f16_act,
                            const int32_t* g_idx, const Bias& bias, void* y, hipStream_t stream,
                            const char** variant);

}  // namespace mnb
