// f32_split.hip -- fp32 activation rows as pairs of fp16 rows, so that the
// fp16 GEMMs (matrix cores) serve fp32 activations with M > 1.
//
// The fp32 operator of onnx-runtime-ep-cuda 0.1.0-dev.3,
// src/kernels/matmul_nbits.rs (MatMulNBitsKernel::run) serves fp32
// activations at any M.  Here each row m of A is scaled by a power of two,
// 2^-e_m, chosen so that its largest finite magnitude lands in [2^14, 2^15),
// then written as hi = fp16(a * 2^-e_m) (row 2m) and lo = fp16(a * 2^-e_m -
// hi) (row 2m + 1).  The GEMM adds the two rows' products and multiplies by
// 2^e_m, exactly.  Per element, |a - (hi + lo) * 2^e_m| <= 2^-22 |a| +
// 2^(e_m - 25), and 2^e_m <= 2^-14 max|a|: far inside the matmul tolerance.
// Non-finite values go to hi whole (lo 0), so NaN and infinities propagate
// as they do for fp32 products.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "mnb_internal.hpp"

namespace mnb {

namespace {

constexpr int kSplitThreads = 256;

typedef float f4v __attribute__((ext_vector_type(4)));
typedef _Float16 h4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float finite_abs(float x)
{
    const float a = __builtin_fabsf(x);
    return a <= 3.40282347e38f ? a : 0.0f;   // NaN and infinities compare false
}

__global__ __launch_bounds__(kSplitThreads) void split_rows_kernel(const float* __restrict__ a,
                                                                   _Float16* __restrict__ hl,
                                                                   float* __restrict__ row_scale, int64_t K)
{
    __shared__ float wmax[kSplitThreads / 64];
    const int64_t m = blockIdx.x;
    const f4v* row = reinterpret_cast<const f4v*>(a + m * K);
    const int64_t nv = K / 4;
    const int tid = threadIdx.x;

    // largest finite magnitude of the row
    float mx = 0.0f;
    for (int64_t v = tid; v < nv; v += kSplitThreads) {
        const f4v x = row[v];
        mx = fmaxf(fmaxf(mx, finite_abs(x.x)), fmaxf(finite_abs(x.y), fmaxf(finite_abs(x.z), finite_abs(x.w))));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if ((tid & 63) == 0) wmax[tid >> 6] = mx;
    __syncthreads();
    mx = 0.0f;
#pragma unroll
    for (int w = 0; w < kSplitThreads / 64; ++w) mx = fmaxf(mx, wmax[w]);

    // mx * 2^-e in [2^14, 2^15); e >= -149 keeps 2^e a binary32 value
    int e = mx > 0.0f ? ilogbf(mx) - 14 : 0;
    e = e < -149 ? -149 : e;
    h4v* hi = reinterpret_cast<h4v*>(hl + 2 * m * K);
    h4v* lo = reinterpret_cast<h4v*>(hl + (2 * m + 1) * K);
    for (int64_t v = tid; v < nv; v += kSplitThreads) {
        const f4v x = row[v];
        h4v h, l;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float s = ldexpf(x[i], -e);                 // exact: a power-of-two scaling
            const _Float16 hh = (_Float16)s;                  // round to nearest even
            const float hf = (float)hh;
            h[i] = hh;
            l[i] = (hf - hf == 0.0f) ? (_Float16)(s - hf) : (_Float16)0.0f;   // s - hf is exact
        }
        hi[v] = h;
        lo[v] = l;
    }
    if (tid == 0) row_scale[m] = ldexpf(1.0f, e);
}

}  // namespace

hipError_t launch_split_f32_rows(const float* a, int64_t M, int64_t K, _Float16* hl, float* row_scale,
                                 hipStream_t stream)
{
    split_rows_kernel<<<dim3((unsigned)M), dim3(kSplitThreads), 0, stream>>>(a, hl, row_scale, K);
    return hipGetLastError();
}

}  // namespace mnb
