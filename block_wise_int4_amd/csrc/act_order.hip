// act_order.hip -- the activation side of act-order weights.
//
// Method: onnx-runtime-ep-cuda 0.1.0-dev.3, src/kernels/matmul_nbits.rs --
// the optional group-index input g_idx (int32 [K], every value a group of
// the weight) and the dequant kernel that looks up the scale and zero point
// of group g_idx[k] for the code at k.  Here the repack sorts k by group
// (mnb_repack_act_order), so the weight looks like an ordinary one with
// contiguous groups; the product is unchanged when A's columns take the
// same order, Y = A[:, perm] . dequant(B)[:, perm]^T, which this kernel
// provides before the ordinary GEMV or GEMM runs.
#include "mnb_device.hpp"
#include "mnb_internal.hpp"

namespace mnb {

namespace {

// One thread per 16 output bytes (8 fp16 or 4 fp32 columns of a row, one
// vector store; the reads gather within the row, which the caches hold).
// K is a multiple of 16 (the group size), so a vector never straddles rows.
template <typename T>
__global__ __launch_bounds__(256) void permute_columns_kernel(const T* __restrict__ a,
                                                              const int32_t* __restrict__ perm,
                                                              T* __restrict__ out, int64_t M,
                                                              int64_t K)
{
    constexpr int V = 16 / sizeof(T);
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= M * K / V) return;
    const int64_t e0 = idx * V;
    const int64_t m = e0 / K;
    const int64_t k0 = e0 - m * K;
    const T* row = a + m * K;
    T v[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        int64_t src = perm[k0 + i];
        if (src < 0 || src >= K) src = 0;
        v[i] = row[src];
    }
    u4_t o;
    __builtin_memcpy(&o, v, 16);
    reinterpret_cast<u4_t*>(out)[idx] = o;
}

// One workgroup per row: the row is staged in LDS with coalesced 16-byte
// loads while the thread's index vectors are requested, then gathered from
// LDS and written 16 bytes per thread.  For rows that fit in the LDS a
// workgroup gets (K * element size <= kMaxRowBytes).
constexpr int kRowThreads = 256;
constexpr int64_t kMaxRowBytes = 64 * 1024;

template <typename T>
__global__ __launch_bounds__(kRowThreads) void permute_row_kernel(const T* __restrict__ a,
                                                                  const int32_t* __restrict__ perm,
                                                                  T* __restrict__ out, int64_t K)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int V = 16 / sizeof(T);
    const int64_t m = blockIdx.x;
    const int nvec = (int)(K / V);
    const u4_t* src = reinterpret_cast<const u4_t*>(a + m * K);
    for (int v = threadIdx.x; v < nvec; v += kRowThreads) reinterpret_cast<u4_t*>(smem)[v] = src[v];
    __syncthreads();
    const T* row = reinterpret_cast<const T*>(smem);
    u4_t* dst = reinterpret_cast<u4_t*>(out + m * K);
    for (int v = threadIdx.x; v < nvec; v += kRowThreads) {
        T o[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const uint32_t k = (uint32_t)perm[(int64_t)v * V + i];
            o[i] = row[k < (uint32_t)K ? k : 0u];
        }
        u4_t ov;
        __builtin_memcpy(&ov, o, 16);
        dst[v] = ov;
    }
}

}  // namespace

hipError_t launch_permute_columns(const void* a, const int32_t* perm, int64_t M, int64_t K,
                                  int elem_bytes, void* out, hipStream_t stream)
{
    if (K * elem_bytes <= kMaxRowBytes) {
        const size_t lds = (size_t)(K * elem_bytes);
        if (elem_bytes == 2)
            permute_row_kernel<uint16_t><<<dim3((unsigned)M), kRowThreads, lds, stream>>>(
                static_cast<const uint16_t*>(a), perm, static_cast<uint16_t*>(out), K);
        else
            permute_row_kernel<uint32_t><<<dim3((unsigned)M), kRowThreads, lds, stream>>>(
                static_cast<const uint32_t*>(a), perm, static_cast<uint32_t*>(out), K);
        return hipGetLastError();
    }
    const int64_t total = M * K / (16 / elem_bytes);
    const unsigned blocks = (unsigned)((total + 255) / 256);
    if (elem_bytes == 2)
        permute_columns_kernel<uint16_t><<<blocks, 256, 0, stream>>>(
            static_cast<const uint16_t*>(a), perm, static_cast<uint16_t*>(out), M, K);
    else
        permute_columns_kernel<uint32_t><<<blocks, 256, 0, stream>>>(
            static_cast<const uint32_t*>(a), perm, static_cast<uint32_t*>(out), M, K);
    return hipGetLastError();
}

}  // namespace mnb
