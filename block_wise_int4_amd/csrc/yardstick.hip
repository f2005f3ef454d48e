// yardstick.hip -- a plain streaming read, the measuring rod of bench.py (not
// part of the matmul library or its C ABI; built into its own
// libmnb_yardstick.so).
//
// It reads `bytes` (a multiple of 16) from a device buffer with 16-byte
// nontemporal loads, four per thread in flight, and keeps the data alive by
// an XOR that is stored only if it equals a value it practically never has,
// so the kernel's time is the time to stream those bytes from memory: the
// floor for a kernel that must read as much.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(1024) void stream_read_kernel(const u4_t* __restrict__ src, uint32_t* __restrict__ sink,
                                                           int64_t n16, int64_t per_block)
{
    const int64_t base = (int64_t)blockIdx.x * per_block;
    uint32_t acc = 0;
    for (int64_t i = threadIdx.x; i < per_block; i += (int64_t)blockDim.x * 4) {
        u4_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t j = i + (int64_t)u * blockDim.x;
            v[u] = (j < per_block && base + j < n16) ? __builtin_nontemporal_load(src + base + j)
                                                     : u4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Read bytes (multiple of 16, src 16-byte aligned) with `blocks` workgroups
// of `threads` (<= 1024) threads on `stream`; sink (device) holds at least
// `blocks` uint32 values.  Returns a hipError_t.
int mnb_yardstick_read(const void* src, int64_t bytes, void* sink, int32_t blocks, int32_t threads, void* stream)
{
    if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || blocks <= 0 || threads <= 0 || threads > 1024)
        return (int)hipErrorInvalidValue;
    const int64_t n16 = bytes / 16;
    const int64_t per_block = (n16 + blocks - 1) / blocks;
    stream_read_kernel<<<dim3((unsigned)blocks), dim3((unsigned)threads), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u4_t*>(src), static_cast<uint32_t*>(sink), n16, per_block);
    return (int)hipGetLastError();
}

}  // extern "C"
