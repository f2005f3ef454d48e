// repack.hip -- offline repack of ONNX MatMulNBits int4 operands into the
// gfx950 layout of include/mnb.h, and the test-only decoder of that layout.
//
// The input indexing is the module doc of onnx-runtime-ep-cuda 0.1.0-dev.6,
// src/kernels/marlin_gemm.rs, section "ONNX MatMulNBits int4 format (input to
// the repack)"; the idea of a one-time, size-preserving reordering of the
// nibbles into the matrix-core operand distribution is that page's section
// "Repacked weight layout".  The distribution targeted here is the gfx950
// v_mfma_f32_16x16x32_f16 B operand (16 columns x 4 k-octets per 64 lanes).
#include "mnb_device.hpp"
#include "mnb_internal.hpp"

namespace mnb {

namespace {

// Gather the 8 nibbles k0..k0+7 of column n (four ONNX bytes, one aligned
// 32-bit load: 8 consecutive k of one group are 4 consecutive bytes) and
// move even k to nibble slots 0..3, odd k to slots 4..7.
__device__ __forceinline__ uint32_t compact_nibbles(uint32_t e)
{
    const uint32_t t = e | (e >> 4);
    return (t & 0xFFu) | ((t >> 8) & 0xFF00u);
}

__global__ __launch_bounds__(256) void repack_codes_kernel(const uint8_t* __restrict__ packed,
                                                           uint32_t* __restrict__ out, int64_t N,
                                                           int64_t K, int g, int64_t C,
                                                           int64_t words)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= words) return;
    const int64_t chunk = idx >> 8;
    const int within = (int)(idx & 255);
    const int lane = within >> 2;
    const int j = within & 3;
    const int64_t t = chunk / C;
    const int64_t c = chunk - t * C;
    const int64_t n = t * kTileN + (lane & 15);
    const int64_t k0 = c * kChunkK + 32 * j + 8 * (lane >> 4);
    uint32_t v = 0;
    if (n < N && k0 < K) {
        const int64_t kb = K / g;
        const int64_t byte = (n * kb + k0 / g) * (g / 2) + (k0 % g) / 2;
        const uint32_t x = *reinterpret_cast<const uint32_t*>(packed + byte);
        v = compact_nibbles(x & 0x0F0F0F0Fu) | (compact_nibbles((x >> 4) & 0x0F0F0F0Fu) << 16);
    }
    out[idx] = v;
}

// The same words for an act-order weight: position k of the repacked order
// holds the code of ONNX position perm[k] (perm sorts k by group, so every
// group of the repacked order is contiguous).  An index outside 0..K-1 reads
// position 0: a wrong permutation gives wrong codes, never a wild read.
__global__ __launch_bounds__(256) void repack_codes_perm_kernel(const uint8_t* __restrict__ packed,
                                                                const int32_t* __restrict__ perm,
                                                                uint32_t* __restrict__ out, int64_t N,
                                                                int64_t K, int g, int64_t C,
                                                                int64_t words)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= words) return;
    const int64_t chunk = idx >> 8;
    const int within = (int)(idx & 255);
    const int lane = within >> 2;
    const int j = within & 3;
    const int64_t t = chunk / C;
    const int64_t c = chunk - t * C;
    const int64_t n = t * kTileN + (lane & 15);
    const int64_t k0 = c * kChunkK + 32 * j + 8 * (lane >> 4);
    uint32_t v = 0;
    if (n < N) {
        const int64_t kb = K / g;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (k0 + i >= K) break;
            int64_t ks = perm[k0 + i];
            if (ks < 0 || ks >= K) ks = 0;
            const uint32_t byte = packed[(n * kb + ks / g) * (g / 2) + (ks % g) / 2];
            const uint32_t nib = (ks & 1) ? (byte >> 4) : (byte & 15u);
            // even offsets to nibble slots 0..3, odd ones to 4..7
            const int slot = (i & 1) ? 4 + (i >> 1) : (i >> 1);
            v |= nib << (4 * slot);
        }
    }
    out[idx] = v;
}

// (column i, in-chunk group q) of a slot; inverse of slot_of().
__device__ __forceinline__ void slot_inverse(int s, int Q, int& i, int& q)
{
    if (Q <= 4) {
        i = s / Q;
        q = s - i * Q;
    } else {
        const int r = s >> 2;
        i = r & 15;
        q = 2 * (s & 3) + (r >> 4);
    }
}

template <typename S>
__global__ __launch_bounds__(256) void repack_scales_kernel(const S* __restrict__ scales,
                                                            S* __restrict__ out, int64_t N,
                                                            int64_t kb, int Q, int64_t C,
                                                            int64_t count)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= count) return;
    const int per_chunk = kTileN * Q;
    const int64_t chunk = idx / per_chunk;
    const int s = (int)(idx - chunk * per_chunk);
    const int64_t t = chunk / C;
    const int64_t c = chunk - t * C;
    int i, q;
    slot_inverse(s, Q, i, q);
    const int64_t n = t * kTileN + i;
    const int64_t G = c * Q + q;
    S v = S(0);
    if (n < N && G < kb) v = scales[n * kb + G];
    out[idx] = v;
}

__device__ __forceinline__ float scale_value(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ float scale_value(uint32_t b) { return __builtin_bit_cast(float, b); }

// The range class of each tile's scales (see kScaleLo in mnb_layout.hpp):
// one wave per tile; lane l takes column l % 16 and every fourth group from
// l / 16, then the four lanes of a column combine their extremes.
template <typename S>
__global__ __launch_bounds__(64) void scale_range_kernel(const S* __restrict__ scales,
                                                         uint8_t* __restrict__ flags, int64_t N,
                                                         int64_t kb)
{
    const int lane = threadIdx.x;
    const int64_t n = (int64_t)blockIdx.x * kTileN + (lane & 15);
    float lo = __builtin_inff(), hi = 0.0f;
    bool bad = false;
    if (n < N) {
        for (int64_t b = lane >> 4; b < kb; b += 4) {
            const float a = __builtin_fabsf(scale_value(scales[n * kb + b]));
            if (a == 0.0f || a != a) continue;   // zero or NaN: not part of the range
            bad = bad || !(a >= kScaleLo && a <= kScaleHi);
            lo = a < lo ? a : lo;
            hi = a > hi ? a : hi;
        }
    }
#pragma unroll
    for (int d = 16; d < 64; d *= 2) {
        const float lo2 = __shfl_xor(lo, d), hi2 = __shfl_xor(hi, d);
        lo = lo2 < lo ? lo2 : lo;
        hi = hi2 > hi ? hi2 : hi;
    }
    // a column with no range-bounded scale has lo = inf, hi = 0: fine
    bad = bad || (hi > lo * kScaleSpread);
    const bool any_bad = __any(bad);
    if (lane == 0) flags[blockIdx.x] = any_bad ? 0 : 1;
}

__global__ __launch_bounds__(256) void repack_zp_kernel(const uint8_t* __restrict__ zp,
                                                        uint8_t* __restrict__ out, int64_t N,
                                                        int64_t kb, int Q, int64_t C,
                                                        int64_t count)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= count) return;
    const int per_chunk = kTileN * Q / 2;
    const int64_t chunk = idx / per_chunk;
    const int b = (int)(idx - chunk * per_chunk);
    const int64_t t = chunk / C;
    const int64_t c = chunk - t * C;
    const int64_t zrb = (kb + 1) / 2;
    uint32_t v = 0;
    for (int h = 0; h < 2; ++h) {
        int i, q;
        slot_inverse(2 * b + h, Q, i, q);
        const int64_t n = t * kTileN + i;
        const int64_t G = c * Q + q;
        if (n < N && G < kb) {
            const uint32_t z = (zp[n * zrb + G / 2] >> (4 * (G & 1))) & 15u;
            v |= z << (4 * h);
        }
    }
    out[idx] = (uint8_t)v;
}

// Decode with the production unpack: codes via unpack8 with z = 0, weights via
// unpack8 with the stored zero point, times the scale in fp32.
template <typename S>
__global__ __launch_bounds__(256) void unpack_debug_kernel(const uint32_t* __restrict__ codes_r,
                                                           const S* __restrict__ scales_r,
                                                           const uint8_t* __restrict__ zp_r,
                                                           uint8_t* __restrict__ codes,
                                                           float* __restrict__ w, int64_t N,
                                                           int64_t K, int g, int64_t C,
                                                           int64_t words)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= words) return;
    const int Q = kChunkK / g;
    const int64_t chunk = idx >> 8;
    const int within = (int)(idx & 255);
    const int lane = within >> 2;
    const int j = within & 3;
    const int64_t t = chunk / C;
    const int64_t c = chunk - t * C;
    const int i = lane & 15;
    const int64_t n = t * kTileN + i;
    const int kin = 32 * j + 8 * (lane >> 4);
    const int64_t k0 = c * kChunkK + kin;
    if (n >= N || k0 >= K) return;
    const uint32_t d = codes_r[idx];
    const int q = kin / g;
    const int s = slot_of(i, q, Q);
    uint32_t z = 8;
    if (zp_r) z = (zp_r[chunk * (kTileN / 2) * Q + s / 2] >> (4 * (s & 1))) & 15u;
    const float scale = to_f32(scales_r[chunk * kTileN * Q + s]);
    h2_t cz[4], c0[4];
    unpack8(d, zp_const(z), cz);
    unpack8(d, zp_const(0), c0);
    for (int p = 0; p < 4; ++p) {
        for (int e = 0; e < 2; ++e) {
            const int64_t k = k0 + 2 * p + e;
            if (codes) codes[n * K + k] = (uint8_t)(float)c0[p][e];
            if (w) w[n * K + k] = (float)cz[p][e] * scale;
        }
    }
}

__global__ __launch_bounds__(256) void zero_fill_kernel(uint8_t* __restrict__ p, int64_t count)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx < count) p[idx] = 0;
}

inline unsigned blocks_for(int64_t count) { return (unsigned)((count + 255) / 256); }

// Zero the alignment padding between and after the sections.
void zero_gap(uint8_t* base, int64_t from, int64_t to, hipStream_t stream)
{
    if (to > from) zero_fill_kernel<<<blocks_for(to - from), 256, 0, stream>>>(base + from, to - from);
}

}  // namespace

hipError_t launch_repack(const Layout& L, const uint8_t* packed, const void* scales,
                         const uint8_t* zp, const int32_t* perm, void* repacked, hipStream_t stream)
{
    uint8_t* base = static_cast<uint8_t*>(repacked);
    const int64_t words = L.codes_bytes / 4;
    if (perm) {
        repack_codes_perm_kernel<<<blocks_for(words), 256, 0, stream>>>(
            packed, perm, reinterpret_cast<uint32_t*>(base + L.codes_off), L.N, L.K, L.g, L.C, words);
    } else {
        repack_codes_kernel<<<blocks_for(words), 256, 0, stream>>>(
            packed, reinterpret_cast<uint32_t*>(base + L.codes_off), L.N, L.K, L.g, L.C, words);
    }
    const int64_t ns = L.T * L.C * kTileN * L.Q;
    if (L.ss == 2) {
        repack_scales_kernel<uint16_t><<<blocks_for(ns), 256, 0, stream>>>(
            static_cast<const uint16_t*>(scales), reinterpret_cast<uint16_t*>(base + L.scales_off),
            L.N, L.kb, L.Q, L.C, ns);
    } else {
        repack_scales_kernel<uint32_t><<<blocks_for(ns), 256, 0, stream>>>(
            static_cast<const uint32_t*>(scales), reinterpret_cast<uint32_t*>(base + L.scales_off),
            L.N, L.kb, L.Q, L.C, ns);
    }
    if (L.has_zp) {
        repack_zp_kernel<<<blocks_for(L.zp_bytes), 256, 0, stream>>>(
            zp, base + L.zp_off, L.N, L.kb, L.Q, L.C, L.zp_bytes);
    }
    if (L.T > 0) {
        if (L.ss == 2)
            scale_range_kernel<uint16_t><<<(unsigned)L.T, 64, 0, stream>>>(static_cast<const uint16_t*>(scales),
                                                                        base + L.flags_off, L.N, L.kb);
        else
            scale_range_kernel<uint32_t><<<(unsigned)L.T, 64, 0, stream>>>(static_cast<const uint32_t*>(scales),
                                                                        base + L.flags_off, L.N, L.kb);
    }
    zero_gap(base, L.codes_off + L.codes_bytes, L.scales_off, stream);
    const int64_t scales_end = L.scales_off + L.scales_bytes;
    const int64_t meta_end = L.has_zp ? L.zp_off + L.zp_bytes : scales_end;
    if (L.has_zp) zero_gap(base, scales_end, L.zp_off, stream);
    zero_gap(base, meta_end, L.flags_off, stream);
    zero_gap(base, L.flags_off + L.flags_bytes, L.total, stream);
    return hipGetLastError();
}

hipError_t launch_unpack_debug(const Layout& L, const void* repacked, uint8_t* codes, float* w,
                               hipStream_t stream)
{
    const uint8_t* base = static_cast<const uint8_t*>(repacked);
    const int64_t words = L.codes_bytes / 4;
    const uint32_t* cr = reinterpret_cast<const uint32_t*>(base + L.codes_off);
    const uint8_t* zr = L.has_zp ? base + L.zp_off : nullptr;
    if (L.ss == 2) {
        unpack_debug_kernel<__half><<<blocks_for(words), 256, 0, stream>>>(
            cr, reinterpret_cast<const __half*>(base + L.scales_off), zr, codes, w, L.N, L.K, L.g,
            L.C, words);
    } else {
        unpack_debug_kernel<float><<<blocks_for(words), 256, 0, stream>>>(
            cr, reinterpret_cast<const float*>(base + L.scales_off), zr, codes, w, L.N, L.K, L.g,
            L.C, words);
    }
    return hipGetLastError();
}

}  // namespace mnb
