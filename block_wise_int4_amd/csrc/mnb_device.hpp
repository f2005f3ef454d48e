// mnb_device.hpp -- device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "mnb_layout.hpp"

namespace mnb {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2_t as_h2(uint32_t x) { return __builtin_bit_cast(h2_t, x); }
__device__ __forceinline__ uint32_t as_u32(h2_t x) { return __builtin_bit_cast(uint32_t, x); }

// Per-group constants of the magic-number unpack, as packed fp16 pairs.
//   neg1024z = -(1024 + z): OR-ing a nibble c into the mantissa of fp16
//              1024.0 (0x6400) gives exactly 1024 + c; adding this gives c - z.
//   neg64z   = -(64 + z):   a nibble OR-ed one position higher (bits 4..7)
//              gives 1024 + 16c; times 1/16 plus this gives c - z.
// Both results are small integers, so every step is exact in fp16.  This is
// the integer-to-half trick of the fp16 GEMVs of onnx-runtime-ep-cuda
// 0.1.0-dev.3, src/kernels/matmul_nbits.rs, re-derived from the binary16
// format, with the zero point folded into the subtracted constant.
struct ZpConst {
    uint32_t neg1024z;
    uint32_t neg64z;
};

__device__ __forceinline__ ZpConst zp_const(uint32_t z)
{
    // z <= 15, so each half is formed without carries: one 24-bit mad each
    return ZpConst{z * 0x00010001u + 0xE400E400u,    // -(1024 + z) in both halves
                   z * 0x00100010u + 0xD400D400u};   // -(64 + z) in both halves
}

// Unpack one repacked word (8 nibbles, slots holding k-offsets
// 0,2,4,6,1,3,5,7) into (c - z) as 4 fp16 pairs in k order:
// (k0,k1), (k2,k3), (k4,k5), (k6,k7).
__device__ __forceinline__ void unpack8(uint32_t d, ZpConst zc, h2_t out[4])
{
    // (x & mask) | 0x64006400 in one v_bitop3_b32 (truth table 0xEA)
    const uint32_t lo = 0x000F000Fu, hi = 0x00F000F0u, magic = 0x64006400u;
    const h2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const uint32_t d8 = d >> 8;
    out[0] = as_h2(__builtin_amdgcn_bitop3_b32(d, lo, magic, 0xEA)) + as_h2(zc.neg1024z);
    out[1] = as_h2(__builtin_amdgcn_bitop3_b32(d, hi, magic, 0xEA)) * sixteenth + as_h2(zc.neg64z);
    out[2] = as_h2(__builtin_amdgcn_bitop3_b32(d8, lo, magic, 0xEA)) + as_h2(zc.neg1024z);
    out[3] = as_h2(__builtin_amdgcn_bitop3_b32(d8, hi, magic, 0xEA)) * sixteenth + as_h2(zc.neg64z);
}

// Both constants of zero point z for unpack_zr in one register: the low half
// is -(1024 + z), the high half -(64 + z) (fp16 64 + z carries z in mantissa
// bits 4..7).  z <= 15, so the halves form without carries: one 24-bit mad.
__device__ __forceinline__ uint32_t zp_pair(uint32_t z) { return __umul24(z, 0x100001u) + 0xD400E400u; }

// unpack8 with both constants of the zero point in one register (zp_pair):
// each packed add or fma takes its constant from one half of zr for both of
// its lanes (an op_sel broadcast), so a group costs one instruction for its
// constants instead of two.
__device__ __forceinline__ void unpack_zr(uint32_t d, uint32_t zr, h2_t out[4])
{
    const uint32_t lo = 0x000F000Fu, hi = 0x00F000F0u, magic = 0x64006400u;
    const h2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2_t r = as_h2(zr);
    const h2_t c_lo = {r[0], r[0]}, c_hi = {r[1], r[1]};
    const uint32_t d8 = d >> 8;
    out[0] = as_h2(__builtin_amdgcn_bitop3_b32(d, lo, magic, 0xEA)) + c_lo;
    out[1] = as_h2(__builtin_amdgcn_bitop3_b32(d, hi, magic, 0xEA)) * sixteenth + c_hi;
    out[2] = as_h2(__builtin_amdgcn_bitop3_b32(d8, lo, magic, 0xEA)) + c_lo;
    out[3] = as_h2(__builtin_amdgcn_bitop3_b32(d8, hi, magic, 0xEA)) * sixteenth + c_hi;
}

// The code of k-offset i (0..7) of a repacked word.
__device__ __forceinline__ uint32_t code_at(uint32_t d, int i)
{
    return (d >> (4 * nibble_slot(i))) & 15u;
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__half x) { return __half2float(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __half from_f32<__half>(float x) { return __float2half_rn(x); }

// One output through the bias epilogue (matmul_nbits.rs, fold_bias_f16):
// no bias: round once; a bias b: fp16(acc + b), or, after_round, fp16(fp16(acc)
// + b); fp32 outputs add once in either mode.
__device__ __forceinline__ __half finish_value(float acc, float b, int after_round)
{
    if (after_round) acc = __half2float(__float2half_rn(acc));
    return __float2half_rn(acc + b);
}
__device__ __forceinline__ __half finish_output(float acc, const __half* bias, int64_t i, int after_round)
{
    if (!bias) return __float2half_rn(acc);
    return finish_value(acc, __half2float(bias[i]), after_round);
}
__device__ __forceinline__ float finish_output(float acc, const float* bias, int64_t i, int)
{
    return bias ? acc + bias[i] : acc;
}

// A wave-uniform value the compiler can keep in scalar registers.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Workgroup barrier that orders LDS traffic only: outstanding global loads
// stay in flight across it.
__device__ __forceinline__ void block_sync_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace mnb
