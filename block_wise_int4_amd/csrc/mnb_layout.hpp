// mnb_layout.hpp -- geometry of the repacked weight buffer (host and device).
//
// The layout itself is specified in include/mnb.h ("Repacked layout"); this
// header is its single implementation inside the library.  The input format
// it re-indexes is the ONNX MatMulNBits int4 storage described in the module
// doc of onnx-runtime-ep-cuda 0.1.0-dev.6, src/kernels/marlin_gemm.rs,
// section "ONNX MatMulNBits int4 format (input to the repack)".
#pragma once

#include <stdint.h>

#ifndef MNB_HD
#if defined(__HIPCC__)
#define MNB_HD __host__ __device__ inline
#else
#define MNB_HD inline
#endif
#endif

namespace mnb {

constexpr int kTileN = 16;        // columns per tile (MFMA 16x16x32 B-operand width)
constexpr int kChunkK = 128;      // k per chunk (4 MFMA k-steps of 32)
constexpr int kChunkBytes = 1024; // 16 columns x 128 k x 4 bits
constexpr int kAlign = 256;

MNB_HD int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct Layout {
    int64_t N, K;
    int g;          // group size
    int Q;          // groups per chunk = 128 / g
    int ss;         // bytes per scale (2 or 4)
    bool has_zp;
    int64_t T, C;   // tiles, chunks
    int64_t kb;     // groups along K = K / g
    int64_t codes_off, codes_bytes;
    int64_t scales_off, scales_bytes;
    int64_t zp_off, zp_bytes;
    int64_t flags_off, flags_bytes;   // one byte per tile: its scales' range class
    int64_t total;
};

MNB_HD Layout make_layout(int64_t N, int64_t K, int g, bool has_zp, bool f16_scales)
{
    Layout L;
    L.N = N;
    L.K = K;
    L.g = g;
    L.Q = kChunkK / g;
    L.ss = f16_scales ? 2 : 4;
    L.has_zp = has_zp;
    L.T = (N + kTileN - 1) / kTileN;
    L.C = (K + kChunkK - 1) / kChunkK;
    L.kb = K / g;
    L.codes_off = 0;
    L.codes_bytes = L.T * L.C * kChunkBytes;
    L.scales_off = align_up(L.codes_off + L.codes_bytes, kAlign);
    L.scales_bytes = L.T * L.C * kTileN * L.Q * L.ss;
    int64_t end = L.scales_off + L.scales_bytes;
    if (has_zp) {
        L.zp_off = align_up(end, kAlign);
        L.zp_bytes = L.T * L.C * (kTileN / 2) * L.Q;
        end = L.zp_off + L.zp_bytes;
    } else {
        L.zp_off = 0;
        L.zp_bytes = 0;
    }
    L.flags_off = align_up(end, kAlign);
    L.flags_bytes = L.T;
    L.total = align_up(L.flags_off + L.flags_bytes, kAlign);
    return L;
}

// Range class of a tile's scales (the byte of the tile in the flags
// section): 1 when every scale of its columns that is neither zero nor NaN
// has magnitude in [2^-100, 2^100] and, per column, the largest such magnitude
// is at most 2^64 times the smallest; 0 otherwise (an infinite, subnormal,
// tiny or huge scale, or a wider spread).  Finite fp16 scales are always in
// class 1.
constexpr float kScaleLo = 0x1p-100f, kScaleHi = 0x1p100f, kScaleSpread = 0x1p64f;

// Slot of (column i in tile, group q in chunk) inside a chunk's 16*Q scale /
// zero-point record.  For Q <= 4 the groups of one column are adjacent; for
// Q = 8 (group 16) the record is split by group parity so that the four
// groups a lane needs for its four 32-k words are adjacent too.
MNB_HD int slot_of(int i, int q, int Q)
{
    return Q <= 4 ? i * Q + q : ((q & 1) * 16 + i) * 4 + (q >> 1);
}

// Position of k-offset i (0..7) of a word: nibble slot p(i).
MNB_HD int nibble_slot(int i) { return (i >> 1) + ((i & 1) << 2); }

}  // namespace mnb
