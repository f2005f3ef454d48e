// gidx.hip -- the product for any group-index input g_idx (act order whose
// groups need not hold group_size members each).
//
// Method: onnx-runtime-ep-cuda 0.1.0-dev.3, src/kernels/matmul_nbits.rs, the
// general route of the fp32 operator with group_indices: the dequant kernel
// gives the code at k (kept at its ONNX position) the scale and zero point of
// group g_idx[k], and a weight of 0 where that group is out of range; a dense
// GEMM follows.  So
//   y[m, n] = sum_k a[m, k] * (code[n, k] - zp[n, G]) * scale[n, G],  G = g_idx[k].
// The sorted route (a repack in group order, then the ordinary kernels) needs
// every group to hold exactly group_size positions; these kernels serve any
// g_idx from a plainly repacked weight, looking the scale and zero point up
// per k.  Each weight is formed in fp32, (c - z) * s (exact for fp16 scales,
// one rounding for fp32 ones), and the products are summed in fp32, as the
// dequant-then-GEMM route does; nothing goes through a dense weight in memory.
//
// gfx950 design, two kernels:
//  * M <= 16 (weight streaming): a workgroup of 16 waves owns one 16-column
//    tile; each wave takes every 16th 128-k chunk, one lane per 16-byte lane
//    record (one column, 32 k), dequantizes its 32 weights in registers and
//    multiplies them into up to 16 rows of A read straight from L2.  No
//    barrier inside the loop; the 4 lanes of a column and then the 16 waves
//    are summed in a fixed order at the end.
//  * M > 16 (a dense contraction): a workgroup of 4 waves owns 64 rows x 64
//    columns (4 tiles); per chunk it stages A (fp32, row-major) and the
//    dequantized weights (fp32, k-major) in LDS and runs
//    v_mfma_f32_16x16x4_f32, each wave 16 rows x 64 columns.
#include <type_traits>

#include "mnb_device.hpp"
#include "mnb_gidx.hpp"

namespace mnb {

namespace {

typedef float fx4_t __attribute__((ext_vector_type(4)));

constexpr int kSmallM = 16;     // largest M of the weight-streaming kernel
constexpr int kSmallWaves = 16;
constexpr int kBigRows = 64;    // rows of A per workgroup of the MFMA kernel
constexpr int kBigTiles = 4;    // 16-column tiles per workgroup of the MFMA kernel
constexpr int kAPad = 4;        // a_s row stride 132 floats: the A-fragment reads hit 64 banks
constexpr int kWPad = 16;       // w_s row stride 80 floats: the B-fragment reads hit 64 banks
// LDS for the tiles' scales and zero points (else they are read from L2):
// the streaming kernel's 1024 threads keep one workgroup per CU anyway; the
// matrix-core kernel's 74 KiB of staging leave this much of the 160 KiB.
constexpr int64_t kSmallMetaLds = 96 * 1024;
constexpr int64_t kBigMetaLds = 80 * 1024;

struct GidxParams {
    const uint4* codes;      // repacked codes section, one 16-byte lane record per element
    const void* scales;      // repacked scales section
    const uint8_t* zp;       // repacked zero-point section or null
    const int32_t* g_idx;    // [K], 16-byte aligned
    const void* a;           // [M, K], 16-byte aligned
    const void* bias;        // element (m, n) at bias[m * bias_stride + n], or null
    int64_t bias_stride;
    int after_round;
    void* y;                 // [M, N]
    int M, N, K, C, Q, qshift, kb;   // Q = 2^qshift groups per chunk
    int64_t T;
};

// The metadata of one tile: its C chunk records of scales (16Q each) and
// zero points (8Q bytes each), consecutive in the repacked sections.
template <typename ST>
struct TileMeta {
    const ST* scales;
    const uint8_t* zp;
};

template <typename ST>
__device__ __forceinline__ TileMeta<ST> global_meta(const GidxParams& p, int64_t t)
{
    const int64_t rec = t * p.C;
    return TileMeta<ST>{static_cast<const ST*>(p.scales) + rec * kTileN * p.Q,
                        p.zp ? p.zp + rec * (kTileN / 2) * p.Q : nullptr};
}

// Bytes of one tile's metadata in LDS: its scales, then its zero points at the
// next 16-byte boundary.
__host__ __device__ inline int64_t meta_scale_bytes(int64_t C, int Q, int ss) { return C * kTileN * Q * ss; }
__host__ __device__ inline int64_t meta_bytes(int64_t C, int Q, int ss, bool has_zp)
{
    return (meta_scale_bytes(C, Q, ss) + 15) / 16 * 16 + (has_zp ? (C * (kTileN / 2) * Q + 15) / 16 * 16 : 0);
}

// Copy tile t's metadata into LDS at dst (16-byte aligned) with the
// workgroup's threads (the caller synchronizes after): the scales in 16-byte
// pieces (each chunk record is a multiple of 32 bytes and the tile's first is
// 32-byte aligned), the zero points in 4-byte pieces (records of 8Q bytes).
template <typename ST, bool HAS_ZP>
__device__ __forceinline__ TileMeta<ST> stage_meta(const GidxParams& p, int64_t t, unsigned char* dst,
                                                   int tid, int nthreads)
{
    const TileMeta<ST> g = global_meta<ST>(p, t);
    const int64_t sb = meta_scale_bytes(p.C, p.Q, (int)sizeof(ST));
    const uint4* ss = reinterpret_cast<const uint4*>(g.scales);
    uint4* sd = reinterpret_cast<uint4*>(dst);
    for (int64_t v = tid; v < sb / 16; v += nthreads) sd[v] = ss[v];
    unsigned char* zd = dst + (sb + 15) / 16 * 16;
    if (HAS_ZP) {
        const int64_t zb = (int64_t)p.C * (kTileN / 2) * p.Q;
        const uint32_t* zs = reinterpret_cast<const uint32_t*>(g.zp);
        for (int64_t v = tid; v < zb / 4; v += nthreads) reinterpret_cast<uint32_t*>(zd)[v] = zs[v];
    }
    return TileMeta<ST>{reinterpret_cast<const ST*>(dst), HAS_ZP ? zd : nullptr};
}

// The weights of one 32-bit word of a lane record of tile t (metadata mt):
// column i = lane % 16, k = k0 + e for e = 0..7.  Each is (code - zp) * scale
// of group g_idx[k], or 0 where that group is out of range.  k0 < K, and K is
// a multiple of 16, so all 8 positions are inside.
template <typename ST, bool HAS_ZP>
__device__ __forceinline__ void dequant_word(const GidxParams& p, const TileMeta<ST>& mt, int i, uint32_t d,
                                             int k0, float w[8])
{
    const int4 g0 = *reinterpret_cast<const int4*>(p.g_idx + k0);
    const int4 g1 = *reinterpret_cast<const int4*>(p.g_idx + k0 + 4);
    const int gs[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int G = gs[e];
        float v = 0.0f;
        if (G >= 0 && G < p.kb) {
            const int cg = G >> p.qshift, q = G & (p.Q - 1);   // the group's chunk and its slot there
            const int s = slot_of(i, q, p.Q);
            const float sc = to_f32(mt.scales[cg * kTileN * p.Q + s]);
            uint32_t z = 8u;
            if (HAS_ZP) z = (mt.zp[cg * (kTileN / 2) * p.Q + (s >> 1)] >> (4 * (s & 1))) & 15u;
            v = ((float)code_at(d, e) - (float)z) * sc;
        }
        w[e] = v;
    }
}

// 8 consecutive activations of row m from k0 (16-byte aligned), as fp32.
template <typename AT>
__device__ __forceinline__ void load_a8(const GidxParams& p, int m, int k0, float x[8])
{
    const AT* row = static_cast<const AT*>(p.a) + (int64_t)m * p.K + k0;
    if constexpr (std::is_same<AT, float>::value) {
        const float4 u = *reinterpret_cast<const float4*>(row);
        const float4 v = *reinterpret_cast<const float4*>(row + 4);
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
        x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
    } else {
        const uint4 u = *reinterpret_cast<const uint4*>(row);
        const uint32_t ws[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const h2_t h = as_h2(ws[j]);
            x[2 * j] = (float)h[0];
            x[2 * j + 1] = (float)h[1];
        }
    }
}

// The output (m, n) from its fp32 sum: the bias epilogue of the other paths.
template <typename AT>
__device__ __forceinline__ void store_out(const GidxParams& p, int m, int64_t n, float acc)
{
    const int64_t o = (int64_t)m * p.N + n;
    if constexpr (std::is_same<AT, float>::value) {
        if (p.bias) acc += static_cast<const float*>(p.bias)[m * p.bias_stride + n];
        static_cast<float*>(p.y)[o] = acc;
    } else {
        static_cast<__half*>(p.y)[o] =
            p.bias ? finish_value(acc, __half2float(static_cast<const __half*>(p.bias)[m * p.bias_stride + n]),
                                  p.after_round)
                   : __float2half_rn(acc);
    }
}

template <typename AT, typename ST, bool HAS_ZP, bool LDS_META>
__global__ __launch_bounds__(kSmallWaves * 64) void gidx_small_kernel(GidxParams p)
{
    __shared__ float red[kSmallWaves][kSmallM][kTileN];
    extern __shared__ __attribute__((aligned(16))) unsigned char meta_s[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = lane & 15, h = lane >> 4;
    const int64_t t = blockIdx.x;
    TileMeta<ST> mt;
    if constexpr (LDS_META) {
        mt = stage_meta<ST, HAS_ZP>(p, t, meta_s, threadIdx.x, kSmallWaves * 64);
        __syncthreads();
    } else {
        mt = global_meta<ST>(p, t);
    }
    float acc[kSmallM];
#pragma unroll
    for (int m = 0; m < kSmallM; ++m) acc[m] = 0.0f;
    for (int c = wave; c < p.C; c += kSmallWaves) {
        const uint4 d4 = p.codes[(t * p.C + c) * 64 + lane];
        const uint32_t ds[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k0 = c * kChunkK + 32 * j + 8 * h;
            if (k0 < p.K) {   // the chunk's tail beyond K holds no weights
                float w[8];
                dequant_word<ST, HAS_ZP>(p, mt, i, ds[j], k0, w);
#pragma unroll
                for (int m = 0; m < kSmallM; ++m) {
                    if (m < p.M) {
                        float x[8];
                        load_a8<AT>(p, m, k0, x);
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[m] = __builtin_fmaf(x[e], w[e], acc[m]);
                    }
                }
            }
        }
    }
    // the 4 lanes of column i (h = 0..3), then the waves in order
#pragma unroll
    for (int m = 0; m < kSmallM; ++m) {
        float v = acc[m];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (h == 0) red[wave][m][i] = v;
    }
    __syncthreads();
    const int tid = threadIdx.x;
    if (tid < kSmallM * kTileN) {
        const int m = tid >> 4, col = tid & 15;
        const int64_t n = t * kTileN + col;
        if (m < p.M && n < p.N) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < kSmallWaves; ++w) s += red[w][m][col];
            store_out<AT>(p, m, n, s);
        }
    }
}

template <typename AT, typename ST, bool HAS_ZP, bool LDS_META>
__global__ __launch_bounds__(256) void gidx_mfma_kernel(GidxParams p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char meta_s[];
    __shared__ __attribute__((aligned(16))) float a_s[kBigRows][kChunkK + kAPad];    // A of the chunk, row-major
    __shared__ __attribute__((aligned(16))) float w_s[kChunkK][kBigTiles * kTileN + kWPad];  // weights, k-major
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int i = lane & 15, h = lane >> 4;
    const int64_t t0 = (int64_t)blockIdx.x * kBigTiles;
    const int m0 = blockIdx.y * kBigRows;
    // wave tt dequantizes tile t0 + tt; its metadata, in LDS when it fits
    const int64_t tw = t0 + wave;
    TileMeta<ST> mt;
    if constexpr (LDS_META) {
        const int64_t mb = meta_bytes(p.C, p.Q, (int)sizeof(ST), HAS_ZP);
        for (int tt = 0; tt < kBigTiles; ++tt) {
            if (t0 + tt < p.T) {
                const TileMeta<ST> m = stage_meta<ST, HAS_ZP>(p, t0 + tt, meta_s + tt * mb, tid, 256);
                if (tt == wave) mt = m;
            }
        }
        __syncthreads();
    } else {
        mt = global_meta<ST>(p, tw < p.T ? tw : 0);
    }
    fx4_t acc[kBigTiles];
#pragma unroll
    for (int tt = 0; tt < kBigTiles; ++tt) acc[tt] = fx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = 0; c < p.C; ++c) {
        // A: 64 rows x 128 k, 8 consecutive k per load (zero beyond M and K)
#pragma unroll
        for (int v = tid; v < kBigRows * (kChunkK / 8); v += 256) {
            const int r = v >> 4, k8 = (v & 15) * 8;
            const int m = m0 + r, k0 = c * kChunkK + k8;
            float x[8];
            if (m < p.M && k0 < p.K) {
                load_a8<AT>(p, m, k0, x);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = 0.0f;
            }
            *reinterpret_cast<fx4_t*>(&a_s[r][k8]) = fx4_t{x[0], x[1], x[2], x[3]};
            *reinterpret_cast<fx4_t*>(&a_s[r][k8 + 4]) = fx4_t{x[4], x[5], x[6], x[7]};
        }
        // weights: wave tt dequantizes the lane records of tile t0 + tt
        {
            const int tt = wave;
            const int64_t t = tw;
            uint4 d4 = make_uint4(0u, 0u, 0u, 0u);
            if (t < p.T) d4 = p.codes[(t * p.C + c) * 64 + lane];
            const uint32_t ds[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int kin = 32 * j + 8 * h;
                const int k0 = c * kChunkK + kin;
                float w[8];
                if (t < p.T && k0 < p.K) {
                    dequant_word<ST, HAS_ZP>(p, mt, i, ds[j], k0, w);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) w[e] = 0.0f;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) w_s[kin + e][tt * kTileN + i] = w[e];
            }
        }
        __syncthreads();
        // v_mfma_f32_16x16x4_f32: A lane (row i, k h), B lane (k h, column i)
        const int r = wave * 16 + i;
#pragma unroll 4
        for (int kk = 0; kk < kChunkK; kk += 4) {
            const float av = a_s[r][kk + h];
#pragma unroll
            for (int tt = 0; tt < kBigTiles; ++tt)
                acc[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, w_s[kk + h][tt * kTileN + i], acc[tt], 0, 0, 0);
        }
        __syncthreads();
    }
    // D lane layout: row 4h + e, column i
#pragma unroll
    for (int tt = 0; tt < kBigTiles; ++tt) {
        const int64_t n = (t0 + tt) * kTileN + i;
        if (n >= p.N) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = m0 + wave * 16 + 4 * h + e;
            if (m < p.M) store_out<AT>(p, m, n, acc[tt][e]);
        }
    }
}

template <typename AT, typename ST, bool HAS_ZP>
hipError_t launch_z(const Layout& L, const GidxParams& p, hipStream_t s)
{
    const int64_t mb = meta_bytes(L.C, L.Q, L.ss, HAS_ZP);
    if (p.M <= kSmallM) {
        const dim3 grid((unsigned)L.T), block(kSmallWaves * 64);
        if (mb <= kSmallMetaLds)
            gidx_small_kernel<AT, ST, HAS_ZP, true><<<grid, block, (size_t)mb, s>>>(p);
        else
            gidx_small_kernel<AT, ST, HAS_ZP, false><<<grid, block, 0, s>>>(p);
    } else {
        const dim3 grid((unsigned)((L.T + kBigTiles - 1) / kBigTiles), (unsigned)((p.M + kBigRows - 1) / kBigRows));
        if (kBigTiles * mb <= kBigMetaLds)
            gidx_mfma_kernel<AT, ST, HAS_ZP, true><<<grid, dim3(256), (size_t)(kBigTiles * mb), s>>>(p);
        else
            gidx_mfma_kernel<AT, ST, HAS_ZP, false><<<grid, dim3(256), 0, s>>>(p);
    }
    return hipGetLastError();
}

template <typename AT, typename ST>
hipError_t launch_s(const Layout& L, const GidxParams& p, hipStream_t s)
{
    return L.has_zp ? launch_z<AT, ST, true>(L, p, s) : launch_z<AT, ST, false>(L, p, s);
}

}  // namespace

int64_t gidx_max_m() { return (int64_t)65535 * kBigRows; }

hipError_t launch_gemm_gidx(const Layout& L, const WeightView& w, const void* a, int64_t m, bool f16_act,
                            const int32_t* g_idx, const Bias& bias, void* y, hipStream_t stream,
                            const char** variant)
{
    GidxParams p;
    p.codes = reinterpret_cast<const uint4*>(w.codes);
    p.scales = w.scales;
    p.zp = w.zp;
    p.g_idx = g_idx;
    p.a = a;
    p.bias = bias.ptr;
    p.bias_stride = bias.row_stride;
    p.after_round = bias.after_round;
    p.y = y;
    p.M = (int)m;
    p.N = (int)L.N;
    p.K = (int)L.K;
    p.C = (int)L.C;
    p.Q = L.Q;
    p.qshift = __builtin_ctz((unsigned)L.Q);
    p.kb = (int)L.kb;
    p.T = L.T;
    if (variant)
        *variant = m <= kSmallM ? (f16_act ? "gemm_gidx_stream_f16" : "gemm_gidx_stream_f32")
                                : (f16_act ? "gemm_gidx_mfma_f16" : "gemm_gidx_mfma_f32");
    if (f16_act)
        return L.ss == 2 ? launch_s<__half, __half>(L, p, stream) : launch_s<__half, float>(L, p, stream);
    return L.ss == 2 ? launch_s<float, __half>(L, p, stream) : launch_s<float, float>(L, p, stream);
}

}  // namespace mnb
