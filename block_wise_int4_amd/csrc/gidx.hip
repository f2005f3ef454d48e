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
// gfx950 design, one weight-streaming kernel: a workgroup of 16 waves owns
// one 16-column tile and a block of rows (up to 16 rows when M <= 16, else
// 64), and first writes a table of the tile's (zero point, scale) pairs per
// group to LDS (read from L2 instead when the table is too large).  Each wave
// takes every 16th 128-k chunk, one lane per 16-byte lane record (one column,
// 32 k), and dequantizes its 32 weights in registers, one table read each.
// It multiplies them into the rows of A, read straight from L2: one row by
// fp32 fma, more on v_mfma_f32_16x16x4_f32, each word's weights reused for
// every block of 16 rows.  No barrier inside the loop; the lanes of a column
// and then the 16 waves are summed in a fixed order at the end.
#include <type_traits>

#include "mnb_device.hpp"
#include "mnb_gidx.hpp"

namespace mnb {

namespace {

typedef float fx4_t __attribute__((ext_vector_type(4)));

constexpr int kSmallM = 16;     // rows per workgroup when M <= 16
constexpr int kBigRows = 64;    // rows per workgroup beyond
constexpr int kSmallWaves = 16;
// LDS for the table of (zero point, scale) pairs, 128 bytes per group (else
// the pairs are read from L2): 1024 threads keep one workgroup per CU
// anyway; beside the 64 KiB reduction array of 64 rows, less.
constexpr int64_t kSmallTableLds = 96 * 1024;
constexpr int64_t kBigTableLds = 80 * 1024;

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

// The streaming kernel's per-tile table in LDS: entry G * 16 + i holds the
// zero point and the scale of group G and column i as fp32 (x, y); entry
// kb * 16 + i is (0, 0), the weight of a group out of range.
__host__ __device__ inline int64_t table_bytes(int64_t kb) { return (kb + 1) * kTileN * 8; }

template <typename ST, bool HAS_ZP>
__device__ __forceinline__ void stage_table(const GidxParams& p, int64_t t, float2* tab, int tid, int nthreads)
{
    const TileMeta<ST> g = global_meta<ST>(p, t);
    const int n = (p.kb + 1) * kTileN;
    for (int v = tid; v < n; v += nthreads) {
        const int G = v >> 4, i = v & 15;
        float2 e = make_float2(0.0f, 0.0f);
        if (G < p.kb) {
            const int cg = G >> p.qshift, q = G & (p.Q - 1);
            const int s = slot_of(i, q, p.Q);
            uint32_t z = 8u;
            if (HAS_ZP) z = (g.zp[cg * (kTileN / 2) * p.Q + (s >> 1)] >> (4 * (s & 1))) & 15u;
            e = make_float2((float)z, to_f32(g.scales[cg * kTileN * p.Q + s]));
        }
        tab[v] = e;
    }
}

// dequant_word through the table: the same weights, (code - zp) * scale,
// and 0 for a group out of range ((code - 0) * 0).
__device__ __forceinline__ void dequant_word_tab(const GidxParams& p, const float2* tab, int i, uint32_t d, int k0,
                                                 float w[8])
{
    const int4 g0 = *reinterpret_cast<const int4*>(p.g_idx + k0);
    const int4 g1 = *reinterpret_cast<const int4*>(p.g_idx + k0 + 4);
    const int gs[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int G = (unsigned)gs[e] < (unsigned)p.kb ? gs[e] : p.kb;
        const float2 zs = tab[G * kTileN + i];
        w[e] = ((float)code_at(d, e) - zs.x) * zs.y;
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

// RB blocks of 16 rows from row blockIdx.y * 16 * RB.  MF (M >= 2): the
// products on v_mfma_f32_16x16x4_f32, one per k offset e of a word: lane
// (i, h) gives A row i at k = k0(h) + e and B column i at the same k, so
// D[row][col] sums over the word's four k-octets.  The tail past K enters as
// zeros, so every lane issues the same MFMAs.  Otherwise (M = 1) fp32 fma.
template <typename AT, typename ST, bool HAS_ZP, bool TABLE, bool MF, int RB>
__global__ __launch_bounds__(kSmallWaves * 64) void gidx_stream_kernel(GidxParams p)
{
    static_assert(MF || RB == 1, "the fp32 fma form serves one block of rows");
    __shared__ float red[kSmallWaves][16 * RB][kTileN];
    extern __shared__ __attribute__((aligned(16))) unsigned char meta_s[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = lane & 15, h = lane >> 4;
    const int64_t t = blockIdx.x;
    const int m0 = blockIdx.y * 16 * RB;   // first row of the workgroup
    const float2* tab = reinterpret_cast<const float2*>(meta_s);
    const TileMeta<ST> mt = global_meta<ST>(p, t);
    if constexpr (TABLE) {
        stage_table<ST, HAS_ZP>(p, t, reinterpret_cast<float2*>(meta_s), threadIdx.x, kSmallWaves * 64);
        __syncthreads();
    }
    float acc[kSmallM];
#pragma unroll
    for (int m = 0; m < kSmallM; ++m) acc[m] = 0.0f;
    fx4_t dacc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) dacc[rb] = fx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = wave; c < p.C; c += kSmallWaves) {
        const uint4 d4 = p.codes[(t * p.C + c) * 64 + lane];
        const uint32_t ds[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k0 = c * kChunkK + 32 * j + 8 * h;
            if constexpr (MF) {
                float w[8];
                if (k0 < p.K) {
                    if constexpr (TABLE)
                        dequant_word_tab(p, tab, i, ds[j], k0, w);
                    else
                        dequant_word<ST, HAS_ZP>(p, mt, i, ds[j], k0, w);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) w[e] = 0.0f;
                }
                // the word's weights, reused for every block of 16 rows
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const int row = m0 + 16 * rb + i;
                    float x[8];
                    if (k0 < p.K && row < p.M) {
                        load_a8<AT>(p, row, k0, x);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) x[e] = 0.0f;
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        dacc[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[e], w[e], dacc[rb], 0, 0, 0);
                }
                continue;
            }
            if (k0 < p.K) {   // the chunk's tail beyond K holds no weights
                float w[8];
                if constexpr (TABLE)
                    dequant_word_tab(p, tab, i, ds[j], k0, w);
                else
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
    if constexpr (MF) {
        // D lane layout: rows 4h + r of each block, column i
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][16 * rb + 4 * h + r][i] = dacc[rb][r];
    } else {
        // the 4 lanes of column i (h = 0..3), then the waves in order
#pragma unroll
        for (int m = 0; m < kSmallM; ++m) {
            float v = acc[m];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            if (h == 0) red[wave][m][i] = v;
        }
    }
    __syncthreads();
    for (int o = threadIdx.x; o < 16 * RB * kTileN; o += kSmallWaves * 64) {
        const int r = o >> 4, col = o & 15;
        const int m = m0 + r;
        const int64_t n = t * kTileN + col;
        if (m < p.M && n < p.N) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < kSmallWaves; ++w) s += red[w][r][col];
            store_out<AT>(p, m, n, s);
        }
    }
}

template <typename AT, typename ST, bool HAS_ZP>
hipError_t launch_z(const Layout& L, const GidxParams& p, hipStream_t s)
{
    if (p.M <= kSmallM) {
        const dim3 grid((unsigned)L.T), block(kSmallWaves * 64);
        const int64_t tb = table_bytes(L.kb);
        const bool table = tb <= kSmallTableLds, mf = p.M > 1;
        if (table && mf)
            gidx_stream_kernel<AT, ST, HAS_ZP, true, true, 1><<<grid, block, (size_t)tb, s>>>(p);
        else if (table)
            gidx_stream_kernel<AT, ST, HAS_ZP, true, false, 1><<<grid, block, (size_t)tb, s>>>(p);
        else if (mf)
            gidx_stream_kernel<AT, ST, HAS_ZP, false, true, 1><<<grid, block, 0, s>>>(p);
        else
            gidx_stream_kernel<AT, ST, HAS_ZP, false, false, 1><<<grid, block, 0, s>>>(p);
    } else {
        // 64 rows per workgroup, the weights dequantized once for all of them
        const dim3 grid((unsigned)L.T, (unsigned)((p.M + kBigRows - 1) / kBigRows)), block(kSmallWaves * 64);
        const int64_t tb = table_bytes(L.kb);
        if (tb <= kBigTableLds)
            gidx_stream_kernel<AT, ST, HAS_ZP, true, true, kBigRows / 16><<<grid, block, (size_t)tb, s>>>(p);
        else
            gidx_stream_kernel<AT, ST, HAS_ZP, false, true, kBigRows / 16><<<grid, block, 0, s>>>(p);
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
    if (variant) *variant = f16_act ? "gemm_gidx_stream_f16" : "gemm_gidx_stream_f32";
    if (f16_act)
        return L.ss == 2 ? launch_s<__half, __half>(L, p, stream) : launch_s<__half, float>(L, p, stream);
    return L.ss == 2 ? launch_s<float, __half>(L, p, stream) : launch_s<float, float>(L, p, stream);
}

}  // namespace mnb
