// gemm_small.hip -- small-M GEMM (2 <= M <= 16), the speculative-verify shape.
//
// Method: onnx-runtime-ep-cuda 0.1.0-dev.6, src/kernels/marlin_gemm.rs --
// fp16 activations times int4 weights on the matrix cores with fp32
// accumulation, a fresh accumulator per quantization group and the group's
// scale applied after that group's accumulate (module doc, "Why this module
// exists" and "Relationship to IST-DASLab/vLLM Marlin"), and a K split over
// groups whose fp32 partials are summed in a fixed order
// (matmul_nbits_marlin_gemm_f16_splitk / matmul_nbits_marlin_splitk_reduce).
//
// gfx950 design: the weight stream is the whole cost (M <= 16 rows reuse each
// weight at most 16 times), so a workgroup owns a few 16-column tiles and its
// waves split K.  Each wave streams one 16-byte code word per tile per
// 128-k chunk, unpacks it in registers to the B operand of
// v_mfma_f32_16x16x32_f16 and multiplies it with the A rows (rows >= M are
// zero), loaded straight from global memory and reused across the tiles.
// Waves then reduce through LDS in a fixed order.  The epilogue writes fp16
// (with an optional bias in either rounding) or, for int8 activation codes
// as A (accuracy_level 4), fp32 times the row's activation scale plus an fp32
// bias.
#include "mnb_device.hpp"
#include "mnb_acc4.hpp"
#include "mnb_internal.hpp"

namespace mnb {

namespace {

constexpr int kWaves = 16;   // the K split of a workgroup: more loads in flight per CU

struct SmallParams {
    const u4_t* codes;
    const void* scales;
    const uint8_t* zp;
    const _Float16* a;
    __half* y;
    const __half* bias;    // optional, element (m, n) at bias[m * bias_stride + n]
    int64_t bias_stride;
    int bias_after_round;
    // int8-activation codes as A: fp32 output y32[m, n] = row_scale[m] *
    // acc (+ bias32[n]) in place of the fp16 output (row_scale non-null)
    float* y32;
    const float* row_scale;
    const float* bias32;
    int64_t bias32_stride;  // fp32 bias element (m, n) at bias32[m * stride + n]
    // fp32 activations split into row pairs (hi, lo): output row m is
    // row_scale[m] * (acc[2m] + acc[2m + 1])
    int pair_rows;
    int M, N, K, C;
    int64_t T;
};

__device__ __forceinline__ f4_t mfma16(const h8_t& a, const h8_t& b, const f4_t& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h8_t make_b(const h2_t q[4])
{
    h8_t b;
    b[0] = q[0][0]; b[1] = q[0][1];
    b[2] = q[1][0]; b[3] = q[1][1];
    b[4] = q[2][0]; b[5] = q[2][1];
    b[6] = q[3][0]; b[7] = q[3][1];
    return b;
}

__device__ __forceinline__ h8_t zero_h8()
{
    h8_t z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (_Float16)0.0f;
    return z;
}

// TPW tiles per workgroup; Q groups per chunk.
template <typename ST, int Q, bool HAS_ZP, int TPW>
__global__ __launch_bounds__(kWaves * 64) void gemm_small_kernel(SmallParams p)
{
    __shared__ float red[kWaves][TPW][256];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int i = lane & 15;      // column in tile (B and D), row of A
    const int h = lane >> 4;      // k-octet (A and B), row quad of D
    const int64_t t0 = (int64_t)blockIdx.x * TPW;
    const int C = p.C;
    const int K = p.K;

    f4_t total[TPW];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) total[tt] = f4_t{0.f, 0.f, 0.f, 0.f};

    const bool row_ok = i < p.M;
    const _Float16* arow = p.a + (int64_t)(row_ok ? i : 0) * K;

    for (int c = wave; c < C; c += kWaves) {
        // loads: code words of every tile, A fragments of the 4 k-steps,
        // scales and zero points
        u4_t d[TPW];
        uint32_t zw[TPW];
        float s[TPW][Q <= 4 ? Q : 8];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int64_t t = t0 + tt;
            const int64_t chunk = (t < p.T ? t : p.T - 1) * C + c;
            d[tt] = __builtin_nontemporal_load(p.codes + chunk * 64 + lane);
            const ST* sp = static_cast<const ST*>(p.scales) + chunk * kTileN * Q;
            if (Q <= 4) {
#pragma unroll
                for (int q = 0; q < Q; ++q) s[tt][q] = to_f32(sp[i * Q + q]);
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) s[tt][q] = to_f32(sp[slot_of(i, q, 8)]);
            }
            zw[tt] = 0;
            if (HAS_ZP) {
                const uint8_t* zp = p.zp + chunk * (kTileN / 2) * Q;
                if (Q == 1) {
                    zw[tt] = (zp[i >> 1] >> (4 * (i & 1))) & 15u;
                } else if (Q == 2) {
                    zw[tt] = zp[i];
                } else {
                    const int sb = Q == 4 ? i * 4 : ((h >> 1) * 16 + i) * 4;
                    zw[tt] = *reinterpret_cast<const uint16_t*>(zp + sb / 2);
                }
            }
        }
        h8_t afr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = c * kChunkK + 32 * j + 8 * h;
            if (row_ok && k < K)
                afr[j] = *reinterpret_cast<const h8_t*>(arow + k);
            else
                afr[j] = zero_h8();
        }

#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const uint32_t dw[4] = {d[tt].x, d[tt].y, d[tt].z, d[tt].w};
            f4_t grp = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // zero point of this lane's k-octet
                const int zs = Q == 1 ? 0 : (Q == 2 ? (j >> 1) : j);
                const uint32_t z = HAS_ZP ? (zw[tt] >> (4 * zs)) & 15u : 8u;
                h2_t q[4];
                unpack8(dw[j], zp_const(z), q);
                const h8_t b = make_b(q);
                if (Q <= 4) {
                    grp = mfma16(afr[j], b, grp);
                    // last k-step of a group: scale and fold into the total
                    constexpr int steps = 4 / (Q <= 4 ? Q : 1);
                    if ((j + 1) % steps == 0) {
                        const float sc = s[tt][Q == 1 ? 0 : (Q == 2 ? (j >> 1) : j)];
#pragma unroll
                        for (int r = 0; r < 4; ++r) total[tt][r] = __builtin_fmaf(grp[r], sc, total[tt][r]);
                        grp = f4_t{0.f, 0.f, 0.f, 0.f};
                    }
                } else {
                    // group 16: a 32-k step spans groups 2j (octets 0,1) and
                    // 2j+1 (octets 2,3); one MFMA per group with the other
                    // group's octets zeroed
                    const h8_t zero = zero_h8();
                    const h8_t be = (h < 2) ? b : zero;
                    const h8_t bo = (h < 2) ? zero : b;
                    const f4_t ge = mfma16(afr[j], be, f4_t{0.f, 0.f, 0.f, 0.f});
                    const f4_t go = mfma16(afr[j], bo, f4_t{0.f, 0.f, 0.f, 0.f});
                    const float se = s[tt][2 * j], so = s[tt][2 * j + 1];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        total[tt][r] = __builtin_fmaf(ge[r], se, total[tt][r]);
                        total[tt][r] = __builtin_fmaf(go[r], so, total[tt][r]);
                    }
                }
            }
        }
    }

    // fixed-order reduction over the waves; D lane layout: row 4h + r, col i
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][tt][(4 * h + r) * 16 + i] = total[tt][r];
    __syncthreads();
    for (int o = tid; o < TPW * 256; o += kWaves * 64) {
        const int tt = o >> 8;
        const int e = o & 255;
        const int row = e >> 4, col = e & 15;
        const int64_t n = (t0 + tt) * kTileN + col;
        if (p.pair_rows) {
            // rows 2r and 2r + 1 hold the hi and lo parts of output row r
            if ((row & 1) == 0 && row < p.M && n < p.N) {
                float v = 0.0f, v2 = 0.0f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    v += red[w][tt][e];
                    v2 += red[w][tt][e + 16];
                }
                const int mo = row >> 1;
                float out = (v + v2) * p.row_scale[mo];
                if (p.bias32) out = out + p.bias32[(int64_t)mo * p.bias32_stride + n];
                p.y32[(int64_t)mo * p.N + n] = out;
            }
            continue;
        }
        if (row < p.M && n < p.N) {
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) v += red[w][tt][e];
            if (p.row_scale) {
                const float rs = p.row_scale[row];
                float o = rs != 0.0f ? v * rs : 0.0f;
                if (p.bias32) o = o + p.bias32[n];
                p.y32[(int64_t)row * p.N + n] = o;
            } else {
                p.y[(int64_t)row * p.N + n] = finish_output(v, p.bias, (int64_t)row * p.bias_stride + n,
                                                            p.bias_after_round);
            }
        }
    }
}

template <typename ST, int Q, bool HAS_ZP, int TPW>
hipError_t launch_t(const SmallParams& p, hipStream_t s)
{
    const int64_t blocks = (p.T + TPW - 1) / TPW;
    gemm_small_kernel<ST, Q, HAS_ZP, TPW><<<dim3((unsigned)blocks), dim3(kWaves * 64), 0, s>>>(p);
    return hipGetLastError();
}

template <typename ST, bool HAS_ZP>
hipError_t launch_q(const Layout& L, const SmallParams& p, hipStream_t s)
{
    switch (L.Q) {
    case 1: return launch_t<ST, 1, HAS_ZP, 4>(p, s);
    case 2: return launch_t<ST, 2, HAS_ZP, 4>(p, s);
    case 4: return launch_t<ST, 4, HAS_ZP, 4>(p, s);
    default: return launch_t<ST, 8, HAS_ZP, 4>(p, s);
    }
}

}  // namespace

size_t gemm_small_workspace(const Layout&, int64_t) { return 0; }

hipError_t launch_gemm_small(const Layout& L, const WeightView& w, const void* a, int64_t m,
                             const Bias& bias, void* y, void*, hipStream_t stream, const char** variant)
{
    SmallParams p;
    p.y32 = nullptr;
    p.row_scale = nullptr;
    p.bias32 = nullptr;
    p.bias32_stride = 0;
    p.pair_rows = 0;
    p.codes = reinterpret_cast<const u4_t*>(w.codes);
    p.scales = w.scales;
    p.zp = w.zp;
    p.a = static_cast<const _Float16*>(a);
    p.y = static_cast<__half*>(y);
    p.bias = static_cast<const __half*>(bias.ptr);
    p.bias_stride = bias.row_stride;
    p.bias_after_round = bias.after_round;
    p.M = (int)m;
    p.N = (int)L.N;
    p.K = (int)L.K;
    p.C = (int)L.C;
    p.T = L.T;
    if (variant) *variant = "gemm_small_m";
    if (L.ss == 2)
        return L.has_zp ? launch_q<__half, true>(L, p, stream) : launch_q<__half, false>(L, p, stream);
    return L.has_zp ? launch_q<float, true>(L, p, stream) : launch_q<float, false>(L, p, stream);
}

hipError_t launch_gemm_small_f32(const Layout& L, const WeightView& w, const void* a16, int64_t m,
                                 const float* row_scale, const float* bias, float* y, void*,
                                 hipStream_t stream, const char** variant, int pair_rows, int64_t bias_stride)
{
    SmallParams p;
    p.codes = reinterpret_cast<const u4_t*>(w.codes);
    p.scales = w.scales;
    p.zp = w.zp;
    p.a = static_cast<const _Float16*>(a16);
    p.y = nullptr;
    p.bias = nullptr;
    p.bias_stride = 0;
    p.bias_after_round = 0;
    p.y32 = y;
    p.row_scale = row_scale;
    p.bias32 = bias;
    p.bias32_stride = bias_stride;
    p.pair_rows = pair_rows;
    p.M = (int)m;
    p.N = (int)L.N;
    p.K = (int)L.K;
    p.C = (int)L.C;
    p.T = L.T;
    if (variant) *variant = pair_rows ? "gemm_small_m_f32act" : "gemm_small_m_accuracy4";
    if (L.ss == 2)
        return L.has_zp ? launch_q<__half, true>(L, p, stream) : launch_q<__half, false>(L, p, stream);
    return L.has_zp ? launch_q<float, true>(L, p, stream) : launch_q<float, false>(L, p, stream);
}

}  // namespace mnb
