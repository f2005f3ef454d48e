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
// v_mfma_f32_16x16x32_f16 and multiplies it with the A rows, which reach a
// slot of the wave's own in LDS by DMA and are reused across the tiles.  At
// these sizes the kernel is bound by issued instructions, so every load is a
// buffer load with the chunk in a scalar offset and the small per-chunk
// records come through LDS too.  Waves then reduce through LDS in a fixed
// order.  The epilogue writes fp16
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

// LDS destination pointer of buffer_load ... lds
typedef void __attribute__((address_space(3))) * lds_ptr_t;

// One 16-byte LDS DMA per lane (lane L's bytes land at dst + 16 L).  The
// builtin is compiled in the device pass only: the host pass compiles this
// kernel just for its launch stub, and with the 16-byte form in it that pass
// dropped the stub.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, lds_ptr_t dst, uint32_t voff, uint32_t soff)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
#endif
}

// Wait until at most N vector-memory operations of this wave are
// outstanding (gfx9 s_waitcnt encoding; expcnt and lgkmcnt left open).
template <int N> __device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// A lane's scales of one tile and chunk as one integer (NS consecutive
// scales), so the load stays a single instruction.
template <typename ST, int NS> struct RawScales;
template <> struct RawScales<__half, 1> { typedef uint16_t type; };
template <> struct RawScales<__half, 2> { typedef uint32_t type; };
template <> struct RawScales<__half, 4> { typedef uint64_t type; };
template <> struct RawScales<float, 1> { typedef uint32_t type; };
template <> struct RawScales<float, 2> { typedef uint64_t type; };
template <> struct RawScales<float, 4> { typedef u4_t type; };

template <typename T> __device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff);
template <> __device__ __forceinline__ uint16_t buf_load<uint16_t>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
template <> __device__ __forceinline__ uint32_t buf_load<uint32_t>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
template <> __device__ __forceinline__ uint64_t buf_load<uint64_t>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
template <> __device__ __forceinline__ u4_t buf_load<u4_t>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

template <typename ST, int NS>
__device__ __forceinline__ float raw_scale(const typename RawScales<ST, NS>::type& r, int s)
{
    if constexpr (sizeof(ST) == 2) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(r >> (16 * s)));
    } else if constexpr (NS == 4) {
        const uint32_t e = r[s];
        return __builtin_bit_cast(float, e);
    } else {
        return __builtin_bit_cast(float, (uint32_t)(r >> (32 * s)));
    }
}

// Chunks per wave requested together: every load of a batch is in flight
// before the first compute, so a wave pays one memory round trip per batch,
// not one per chunk.  Two where the batch's registers fit the 128 a 16-wave
// workgroup allows (fp16 scales, groups of 32 k or more), else one.
template <typename ST, int Q> constexpr int batch_of() { return sizeof(ST) == 2 && Q <= 4 ? 2 : 1; }

// TPW tiles per workgroup; Q groups per chunk.  KTAIL: K is not a multiple
// of 128, so the activation loads of the last chunk are masked per k.
//
// Every load is a buffer load: the workgroup's tiles and the activation are
// buffer ranges, a lane's part of each offset is fixed, and the chunk's part
// is wave-uniform (a scalar offset), so addressing costs no vector
// instructions.  Activation rows >= M read zero through the range check.
//
// The arguments are scalars, those the first loads need first (the codes,
// scales and zero points, A, M, K, C and the tile count): built with kernarg
// preloading (-amdgpu-kernarg-preload-count), the first 16 dwords arrive in
// SGPRs when the wave starts instead of through a scalar load of the
// argument block.
template <typename ST, int Q, bool HAS_ZP, int TPW, bool KTAIL>
__global__ __launch_bounds__(kWaves * 64) void gemm_small_kernel(
    const u4_t* codes, const void* scales, const uint8_t* zp, const _Float16* a, int M_, int K_, int C_, int64_t T_,
    int N_, __half* y, const __half* bias, int64_t bias_stride, int bias_after_round, float* y32,
    const float* row_scale, const float* bias32, int64_t bias32_stride, int pair_rows)
{
    SmallParams p;
    p.codes = codes;
    p.scales = scales;
    p.zp = zp;
    p.a = a;
    p.y = y;
    p.bias = bias;
    p.bias_stride = bias_stride;
    p.bias_after_round = bias_after_round;
    p.y32 = y32;
    p.row_scale = row_scale;
    p.bias32 = bias32;
    p.bias32_stride = bias32_stride;
    p.pair_rows = pair_rows;
    p.M = M_;
    p.N = N_;
    p.K = K_;
    p.C = C_;
    p.T = T_;
    constexpr int kBatch = batch_of<ST, Q>();
    // Each wave's slices of A (its chunks' 128 k of all 16 rows, 4 KiB per
    // chunk) reach a slot of its own by 16-byte LDS DMAs; the 16-byte
    // segments of a row are XOR-swizzled by the row so fragment reads are
    // conflict free.  After the wave's last chunk its slot holds its partial
    // sums for the cross-wave reduction.
    constexpr int kASlot = kBatch * 16 * kChunkK * 2;
    static_assert(TPW * 256 * 4 <= kASlot, "the wave partials fit the wave's slot");
    __shared__ __align__(16) unsigned char a_lds[kWaves][kASlot];
    constexpr int NS = Q <= 4 ? Q : 4;           // scales per load (two loads for groups of 16)
    constexpr int NL = Q <= 4 ? 1 : 2;
    constexpr int SREC = kTileN * Q * (int)sizeof(ST), ZREC = kTileN / 2 * Q;
    // For groups of 32 k or more the scales and zero points of a batch come
    // through LDS: a few dword DMAs per wave (buffer_load ... lds, 64 dwords
    // each) instead of one small load per record, then LDS reads.  A wave's
    // region holds a full 64-lane slot per DMA, scales first, then zero points.
    constexpr bool META_LDS = Q <= 4;
    constexpr int R = kBatch * TPW;                                  // records per batch
    constexpr int kSInstr = (R * SREC / 4 + 63) / 64;
    constexpr int kMetaBytes = kSInstr * 256 + 256;
    __shared__ __align__(16) unsigned char meta_lds[META_LDS ? kWaves : 1][META_LDS ? kMetaBytes : 16];
    constexpr uint32_t kFar = 0x80000000u;       // past every range: reads zero
    typedef typename RawScales<ST, NS>::type RawS;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int i = lane & 15;      // column in tile (B and D), row of A
    const int h = lane >> 4;      // k-octet (A and B), row quad of D
    const int64_t t0 = (int64_t)blockIdx.x * TPW;
    const int C = p.C;
    const int K = p.K;
    const int tiles_here = (int)((p.T - t0) < TPW ? (p.T - t0) : TPW);

    const __amdgpu_buffer_rsrc_t c_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.codes + t0 * C * 64), (short)0, tiles_here * C * kChunkBytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const uint8_t*>(p.scales) + t0 * C * SREC), (short)0, tiles_here * C * SREC, 0x00020000);
    const __amdgpu_buffer_rsrc_t z_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(HAS_ZP ? p.zp + t0 * C * ZREC : reinterpret_cast<const uint8_t*>(p.codes)), (short)0,
        HAS_ZP ? tiles_here * C * ZREC : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.a, (short)0, p.M * K * 2, 0x00020000);

    // lane parts of the offsets
    // A DMA of row quad qd: lane L fetches row 4 qd + L / 16, logical
    // segment (L % 16) ^ row (8 k each); rows >= M lie past the range (zeros)
    uint32_t a_dvoff[4];
    int a_dseg[4];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
        const int r = 4 * qd + (lane >> 4);
        a_dseg[qd] = ((lane & 15) ^ r) * 8;
        a_dvoff[qd] = ((uint32_t)r * (uint32_t)K + (uint32_t)a_dseg[qd]) * 2u;
    }
    const uint32_t s_voff = (uint32_t)(Q <= 4 ? i * Q : i * 4) * (uint32_t)sizeof(ST);
    const uint32_t z_voff = Q == 1 ? (uint32_t)(i >> 1) : (Q == 2 ? (uint32_t)i : (Q == 4 ? 2u * i : 2u * ((h >> 1) * 16 + i)));

    f4_t total[TPW];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) total[tt] = f4_t{0.f, 0.f, 0.f, 0.f};

    // DMA offsets (fixed per lane): scale dword p = lane + 64 m of record
    // r = p / (SREC / 4); zero-point dword d = lane of record d / (ZREC / 4).
    // Record r = u * TPW + tt is chunk cb + kWaves * u of tile tt.
    uint32_t ms_voff[kSInstr];
#pragma unroll
    for (int m = 0; m < kSInstr; ++m) {
        const int pc = lane + 64 * m;
        const int r = pc / (SREC / 4), w = pc % (SREC / 4);
        ms_voff[m] = pc < R * SREC / 4
            ? (uint32_t)(((r % TPW) * C + kWaves * (r / TPW)) * SREC + w * 4) : kFar;
    }
    uint32_t mz_voff;
    {
        constexpr int ZD = ZREC / 4 > 0 ? ZREC / 4 : 1;
        const int r = lane / ZD, w = lane % ZD;
        mz_voff = (HAS_ZP && lane < R * ZD) ? (uint32_t)(((r % TPW) * C + kWaves * (r / TPW)) * ZREC + w * 4) : kFar;
    }

    for (int cb = wave; cb < C; cb += kWaves * kBatch) {
        // Issue order: the batch's A slices (LDS DMAs), then its scales and
        // zero points, then its code words.  Waits count completions in
        // issue order, so the small loads never wait behind the code stream.
        // A chunk past K loads the last chunk's weights again and is not
        // computed.  Row quads wholly past M are not fetched: those rows of
        // the slot hold stale values, and MFMA output rows depend on their
        // own A row only, so they reach no stored output.
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int cu = cb + kWaves * u;               // wave-uniform
                if (4 * qd < p.M) {
                    uint32_t vo = a_dvoff[qd];
                    if (KTAIL && cu * kChunkK + a_dseg[qd] >= K) vo = kFar;
                    lds_dma16(a_rsrc, (lds_ptr_t)(a_lds[wave] + u * 4096 + qd * 1024), vo, (uint32_t)cu * (kChunkK * 2));
                }
            }
        __builtin_amdgcn_sched_barrier(0);
        RawS sr[kBatch][TPW][NL];
        uint32_t zw[kBatch][TPW];
        uint32_t rec[kBatch][TPW];
        if constexpr (META_LDS) {
            unsigned char* mb = meta_lds[wave];
#pragma unroll
            for (int m = 0; m < kSInstr; ++m)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lds_ptr_t)(mb + m * 256), 4, ms_voff[m],
                                                         (uint32_t)cb * SREC, 0, 0);
            if (HAS_ZP)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(z_rsrc, (lds_ptr_t)(mb + kSInstr * 256), 4, mz_voff,
                                                         (uint32_t)cb * ZREC, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const int c = cb + kWaves * u;
                // a tile past N reads zero (outside the range); its outputs are not stored
                rec[u][tt] = (uint32_t)(tt * C + (c < C ? c : C - 1));
                if (META_LDS) continue;
                sr[u][tt][0] = buf_load<RawS>(s_rsrc, s_voff, rec[u][tt] * SREC);
                // groups of 16: the even groups of the 16 columns, then the odd ones
                if (NL > 1) sr[u][tt][NL - 1] = buf_load<RawS>(s_rsrc, s_voff + 16 * sizeof(RawS), rec[u][tt] * SREC);
                zw[u][tt] = 0;
                if (HAS_ZP) {
                    if (Q <= 2)
                        zw[u][tt] = __builtin_amdgcn_raw_buffer_load_b8(z_rsrc, z_voff, rec[u][tt] * ZREC, 0);
                    else
                        zw[u][tt] = buf_load<uint16_t>(z_rsrc, z_voff, rec[u][tt] * ZREC);
                }
            }
        __builtin_amdgcn_sched_barrier(0);
        u4_t d[kBatch][TPW];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt)
                d[u][tt] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(
                    c_rsrc, (uint32_t)lane * 16u, rec[u][tt] * kChunkBytes, 2));
        __builtin_amdgcn_sched_barrier(0);
        // wait until the DMAs (activation, and scales and zero points through
        // LDS) have landed; the batch's code words (and for groups of 16 its
        // scale and zero-point loads) may stay in flight.  The LDS reads
        // below stay after it.
        if constexpr (META_LDS) wait_vm<R>();
        else wait_vm<R + R * (NL + (HAS_ZP ? 1 : 0))>();
        asm volatile("" ::: "memory");
        h8_t afr[kBatch][4];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                afr[u][j] = *reinterpret_cast<const h8_t*>(a_lds[wave] + u * 4096 + i * 256 + (((4 * j + h) ^ i) * 16));
        if constexpr (META_LDS) {
            const unsigned char* mb = meta_lds[wave];
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt) {
                    const int r = u * TPW + tt;
                    sr[u][tt][0] = *reinterpret_cast<const RawS*>(mb + r * SREC + i * Q * (int)sizeof(ST));
                    zw[u][tt] = 0;
                    if (HAS_ZP) {
                        const unsigned char* zr = mb + kSInstr * 256 + r * ZREC;
                        if (Q == 1) zw[u][tt] = zr[i >> 1];
                        else if (Q == 2) zw[u][tt] = zr[i];
                        else zw[u][tt] = *reinterpret_cast<const uint16_t*>(zr + 2 * i);
                    }
                }
        }

#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (cb + kWaves * u >= C) continue;   // wave-uniform
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const uint32_t dw[4] = {d[u][tt].x, d[u][tt].y, d[u][tt].z, d[u][tt].w};
                // zero point of group q of the lane's column (or of its octet
                // half's group q for groups of 16)
                auto zr_of = [&](int q) {
                    uint32_t z = 8u;
                    if (HAS_ZP) z = Q == 1 ? (zw[u][tt] >> (4 * (i & 1))) & 15u : (zw[u][tt] >> (4 * q)) & 15u;
                    return zp_pair(z);
                };
                if constexpr (Q <= 4) {
                    // one independent chain per group, then the scales in
                    // group order
                    constexpr int steps = 4 / Q;   // k-steps per group
                    f4_t grp[Q];
                    uint32_t zr[Q];
#pragma unroll
                    for (int gq = 0; gq < Q; ++gq) zr[gq] = zr_of(gq);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        h2_t q[4];
                        unpack_zr(dw[j], zr[j / steps], q);
                        grp[j / steps] = mfma16(afr[u][j], make_b(q),
                                                (j % steps == 0) ? f4_t{0.f, 0.f, 0.f, 0.f} : grp[j / steps]);
                    }
#pragma unroll
                    for (int gq = 0; gq < Q; ++gq) {
                        const float sc = raw_scale<ST, NS>(sr[u][tt][0], gq);
#pragma unroll
                        for (int r = 0; r < 4; ++r) total[tt][r] = __builtin_fmaf(grp[gq][r], sc, total[tt][r]);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        h2_t q[4];
                        unpack_zr(dw[j], zr_of(j), q);
                        const h8_t b = make_b(q);
                        // group 16: a 32-k step spans groups 2j (octets 0,1) and
                        // 2j+1 (octets 2,3); one MFMA per group with the other
                        // group's activation octets zeroed (not its weights:
                        // an infinite activation times a zeroed weight would
                        // put a NaN into the other group)
                        const h8_t zero = zero_h8();
                        const h8_t ae = (h < 2) ? afr[u][j] : zero;
                        const h8_t ao = (h < 2) ? zero : afr[u][j];
                        const f4_t ge = mfma16(ae, b, f4_t{0.f, 0.f, 0.f, 0.f});
                        const f4_t go = mfma16(ao, b, f4_t{0.f, 0.f, 0.f, 0.f});
                        const float se = raw_scale<ST, NS>(sr[u][tt][0], j);
                        const float so = raw_scale<ST, NS>(sr[u][tt][NL - 1], j);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            total[tt][r] = __builtin_fmaf(ge[r], se, total[tt][r]);
                            total[tt][r] = __builtin_fmaf(go[r], so, total[tt][r]);
                        }
                    }
                }
            }
        }
    }

    // fixed-order reduction over the waves; D lane layout: row 4h + r, col i.
    // A wave's partials go to its own slot, whose A reads are all done.
    auto red_of = [&](int w) { return reinterpret_cast<float*>(a_lds[w]); };
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red_of(wave)[tt * 256 + (4 * h + r) * 16 + i] = total[tt][r];
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
                    v += red_of(w)[tt * 256 + e];
                    v2 += red_of(w)[tt * 256 + e + 16];
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
            for (int w = 0; w < kWaves; ++w) v += red_of(w)[tt * 256 + e];
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
    if (p.K % kChunkK != 0)
        gemm_small_kernel<ST, Q, HAS_ZP, TPW, true><<<dim3((unsigned)blocks), dim3(kWaves * 64), 0, s>>>(
            p.codes, p.scales, p.zp, p.a, p.M, p.K, p.C, p.T, p.N, p.y, p.bias, p.bias_stride, p.bias_after_round, p.y32,
            p.row_scale, p.bias32, p.bias32_stride, p.pair_rows);
    else
        gemm_small_kernel<ST, Q, HAS_ZP, TPW, false><<<dim3((unsigned)blocks), dim3(kWaves * 64), 0, s>>>(
            p.codes, p.scales, p.zp, p.a, p.M, p.K, p.C, p.T, p.N, p.y, p.bias, p.bias_stride, p.bias_after_round, p.y32,
            p.row_scale, p.bias32, p.bias32_stride, p.pair_rows);
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

// Largest K the kernel's 32-bit buffer ranges cover: the code bytes of a
// workgroup's 4 tiles (4 * K / 128 * 1024 = 32 K) and 16 rows of fp16
// activations (32 K) stay below 2^31 for K <= 2^25.
int64_t gemm_small_max_k() { return int64_t(1) << 25; }

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
