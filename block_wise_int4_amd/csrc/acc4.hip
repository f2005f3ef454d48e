// acc4.hip -- int8 activations (accuracy_level 4) on the int8 matrix cores.
//
// Method: onnx-runtime-ep-cuda 0.1.0-dev.3, src/kernels/matmul_nbits.rs --
// the accuracy_level=4 path of the fp32 operator (kernels
// matmul_nbits_accuracy4, matmul_nbits_quantize_accuracy4_block32 and
// matmul_nbits_gemv_accuracy4_block32): each row of A gets one binary32
// scale, max|a| / 127; an activation's code is a * (1/scale), clamped to
// [-127, 127] and rounded half away from zero; per block the integer dot
// sum q * (code - zp) is exact, scaled by the block's weight scale, summed,
// and the sum is scaled by the row's activation scale.  A row whose maximum
// is 0 gives the bias (or 0).
//
// M = 1 (this file's GEMV): every workgroup quantizes the activation row
// itself while its code words stream in (no second launch, no round trip
// through memory), then runs the 16-column tile on v_mfma_i32_16x16x64_i8.
// The B operand is the raw codes 0..15 (two masks per word); the zero point
// enters as z * (sum of the block's codes), an exact integer correction, so
// the integer dot of every block is exact and rounds once, at its scale.
#include "mnb_acc4.hpp"
#include "mnb_device.hpp"

namespace mnb {

namespace {

typedef int32_t i4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

constexpr int kMaxWaves = 16;
constexpr int kResidentWaves = 256 * 32;   // CUs x wave slots per CU
constexpr int kAV = 4;                     // activation vectors a thread keeps in registers
constexpr int64_t kMaxRecordBytes = 32 * 1024;

// One activation's int8 code, in the binary32 steps of the pages.
__device__ __forceinline__ int quant1(float x, float inv)
{
    return (int)roundf(fminf(127.0f, fmaxf(-127.0f, x * inv)));
}

struct Acc4Params {
    const u4_t* codes;
    const void* scales;
    const uint8_t* zp;
    const float* a;
    const float* bias;
    float* y;
    _Float16* q_out;
    float* s_out;
    int N, K, C;
};

// Scales a lane needs per chunk: its column's groups 0..Q-1, or with eight
// groups per chunk the four of its lane half (h', h'+2, h'+4, h'+6), as
// one integer so the load is a single instruction.
template <typename ST, int NS> struct RawScales;
template <> struct RawScales<__half, 1> { typedef uint16_t type; };
template <> struct RawScales<__half, 2> { typedef uint32_t type; };
template <> struct RawScales<__half, 4> { typedef uint64_t type; };
template <> struct RawScales<float, 1> { typedef uint32_t type; };
template <> struct RawScales<float, 2> { typedef u2_t type; };
template <> struct RawScales<float, 4> { typedef u4_t type; };

template <typename ST, int NS>
__device__ __forceinline__ float raw_scale(const typename RawScales<ST, NS>::type& r, int s)
{
    if constexpr (sizeof(ST) == 2) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(r >> (16 * s)));
    } else if constexpr (NS == 1) {
        return __builtin_bit_cast(float, r);
    } else {
        const uint32_t e = r[s];
        return __builtin_bit_cast(float, e);
    }
}

template <typename ST, int Q> struct Chunk {
    static constexpr int NS = Q >= 4 ? 4 : Q;
    u4_t d;
    typename RawScales<ST, NS>::type s;
    uint32_t zw;
};

template <typename ST, int Q, bool HAS_ZP>
__device__ __forceinline__ void load_meta(const Acc4Params& p, int64_t chunk, int lane, Chunk<ST, Q>& r)
{
    constexpr int NS = Chunk<ST, Q>::NS;
    const int i = lane & 15, hh = (lane >> 4) & 1;
    const int sbase = Q <= 4 ? i * Q : (hh * 16 + i) * 4;
    const ST* sp = static_cast<const ST*>(p.scales) + chunk * kTileN * Q + sbase;
    r.s = *reinterpret_cast<const typename RawScales<ST, NS>::type*>(sp);
    if (HAS_ZP) {
        const uint8_t* zp = p.zp + chunk * (kTileN / 2) * Q;
        if (Q == 1)
            r.zw = (zp[i >> 1] >> (4 * (i & 1))) & 15u;
        else if (Q == 2)
            r.zw = zp[i];
        else
            r.zw = *reinterpret_cast<const uint16_t*>(zp + sbase / 2);
    } else {
        r.zw = 0;
    }
}

template <typename ST, int Q>
__device__ __forceinline__ void load_codes(const Acc4Params& p, int64_t chunk, int lane, Chunk<ST, Q>& r)
{
    r.d = __builtin_nontemporal_load(p.codes + chunk * 64 + lane);
}

// One chunk (16 columns x 128 k).  Word j of lane (column i, k-octet h)
// holds k = 32j + 8h + {0,2,4,6,1,3,5,7} in its nibble slots, so its low
// nibbles are k-offsets 0,4,1,5 and its high nibbles 2,6,3,7: two masks give
// the eight codes as bytes in that order, and the activation records in LDS
// are stored in the same order.  The 64-k halves of the chunk are two
// 16x16x64 products; one row of the A operand per group of the chunk carries
// that group's activations and zeros elsewhere, so that output row is the
// group's integer dot for every column.  Lane (h', i) receives rows
// 4h'..4h'+3 of column i.  With up to four groups per chunk, group q is row
// q (lanes h' = 0).  With eight, the scale and zero-point slots give lane
// half h' the groups h', h'+2, h'+4, h'+6, so group q is row 4(q & 1) + q/2.
template <typename ST, int Q, bool HAS_ZP>
__device__ __forceinline__ float chunk_acc4(const Chunk<ST, Q>& r, const unsigned char* rec,
                                            const int32_t* qsum, int c, int h, int row, float acc)
{
    constexpr int G = kChunkK / Q;
    constexpr int NS = Chunk<ST, Q>::NS;
    const uint32_t dw[4] = {r.d.x, r.d.y, r.d.z, r.d.w};
    i4_t A[2], B[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int q = (32 * j + 8 * h) / G;
        const int qrow = Q == 8 ? 4 * (q & 1) + (q >> 1) : q;
        const u2_t a = *reinterpret_cast<const u2_t*>(rec + c * kChunkK + 32 * j + 8 * h);
        const bool use = row == qrow;
        B[j >> 1][2 * (j & 1)] = (int32_t)(dw[j] & 0x0F0F0F0Fu);
        B[j >> 1][2 * (j & 1) + 1] = (int32_t)((dw[j] >> 4) & 0x0F0F0F0Fu);
        A[j >> 1][2 * (j & 1)] = use ? (int32_t)a.x : 0;
        A[j >> 1][2 * (j & 1) + 1] = use ? (int32_t)a.y : 0;
    }
    const i4_t zero = {0, 0, 0, 0};
    i4_t D = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[0], B[0], zero, 0, 0, 0);
    D = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[1], B[1], D, 0, 0, 0);
    // the lane's groups: 0..Q-1 on lanes h = 0, or h, h+2, h+4, h+6 on
    // lanes h < 2 when Q = 8; slot v of its scales and zero points
    if (Q == 8 ? h < 2 : h == 0) {
#pragma unroll
        for (int v = 0; v < NS; ++v) {
            const int grp = Q == 8 ? 2 * v + h : v;
            const int z = HAS_ZP ? (int)((r.zw >> (4 * v)) & 15u) : 8;
            const int dot = D[v] - z * qsum[c * Q + grp];
            acc = __builtin_fmaf((float)dot, raw_scale<ST, NS>(r.s, v), acc);
        }
    }
    return acc;
}

template <typename ST, int Q, bool HAS_ZP, int kBatch>
__global__ __launch_bounds__(kMaxWaves * 64) void acc4_gemv_kernel(Acc4Params p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    typedef Chunk<ST, Q> Regs;
    constexpr int G = kChunkK / Q;

    const int tid = threadIdx.x;
    const int bd = blockDim.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int nw = bd >> 6;
    const int h = lane >> 4;
    const int64_t t = blockIdx.x;
    const int C = p.C;
    const int kpad = C * kChunkK;
    const int nv = kpad / 4;      // 4-activation vectors, padding included
    const int nvk = p.K / 4;      // valid ones (K is a multiple of the group size)

    unsigned char* rec = smem;                                                  // [kpad] int8
    int32_t* qsum = reinterpret_cast<int32_t*>(smem + kpad);                    // [C*Q]
    float* red = reinterpret_cast<float*>(smem + kpad + C * Q * 4);             // [kMaxWaves*16]
    float* wmax = red + kMaxWaves * 16;                                         // [kMaxWaves]

    // 1. the thread's activation vectors, then the batch's scales and zero
    //    points, then its code words: all in flight before the first wait
    const f4_t* a4 = reinterpret_cast<const f4_t*>(p.a);
    f4_t av[kAV];
#pragma unroll
    for (int u = 0; u < kAV; ++u) {
        const int v = tid + u * bd;
        // workgroup-uniform test: only the vectors that exist are requested
        av[u] = (u == 0 || u * bd < nvk) ? a4[v < nvk ? v : 0] : f4_t{0.f, 0.f, 0.f, 0.f};
    }
    __builtin_amdgcn_sched_barrier(0);

    const int stride = nw * kBatch;
    auto load_batch = [&](Regs (&r)[kBatch], int cb) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            int c = cb + nw * u;
            c = c < C ? c : C - 1;
            load_meta<ST, Q, HAS_ZP>(p, t * C + c, lane, r[u]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            int c = cb + nw * u;
            c = c < C ? c : C - 1;
            load_codes<ST, Q>(p, t * C + c, lane, r[u]);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    Regs cur[kBatch];
    load_batch(cur, wave < C ? wave : 0);

    // 2. the row's maximum magnitude (NaN skipped, as fmaxf does), over the
    //    workgroup; every workgroup finds the same value
    float mx = 0.0f;
#pragma unroll
    for (int u = 0; u < kAV; ++u) {
        const int v = tid + u * bd;
        if (v < nvk) {
            mx = fmaxf(mx, fabsf(av[u].x));
            mx = fmaxf(mx, fabsf(av[u].y));
            mx = fmaxf(mx, fabsf(av[u].z));
            mx = fmaxf(mx, fabsf(av[u].w));
        }
    }
    for (int v = tid + kAV * bd; v < nvk; v += bd) {
        const f4_t x = a4[v];
        mx = fmaxf(fmaxf(mx, fabsf(x.x)), fmaxf(fabsf(x.y), fmaxf(fabsf(x.z), fabsf(x.w))));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) wmax[wave] = mx;
    block_sync_lds();
    mx = 0.0f;
    for (int ww = 0; ww < nw; ++ww) mx = fmaxf(mx, wmax[ww]);
    const float s = mx == 0.0f ? 0.0f : mx / 127.0f;     // correctly rounded division
    const float inv = s == 0.0f ? 0.0f : 1.0f / s;

    // 3. codes into LDS: a thread holds 4 consecutive activations; with its
    //    neighbour's 4 it forms the octet's record in the code words' byte
    //    order (k-offsets 0,4,1,5 | 2,6,3,7), and the lanes of a group sum
    //    their codes for the zero-point correction.  Past K everything is 0.
    const bool first_wg = blockIdx.x == 0;
    auto quant_vec = [&](int v, const f4_t& x) {
        uint32_t nat = 0;
        int qs = 0;
        if (v < nvk && s != 0.0f) {
            const int q0 = quant1(x.x, inv), q1 = quant1(x.y, inv);
            const int q2 = quant1(x.z, inv), q3 = quant1(x.w, inv);
            nat = (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) | ((uint32_t)(q2 & 255) << 16) |
                  ((uint32_t)(q3 & 255) << 24);
            qs = q0 + q1 + q2 + q3;
        }
        const uint32_t other = (uint32_t)__shfl_xor((int)nat, 1);
        if ((v & 1) == 0) {
            u2_t r2;
            r2.x = __builtin_amdgcn_perm(other, nat, 0x05010400u);
            r2.y = __builtin_amdgcn_perm(other, nat, 0x07030602u);
            reinterpret_cast<u2_t*>(rec)[v >> 1] = r2;
        }
#pragma unroll
        for (int off = 1; off < G / 4; off <<= 1) qs += __shfl_xor(qs, off);
        if ((v & (G / 4 - 1)) == 0) qsum[(4 * v) / G] = qs;
        if (first_wg && p.q_out && v < nvk) {
            typedef _Float16 hv4_t __attribute__((ext_vector_type(4)));
            hv4_t o;
            o[0] = (_Float16)(int8_t)(nat & 255u);
            o[1] = (_Float16)(int8_t)((nat >> 8) & 255u);
            o[2] = (_Float16)(int8_t)((nat >> 16) & 255u);
            o[3] = (_Float16)(int8_t)(nat >> 24);
            reinterpret_cast<hv4_t*>(p.q_out)[v] = o;
        }
    };
#pragma unroll
    for (int u = 0; u < kAV; ++u) {
        const int v = tid + u * bd;
        if (v < nv) quant_vec(v, av[u]);
    }
    for (int v = tid + kAV * bd; v < nv; v += bd) quant_vec(v, a4[v < nvk ? v : 0]);
    if (first_wg && p.s_out && tid == 0) p.s_out[0] = s;
    block_sync_lds();

    // 4. the chunks, a batch at a time, the next batch in flight
    const int row = lane & 15;
    float acc = 0.0f;
    auto compute_batch = [&](Regs (&r)[kBatch], int cb) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int c = cb + nw * u;
            if (c < C) acc = chunk_acc4<ST, Q, HAS_ZP>(r[u], rec, qsum, c, h, row, acc);
        }
    };
    if (wave + stride >= C) {
        if (wave < C) compute_batch(cur, wave);
    } else {
        // two register sets in turn, unconditional (clamped) loads: the
        // waits before each compute count only that batch's loads
        Regs alt[kBatch];
        for (int cb = wave; cb < C; cb += 2 * stride) {
            load_batch(alt, cb + stride);
            compute_batch(cur, cb);
            load_batch(cur, cb + 2 * stride);
            compute_batch(alt, cb + stride);
        }
    }

    // 5. lanes of a column, then waves, in a fixed order; the sum over the
    //    blocks times the activation scale, then the bias
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    if (h == 0) red[wave * 16 + lane] = acc;
    float bias_f = 0.0f;
    const int64_t n_out = t * kTileN + lane;
    if (p.bias && wave == 0 && lane < 16 && n_out < p.N) bias_f = p.bias[n_out];
    __syncthreads();
    if (wave == 0 && lane < 16 && n_out < p.N) {
        float total = 0.0f;
        for (int ww = 0; ww < nw; ++ww) total += red[ww * 16 + lane];
        float out = s != 0.0f ? total * s : 0.0f;
        if (p.bias) out = out + bias_f;
        p.y[n_out] = out;
    }
}

// M > 1: one workgroup per row.  The row's maximum, then its codes, written
// as fp16 integers (exact: |q| <= 127) for the fp16 matrix-core GEMMs.  A
// thread requests up to kQV of its row's 4-activation vectors at once and
// keeps them in registers, so the row is read once (longer rows read the
// rest again for the codes).
constexpr int kQuantThreads = 256;
constexpr int kQV = 8;

__global__ __launch_bounds__(kQuantThreads) void acc4_quantize_kernel(const float* __restrict__ a,
                                                                      _Float16* __restrict__ q,
                                                                      float* __restrict__ sc, int64_t K)
{
    __shared__ float wmax[kQuantThreads / 64];
    const int64_t m = blockIdx.x;
    const f4_t* row = reinterpret_cast<const f4_t*>(a + m * K);
    const int nvk = (int)(K / 4);
    const int tid = threadIdx.x;
    f4_t x[kQV];
#pragma unroll
    for (int u = 0; u < kQV; ++u) {
        const int v = tid + u * kQuantThreads;
        // workgroup-uniform test: only the vectors that exist are requested
        x[u] = (u == 0 || u * kQuantThreads < nvk) ? row[v < nvk ? v : 0] : f4_t{0.f, 0.f, 0.f, 0.f};
    }
    float mx = 0.0f;
#pragma unroll
    for (int u = 0; u < kQV; ++u) {
        if (tid + u * kQuantThreads < nvk)
            mx = fmaxf(fmaxf(mx, fabsf(x[u].x)), fmaxf(fabsf(x[u].y), fmaxf(fabsf(x[u].z), fabsf(x[u].w))));
    }
    for (int v = tid + kQV * kQuantThreads; v < nvk; v += kQuantThreads) {
        const f4_t y = row[v];
        mx = fmaxf(fmaxf(mx, fabsf(y.x)), fmaxf(fabsf(y.y), fmaxf(fabsf(y.z), fabsf(y.w))));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if ((tid & 63) == 0) wmax[tid >> 6] = mx;
    __syncthreads();
    mx = 0.0f;
#pragma unroll
    for (int w = 0; w < kQuantThreads / 64; ++w) mx = fmaxf(mx, wmax[w]);
    const float s = mx == 0.0f ? 0.0f : mx / 127.0f;     // correctly rounded division
    const float inv = s == 0.0f ? 0.0f : 1.0f / s;
    typedef _Float16 hv4_t __attribute__((ext_vector_type(4)));
    hv4_t* out = reinterpret_cast<hv4_t*>(q + m * K);
    auto codes4 = [&](const f4_t& y) {
        hv4_t o = {(_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};
        if (s != 0.0f) {
            o[0] = (_Float16)quant1(y.x, inv);
            o[1] = (_Float16)quant1(y.y, inv);
            o[2] = (_Float16)quant1(y.z, inv);
            o[3] = (_Float16)quant1(y.w, inv);
        }
        return o;
    };
#pragma unroll
    for (int u = 0; u < kQV; ++u) {
        const int v = tid + u * kQuantThreads;
        if (v < nvk) out[v] = codes4(x[u]);
    }
    for (int v = tid + kQV * kQuantThreads; v < nvk; v += kQuantThreads) out[v] = codes4(row[v]);
    if (tid == 0) sc[m] = s;
}

template <typename ST, int Q, bool HAS_ZP>
hipError_t launch_t(const Acc4Params& p, int waves, size_t smem, int64_t tiles, hipStream_t s)
{
    if (waves > kMaxWaves / 2)
        acc4_gemv_kernel<ST, Q, HAS_ZP, 2><<<dim3((unsigned)tiles), dim3(waves * 64), smem, s>>>(p);
    else
        acc4_gemv_kernel<ST, Q, HAS_ZP, 4><<<dim3((unsigned)tiles), dim3(waves * 64), smem, s>>>(p);
    return hipGetLastError();
}

template <typename ST, bool HAS_ZP>
hipError_t launch_q(const Layout& L, const Acc4Params& p, int waves, size_t smem, hipStream_t s)
{
    switch (L.Q) {
    case 1: return launch_t<ST, 1, HAS_ZP>(p, waves, smem, L.T, s);
    case 2: return launch_t<ST, 2, HAS_ZP>(p, waves, smem, L.T, s);
    case 4: return launch_t<ST, 4, HAS_ZP>(p, waves, smem, L.T, s);
    default: return launch_t<ST, 8, HAS_ZP>(p, waves, smem, L.T, s);
    }
}

}  // namespace

int64_t acc4_gemv_max_k() { return kMaxRecordBytes; }

hipError_t launch_acc4_quantize(const float* a, int64_t M, int64_t K, _Float16* q, float* s,
                                hipStream_t stream)
{
    acc4_quantize_kernel<<<dim3((unsigned)M), dim3(kQuantThreads), 0, stream>>>(a, q, s, K);
    return hipGetLastError();
}

hipError_t launch_acc4_gemv(const Layout& L, const WeightView& w, const float* a, const float* bias,
                            float* y, _Float16* q_out, float* s_out, hipStream_t stream,
                            const char** variant)
{
    Acc4Params p;
    p.codes = reinterpret_cast<const u4_t*>(w.codes);
    p.scales = w.scales;
    p.zp = w.zp;
    p.a = a;
    p.bias = bias;
    p.y = y;
    p.q_out = q_out;
    p.s_out = s_out;
    p.N = (int)L.N;
    p.K = (int)L.K;
    p.C = (int)L.C;
    const int max_waves = L.T * kMaxWaves <= kResidentWaves ? kMaxWaves : kMaxWaves / 2;
    int waves = (int)(L.C < max_waves ? L.C : max_waves);
    if (waves < 1) waves = 1;
    const size_t kpad = (size_t)L.C * kChunkK;
    const size_t smem = kpad + (size_t)L.C * L.Q * 4 + (kMaxWaves * 16 + kMaxWaves) * sizeof(float);
    if (variant) *variant = "gemv_accuracy4_i8";
    if (L.ss == 2)
        return L.has_zp ? launch_q<__half, true>(L, p, waves, smem, stream)
                        : launch_q<__half, false>(L, p, waves, smem, stream);
    return L.has_zp ? launch_q<float, true>(L, p, waves, smem, stream)
                    : launch_q<float, false>(L, p, waves, smem, stream);
}

}  // namespace mnb
