// gemv.hip -- decode GEMV (M = 1) and the fused gate/up + SwiGLU GEMV.
//
// Method: onnx-runtime-ep-cuda 0.1.0-dev.3, src/kernels/matmul_nbits.rs --
// the f32 GEMV (matmul_nbits_gemv_f32), the fp16 GEMVs (fp32 partial per
// block times its scale, lane reduction), the down-projection variant that
// stages the activation once in shared memory, and the paired gate/up GEMV
// with its SwiGLU epilogue (matmul_nbits_gemv_f16_gate_up_swiglu).
//
// gfx950 design: one workgroup per 16-column tile; its waves split the tile's
// 128-k chunks.  Each lane streams one 16-byte word per chunk (a wave reads
// a contiguous 1 KiB), unpacks nibbles to exact fp16 (c - z) in registers
// (already in the B-operand distribution of v_mfma_f32_16x16x32_f16), and
// the matrix cores multiply them with the activation staged once in LDS and
// reduce over k; each group's fp32 partial is scaled into an fp32 sum.  fp32
// activations take a VALU path with fp32 products instead.  Waves reduce
// through LDS in a fixed order (results are deterministic).  The store takes
// an optional bias in either rounding of matmul_nbits.rs fold_bias_f16.  For
// act-order weights (the g_idx input) the workgroup also gathers the staged
// activation into the codes' column order in LDS before computing.
#include <type_traits>

#include "mnb_device.hpp"
#include "mnb_internal.hpp"

namespace mnb {

namespace {

// Waves per workgroup and chunks per wave in flight: 16 x 2 when every
// workgroup of the grid fits on the chip at once with 16 waves, else 8 x 4
// (the same bytes in flight per workgroup, half the wave slots).
constexpr int kMaxWaves = 16;
constexpr int kResidentWaves = 256 * 32;   // CUs x wave slots per CU
// activation staging plus the wave reduction stay under the 64 KiB a
// workgroup gets without opt-in
constexpr int64_t kMaxStageBytes = 62 * 1024;

struct GemvWeight {
    const u4_t* codes;
    const void* scales;
    const uint8_t* zp;
};

struct GemvParams {
    GemvWeight w[2];
    const void* a;
    void* y;
    const void* bias;      // optional [N], the output's dtype
    int bias_after_round;
    const int32_t* perm;   // act order: column k of the product is a[perm[k]]
    int N, K, C;
};

template <int Q> struct LaneGroups {
    static constexpr int NS = Q >= 4 ? 4 : Q;   // scales a lane needs per chunk
    __device__ static int sidx(int j) { return Q == 1 ? 0 : (Q == 2 ? (j >> 1) : j); }
};

// A lane's scales of one chunk, loaded as one integer so the load stays a
// single instruction where it is written.
template <typename ST, int NS> struct ScaleVec;
template <> struct ScaleVec<__half, 1> { typedef uint16_t raw; };
template <> struct ScaleVec<__half, 2> { typedef uint32_t raw; };
template <> struct ScaleVec<__half, 4> { typedef uint64_t raw; };
template <> struct ScaleVec<float, 1> { typedef uint32_t raw; };
template <> struct ScaleVec<float, 2> { typedef uint64_t raw; };
template <> struct ScaleVec<float, 4> { typedef u4_t raw; };

template <typename ST, int NS>
__device__ __forceinline__ float scale_at(const typename ScaleVec<ST, NS>::raw& r, int s)
{
    if constexpr (sizeof(ST) == 2) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(r >> (16 * s)));
    } else if constexpr (NS == 4) {
        // element first, then the cast: this compiler's __builtin_bit_cast of
        // a vector subscript reads element 0 whatever the index
        const uint32_t e = r[s];
        return __builtin_bit_cast(float, e);
    } else {
        return __builtin_bit_cast(float, (uint32_t)(r >> (32 * s)));
    }
}

template <typename ST, int Q, bool HAS_ZP> struct ChunkRegs {
    static constexpr int NS = LaneGroups<Q>::NS;
    u4_t d;
    typename ScaleVec<ST, NS>::raw s;
    uint32_t zw;
};

// One tile's sections of a repacked weight as buffer resources: chunk c of
// the tile is at c times the chunk's record size, and a chunk past the tile's
// C chunks lies outside the range, where a buffer load returns zeros without
// a memory access.  So a wave's loads can be unconditional (all in flight at
// once) without reading any chunk twice.
struct TileRsrc {
    __amdgpu_buffer_rsrc_t codes, scales, zp;
};

template <typename ST, int Q>
__device__ __forceinline__ TileRsrc tile_rsrc(const GemvWeight& w, int64_t t, int C)
{
    constexpr int SREC = kTileN * Q * (int)sizeof(ST), ZREC = kTileN / 2 * Q;
    TileRsrc r;
    r.codes = __builtin_amdgcn_make_buffer_rsrc((void*)(w.codes + t * C * 64), (short)0, C * kChunkBytes,
                                                0x00020000);
    r.scales = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const uint8_t*>(w.scales) + t * C * SREC), (short)0, C * SREC, 0x00020000);
    r.zp = __builtin_amdgcn_make_buffer_rsrc((void*)(w.zp ? w.zp + t * C * ZREC : reinterpret_cast<const uint8_t*>(w.codes)), (short)0,
                                             w.zp ? C * ZREC : 0, 0x00020000);
    return r;
}

template <typename T> __device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, int voff, int soff);
template <> __device__ __forceinline__ uint16_t buf_load<uint16_t>(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
template <> __device__ __forceinline__ uint32_t buf_load<uint32_t>(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
template <> __device__ __forceinline__ uint64_t buf_load<uint64_t>(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
template <> __device__ __forceinline__ u4_t buf_load<u4_t>(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// The scales and zero points of chunk c of the tile (small loads, issued
// ahead of the code stream so that their wait does not cover the code loads).
template <typename ST, int Q, bool HAS_ZP>
__device__ __forceinline__ void load_meta(const TileRsrc& tr, int c, int lane, ChunkRegs<ST, Q, HAS_ZP>& r)
{
    constexpr int NS = LaneGroups<Q>::NS;
    typedef typename ScaleVec<ST, NS>::raw RawS;
    const int i = lane & 15, h = lane >> 4;
    const int sbase = Q <= 4 ? i * Q : ((h >> 1) * 16 + i) * 4;
    r.s = buf_load<RawS>(tr.scales, sbase * (int)sizeof(ST), c * (kTileN * Q * (int)sizeof(ST)));
    if (HAS_ZP) {
        const int zoff = c * (kTileN / 2 * Q);
        if (Q == 1) {
            r.zw = (__builtin_amdgcn_raw_buffer_load_b8(tr.zp, i >> 1, zoff, 0) >> (4 * (i & 1))) & 15u;
        } else if (Q == 2) {
            r.zw = __builtin_amdgcn_raw_buffer_load_b8(tr.zp, i, zoff, 0);
        } else {
            r.zw = buf_load<uint16_t>(tr.zp, sbase / 2, zoff);
        }
    } else {
        r.zw = 0;
    }
}

// Chunk c's code words: one 16-byte load per lane, a contiguous 1 KiB per
// wave, nontemporal (each word is read once).
template <typename ST, int Q, bool HAS_ZP>
__device__ __forceinline__ void load_codes(const TileRsrc& tr, int c, int lane, ChunkRegs<ST, Q, HAS_ZP>& r)
{
    r.d = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(tr.codes, lane * 16, c * kChunkBytes, 2));
}

// fp16 activations: the four 32-k steps of one chunk on the matrix cores.
// Every row of the v_mfma_f32_16x16x32_f16 A operand holds the same 8
// activations (each lane reads the slice of its k-octet), so all 16 output
// rows equal the column's partial sum over the step: the instruction does
// the k-reduction across lanes, and every lane ends with its column's sum.
// Each group's partial starts from zero and is scaled into the fp32 total
// once the group is complete.
__device__ __forceinline__ f4_t mfma16(const h8_t& a, const h8_t& b, const f4_t& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h8_t as_h8(const h2_t q[4])
{
    h8_t b;
    b[0] = q[0][0]; b[1] = q[0][1];
    b[2] = q[1][0]; b[3] = q[1][1];
    b[4] = q[2][0]; b[5] = q[2][1];
    b[6] = q[3][0]; b[7] = q[3][1];
    return b;
}

template <typename ST, int Q, bool HAS_ZP>
__device__ __forceinline__ float chunk_dot_f16(const ChunkRegs<ST, Q, HAS_ZP>& r,
                                               const _Float16* as, int c, int h, float acc)
{
    constexpr int NS = LaneGroups<Q>::NS;
    const uint32_t dw[4] = {r.d.x, r.d.y, r.d.z, r.d.w};
    const f4_t zero = {0.f, 0.f, 0.f, 0.f};
    if constexpr (Q <= 4) {
        // all four operands first, then one independent MFMA chain per
        // group, then the scales in group order: the chains overlap instead
        // of each waiting for the one before
        constexpr int steps = 4 / Q;   // k-steps per group
        h8_t b[4], a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int sj = LaneGroups<Q>::sidx(j);
            const uint32_t z = HAS_ZP ? (r.zw >> (4 * sj)) & 15u : 8u;
            h2_t q[4];
            unpack_zr(dw[j], zp_pair(z), q);
            b[j] = as_h8(q);
            a[j] = *reinterpret_cast<const h8_t*>(as + c * kChunkK + 32 * j + 8 * h);
        }
        f4_t grp[Q];
#pragma unroll
        for (int j = 0; j < 4; ++j) grp[j / steps] = mfma16(a[j], b[j], (j % steps == 0) ? zero : grp[j / steps]);
#pragma unroll
        for (int gq = 0; gq < Q; ++gq)
            acc = __builtin_fmaf(grp[gq][0], scale_at<ST, NS>(r.s, LaneGroups<Q>::sidx(gq * steps)), acc);
        return acc;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int sj = LaneGroups<Q>::sidx(j);
        const uint32_t z = HAS_ZP ? (r.zw >> (4 * sj)) & 15u : 8u;
        h2_t q[4];
        unpack_zr(dw[j], zp_pair(z), q);
        const h8_t b = as_h8(q);
        const h8_t a = *reinterpret_cast<const h8_t*>(as + c * kChunkK + 32 * j + 8 * h);
        {
            // group 16: octets 0,1 of the step are group 2j, octets 2,3 group
            // 2j+1; one MFMA per group with the other group's activation
            // octets zeroed (not its weights: an infinite activation times a
            // zeroed weight would put a NaN into the other group).  A lane's
            // scale vector holds the groups of its own octet half (h >> 1),
            // so the other half's scale comes from the lane 32 positions
            // away.
            h8_t zh;
#pragma unroll
            for (int e = 0; e < 8; ++e) zh[e] = (_Float16)0.0f;
            const f4_t ge = mfma16((h < 2) ? a : zh, b, zero);
            const f4_t go = mfma16((h < 2) ? zh : a, b, zero);
            const float s_own = scale_at<ST, NS>(r.s, sj);
            const float s_other = __shfl_xor(s_own, 32);
            const float se = (h < 2) ? s_own : s_other;
            const float so = (h < 2) ? s_other : s_own;
            acc = __builtin_fmaf(ge[0], se, acc);
            acc = __builtin_fmaf(go[0], so, acc);
        }
    }
    return acc;
}

// fp32 activations: the same word, products in fp32.  Lanes L, L^16, L^32,
// L^48 hold parts of the same column; they are summed after the chunks.
template <typename ST, int Q, bool HAS_ZP>
__device__ __forceinline__ float chunk_dot_f32(const ChunkRegs<ST, Q, HAS_ZP>& r, const float* as,
                                               int c, int h, float acc)
{
    constexpr int NS = LaneGroups<Q>::NS;
    const uint32_t dw[4] = {r.d.x, r.d.y, r.d.z, r.d.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int sj = LaneGroups<Q>::sidx(j);
        const float zf = HAS_ZP ? (float)((r.zw >> (4 * sj)) & 15u) : 8.0f;
        const float* ap = as + c * kChunkK + 32 * j + 8 * h;
        const f4_t a0 = *reinterpret_cast<const f4_t*>(ap);
        const f4_t a1 = *reinterpret_cast<const f4_t*>(ap + 4);
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            part = __builtin_fmaf(av[e], (float)code_at(dw[j], e) - zf, part);
        }
        acc = __builtin_fmaf(part, scale_at<ST, NS>(r.s, sj), acc);
    }
    return acc;
}

__device__ __forceinline__ float silu_f32(float x) { return x / (1.0f + __expf(-x)); }

typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

// LDS behind the staged activation: the per-wave partials of both outputs
constexpr int kRedBytes = 2 * kMaxWaves * 16 * sizeof(float);
// act order: index vectors (4 columns each) a thread requests up front
constexpr int kPermPre = 4;

// LDS bytes of the staged activation: a slot of kBatch chunks per wave
// (WAVE_STAGE), or the whole activation padded to whole chunks.  The wave
// partials follow it (kRedBytes), then, for act order, the gathered copy.
template <typename AT, int kBatch, bool WAVE_STAGE>
__host__ __device__ inline size_t stage_bytes(int waves, int C)
{
    return WAVE_STAGE ? (size_t)waves * kBatch * kChunkK * sizeof(AT) : (size_t)C * kChunkK * sizeof(AT);
}

// kBatch chunks per wave are in flight together.  LOOP = false: every chunk of
// the tile fits in one batch per wave (waves * kBatch >= C), so the kernel is
// straight-line code holding one register set; LOOP = true: batches alternate
// between two register sets.
template <typename AT, typename ST, int Q, bool HAS_ZP, bool FUSED, int kBatch, bool PERM, bool LOOP>
//
// The arguments are scalars in the order the kernel first needs them (the
// weight's codes, scales and zero points, A, Y, the sizes and the wave
// count), not one structure: built with kernarg preloading
// (-amdgpu-kernarg-preload-count), the first 16 dwords arrive in SGPRs when
// the wave starts, so the first loads are issued without waiting on a
// scalar load of the argument block.  The rest are loaded when used.
__global__ __launch_bounds__(kMaxWaves * 64) void gemv_kernel(
    const u4_t* codes0, const void* scales0, const uint8_t* zp0, const void* a, void* y, int N, int K, int C,
    int nw, const u4_t* codes1, const void* scales1, const uint8_t* zp1, const void* bias, int bias_after_round,
    const int32_t* perm)
{
    GemvParams p;
    p.w[0] = GemvWeight{codes0, scales0, zp0};
    p.w[1] = GemvWeight{codes1, scales1, zp1};
    p.a = a;
    p.y = y;
    p.bias = bias;
    p.bias_after_round = bias_after_round;
    p.perm = perm;
    p.N = N;
    p.K = K;
    p.C = C;
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr bool F16 = sizeof(AT) == 2;
    constexpr bool WAVE_STAGE = !LOOP && !PERM;
    constexpr int NW = FUSED ? 2 : 1;
    typedef ChunkRegs<ST, Q, HAS_ZP> Regs;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int h = lane >> 4;
    const int64_t t = blockIdx.x;
    const int64_t kpad = (int64_t)C * kChunkK;

    // Issue order of a wave: its first activation vector, then the scales
    // and zero points of its batch, then the batch's code words.  Waits
    // count completions in issue order, so the small loads never wait behind
    // the code stream, and chunk u is computed as soon as its own code word
    // is in while the later ones are still streaming.

    // 0. act order: the thread's first column indices, four per vector
    //    (K is a whole number of groups, so a multiple of 4)
    const int nq = p.K / 4;
    const int nq_pad = (int)(kpad / 4);
    const u4_t* perm_vec = reinterpret_cast<const u4_t*>(p.perm);
    u4_t pidx[kPermPre];
    if constexpr (PERM) {
#pragma unroll
        for (int j = 0; j < kPermPre; ++j) {
            const int v = tid + j * (nw * 64);
            // workgroup-uniform test: only the vectors that exist are requested
            pidx[j] = (j == 0 || j * (nw * 64) < nq) ? perm_vec[v < nq ? v : 0] : u4_t{0u, 0u, 0u, 0u};
        }
    }

    // 1. the activation.  WAVE_STAGE: this wave's own slices of it (the 128
    //    k of each of its chunks), requested first; else the thread's first
    //    16-byte vector of the whole activation, staged for the workgroup.
    constexpr int kPerVec = 16 / sizeof(AT);
    const int nvec = (int)(kpad / kPerVec);
    const int nvec_valid = p.K / kPerVec;
    const u4_t* a_vec = static_cast<const u4_t*>(p.a);
    u4_t* s_vec = reinterpret_cast<u4_t*>(smem);
    constexpr int kVecPerChunk = kChunkK / kPerVec;                  // 16 (fp16) or 32 (fp32)
    constexpr int kWaveVecs = (kBatch * kVecPerChunk + 63) / 64;      // per lane
    u4_t own[WAVE_STAGE ? kWaveVecs : 1];
    u4_t first = u4_t{0u, 0u, 0u, 0u};
    if constexpr (WAVE_STAGE) {
#pragma unroll
        for (int i = 0; i < kWaveVecs; ++i) {
            const int v = lane + 64 * i;
            const int u = v / kVecPerChunk, e = v % kVecPerChunk;
            const int c = wave + nw * u;
            // K is a whole number of groups, so a vector is all inside or all
            // outside the activation
            const int kv = c * kVecPerChunk + e;
            own[i] = (u < kBatch && c < C && kv < nvec_valid) ? a_vec[kv] : u4_t{0u, 0u, 0u, 0u};
        }
    } else {
        first = a_vec[tid < nvec_valid ? tid : 0];   // zeroed at the store
    }
    __builtin_amdgcn_sched_barrier(0);

    float acc[NW];
#pragma unroll
    for (int x = 0; x < NW; ++x) acc[x] = 0.0f;

    // 2. the wave's chunks c = wave + nw*u, a batch of kBatch at a time.
    //    A batch's loads are unconditional and all in flight together (a
    //    chunk past the tile reads zeros without a memory access); the
    //    compute is guarded instead.
    const int stride = nw * kBatch;
    TileRsrc tr[NW];
#pragma unroll
    for (int x = 0; x < NW; ++x) tr[x] = tile_rsrc<ST, Q>(p.w[x], t, C);
    auto load_batch = [&](Regs (&r)[NW][kBatch], int cb) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
#pragma unroll
            for (int x = 0; x < NW; ++x) load_meta<ST, Q, HAS_ZP>(tr[x], cb + nw * u, lane, r[x][u]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
#pragma unroll
            for (int x = 0; x < NW; ++x) load_codes<ST, Q, HAS_ZP>(tr[x], cb + nw * u, lane, r[x][u]);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    Regs cur[NW][kBatch];
    load_batch(cur, wave);

    // 3. stage the activation in LDS (zero beyond K) while the codes stream
    //    in.  WAVE_STAGE: each wave writes its slices to a slot of its own and
    //    reads only those, so no workgroup barrier stands between a wave and
    //    its compute (a barrier here would hold every wave until the slowest
    //    had issued its loads, which stalls under a full memory queue).
    const unsigned char* act = smem;
    if constexpr (WAVE_STAGE) {
        u4_t* slot = s_vec + wave * (kBatch * kVecPerChunk);
#pragma unroll
        for (int i = 0; i < kWaveVecs; ++i) {
            const int v = lane + 64 * i;
            if (v < kBatch * kVecPerChunk) slot[v] = own[i];
        }
        // the wave's own LDS writes complete before its reads (in order);
        // this keeps the compiler from moving the reads above them
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        act = reinterpret_cast<const unsigned char*>(slot);
    } else {
        if (tid < nvec) s_vec[tid] = tid < nvec_valid ? first : u4_t{0u, 0u, 0u, 0u};
        for (int v = tid + nw * 64; v < nvec; v += nw * 64)
            s_vec[v] = v < nvec_valid ? a_vec[v] : u4_t{0u, 0u, 0u, 0u};
        block_sync_lds();
    }

    // 3b. act order: gather the staged activation into the codes' column
    //     order, behind the reduction area (an index outside 0..K-1 reads
    //     column 0; columns past K stay zero)
    if constexpr (PERM) {
        typedef typename std::conditional<F16, uint16_t, uint32_t>::type RT;
        typedef typename std::conditional<F16, u2_t, u4_t>::type VT;
        const RT* src = reinterpret_cast<const RT*>(smem);
        unsigned char* dst = smem + kpad * sizeof(AT) + kRedBytes;
        auto gather4 = [&](int v, const u4_t& ix) {
            RT o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t k = ix[i] < (uint32_t)p.K ? ix[i] : 0u;
                o[i] = v < nq ? src[k] : RT(0);
            }
            VT ov;
            __builtin_memcpy(&ov, o, sizeof(ov));
            reinterpret_cast<VT*>(dst)[v] = ov;
        };
#pragma unroll
        for (int j = 0; j < kPermPre; ++j) {
            const int v = tid + j * (nw * 64);
            if (v < nq_pad) gather4(v, pidx[j]);
        }
        for (int v = tid + kPermPre * (nw * 64); v < nq_pad; v += nw * 64)
            gather4(v, perm_vec[v < nq ? v : 0]);
        block_sync_lds();
        act = dst;
    }

    // 4. compute a batch while the next one is in flight
    auto compute_batch = [&](Regs (&r)[NW][kBatch], int cb) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int c = cb + nw * u;
            // the activation of chunk c: in the wave's slot (slot chunk u) or
            // in the workgroup's copy (chunk c)
            const int ca = WAVE_STAGE ? u : c;
            if (c < C) {
#pragma unroll
                for (int x = 0; x < NW; ++x) {
                    if (F16)
                        acc[x] = chunk_dot_f16<ST, Q, HAS_ZP>(
                            r[x][u], reinterpret_cast<const _Float16*>(act), ca, h, acc[x]);
                    else
                        acc[x] = chunk_dot_f32<ST, Q, HAS_ZP>(
                            r[x][u], reinterpret_cast<const float*>(act), ca, h, acc[x]);
                }
            }
        }
    };
    if (!LOOP || wave + stride >= C) {
        // one batch per wave (the common decode shapes): straight-line code
        if (wave < C) compute_batch(cur, wave);
    } else if constexpr (LOOP) {
        // two register sets in turn, the loop unrolled by two: the next
        // batch is requested before the current one is computed, and no
        // registers are copied, so the waits at the top of each compute count
        // only that batch's loads (a copy at the back edge would make them
        // wait for everything in flight).  The loads are unconditional
        // (chunks past the end read zeros, and the compute skips them), so
        // every path has the same loads in flight.
        Regs alt[NW][kBatch];
        for (int cb = wave; cb < C; cb += 2 * stride) {
            load_batch(alt, cb + stride);
            compute_batch(cur, cb);
            load_batch(cur, cb + 2 * stride);
            compute_batch(alt, cb + stride);
        }
    }

    // 5. every lane now holds its column's partial (the fp32 path after its
    //    lane sum), and every lane stores it: the four lanes of a column write
    //    the same value, so no part of the computation is confined to some
    //    lanes (where the compiler would sink the scale loads behind it).
    if (!F16) {
#pragma unroll
        for (int x = 0; x < NW; ++x) {
            acc[x] += __shfl_xor(acc[x], 16);
            acc[x] += __shfl_xor(acc[x], 32);
        }
    }
    float* red = reinterpret_cast<float*>(smem + stage_bytes<AT, kBatch, WAVE_STAGE>(nw, C));
#pragma unroll
    for (int x = 0; x < NW; ++x) red[(x * kMaxWaves + wave) * 16 + (lane & 15)] = acc[x];
    // the store's bias, requested before the barrier so that its latency
    // overlaps the wait for the other waves and their reduction
    float bias_f = 0.0f;
    const int64_t n_out = t * kTileN + lane;
    if (!FUSED && p.bias && wave == 0 && lane < 16 && n_out < p.N)
        bias_f = (float)static_cast<const AT*>(p.bias)[n_out];
    __syncthreads();
    if (wave == 0 && lane < 16) {
        float r[NW];
#pragma unroll
        for (int x = 0; x < NW; ++x) {
            r[x] = 0.0f;
            // the common wave counts unrolled: every read in flight at once,
            // then the same sum in the same order
            auto sum_all = [&](auto n_c) __attribute__((always_inline)) {
                constexpr int NWV = decltype(n_c)::value;
                float pv[NWV];
#pragma unroll
                for (int ww = 0; ww < NWV; ++ww) pv[ww] = red[(x * kMaxWaves + ww) * 16 + lane];
#pragma unroll
                for (int ww = 0; ww < NWV; ++ww) r[x] += pv[ww];
            };
            if (nw == kMaxWaves)
                sum_all(std::integral_constant<int, kMaxWaves>());
            else if (nw == kMaxWaves / 2)
                sum_all(std::integral_constant<int, kMaxWaves / 2>());
            else
                for (int ww = 0; ww < nw; ++ww) r[x] += red[(x * kMaxWaves + ww) * 16 + lane];
        }
        const int64_t n = t * kTileN + lane;
        if (n < p.N) {
            float out = r[0];
            if (FUSED) out = silu_f32(r[0]) * r[NW - 1];
            AT v;
            if constexpr (F16)
                v = (!FUSED && p.bias) ? finish_value(out, bias_f, p.bias_after_round) : __float2half_rn(out);
            else
                v = (!FUSED && p.bias) ? out + bias_f : out;
            static_cast<AT*>(p.y)[n] = v;
        }
    }
}

// Chunks per wave: when the tile's C chunks fit in one batch of at most
// kMaxBatch per wave, the smallest batch size of {1, 2, 4} that covers them
// (every load of the wave in flight before its first wait, one register set);
// else the two-set loop with batches of 2 (16 waves, or the fused pair) or 4
// (a single weight on 8 waves).  The fused pair's two weights in batches of 4
// outgrow the 128 registers the 16-wave launch bound leaves a wave and spill
// inside the loop; in batches of 2 it is 9-13% faster (K = 5120, N = 13824
// and K = 8192, N = 28672, same bits).  Larger
// single batches (6 or 8 chunks in flight per wave) measured slower: the
// loads finish sooner, but every chunk of a wave then lands near the end of
// the stream and the unpack work runs after it instead of beside it.
constexpr int kMaxBatch = 4;

template <typename AT, typename ST, int Q, bool HAS_ZP, bool FUSED, int B, bool PERM, bool LOOP>
void launch_k(const GemvParams& p, int waves, int64_t tiles, hipStream_t s)
{
    constexpr bool WAVE_STAGE = !LOOP && !PERM;
    const size_t stage = stage_bytes<AT, B, WAVE_STAGE>(waves, p.C);
    const size_t smem = stage + kRedBytes + (PERM ? stage : 0);
    gemv_kernel<AT, ST, Q, HAS_ZP, FUSED, B, PERM, LOOP><<<dim3((unsigned)tiles), dim3(waves * 64), smem, s>>>(
        p.w[0].codes, p.w[0].scales, p.w[0].zp, p.a, p.y, p.N, p.K, p.C, waves, p.w[1].codes, p.w[1].scales,
        p.w[1].zp, p.bias, p.bias_after_round, p.perm);
}

template <typename AT, typename ST, int Q, bool HAS_ZP, bool FUSED, bool PERM>
hipError_t launch_b(const GemvParams& p, int waves, int64_t tiles, hipStream_t s)
{
    const int per_wave = (p.C + waves - 1) / waves;
    if (per_wave <= 1)
        launch_k<AT, ST, Q, HAS_ZP, FUSED, 1, PERM, false>(p, waves, tiles, s);
    else if (per_wave <= 2)
        launch_k<AT, ST, Q, HAS_ZP, FUSED, 2, PERM, false>(p, waves, tiles, s);
    else if (per_wave <= kMaxBatch)
        launch_k<AT, ST, Q, HAS_ZP, FUSED, kMaxBatch, PERM, false>(p, waves, tiles, s);
    else if (waves > kMaxWaves / 2 || FUSED)
        launch_k<AT, ST, Q, HAS_ZP, FUSED, 2, PERM, true>(p, waves, tiles, s);
    else if constexpr (!FUSED)
        launch_k<AT, ST, Q, HAS_ZP, FUSED, 4, PERM, true>(p, waves, tiles, s);
    return hipGetLastError();
}

template <typename AT, typename ST, int Q, bool HAS_ZP, bool FUSED>
hipError_t launch_t(const GemvParams& p, int waves, int64_t tiles, hipStream_t s)
{
    // act order comes without the fused gate/up form
    if constexpr (!FUSED)
        if (p.perm) return launch_b<AT, ST, Q, HAS_ZP, false, true>(p, waves, tiles, s);
    return launch_b<AT, ST, Q, HAS_ZP, FUSED, false>(p, waves, tiles, s);
}

template <typename AT, typename ST, bool HAS_ZP, bool FUSED>
hipError_t launch_q(const Layout& L, const GemvParams& p, int waves, hipStream_t s)
{
    switch (L.Q) {
    case 1: return launch_t<AT, ST, 1, HAS_ZP, FUSED>(p, waves, L.T, s);
    case 2: return launch_t<AT, ST, 2, HAS_ZP, FUSED>(p, waves, L.T, s);
    case 4: return launch_t<AT, ST, 4, HAS_ZP, FUSED>(p, waves, L.T, s);
    default: return launch_t<AT, ST, 8, HAS_ZP, FUSED>(p, waves, L.T, s);
    }
}

template <typename AT, bool FUSED>
hipError_t launch_a(const Layout& L, const GemvParams& p, int waves, hipStream_t s)
{
    if (L.ss == 2) {
        return L.has_zp ? launch_q<AT, __half, true, FUSED>(L, p, waves, s)
                        : launch_q<AT, __half, false, FUSED>(L, p, waves, s);
    }
    return L.has_zp ? launch_q<AT, float, true, FUSED>(L, p, waves, s)
                    : launch_q<AT, float, false, FUSED>(L, p, waves, s);
}

GemvWeight gw(const WeightView& v)
{
    return GemvWeight{reinterpret_cast<const u4_t*>(v.codes), v.scales, v.zp};
}

}  // namespace

int64_t gemv_max_k(bool f16_act, bool act_order)
{
    return kMaxStageBytes / (act_order ? 2 : 1) / (f16_act ? 2 : 4) / kChunkK * kChunkK;
}

hipError_t launch_gemv(const Layout& L, const WeightView& gate, const WeightView* up,
                       const void* a, const int32_t* perm, bool f16_act, const Bias& bias, void* y,
                       hipStream_t stream, const char** variant)
{
    GemvParams p;
    p.w[0] = gw(gate);
    p.w[1] = up ? gw(*up) : gw(gate);
    p.a = a;
    p.y = y;
    p.bias = bias.ptr;
    p.bias_after_round = bias.after_round;
    p.perm = up ? nullptr : perm;
    p.N = (int)L.N;
    p.K = (int)L.K;
    p.C = (int)L.C;
    const int max_waves = L.T * kMaxWaves <= kResidentWaves ? kMaxWaves : kMaxWaves / 2;
    int waves = (int)(L.C < max_waves ? L.C : max_waves);
    if (waves < 1) waves = 1;
    const bool fused = up != nullptr;
    if (variant) *variant = fused ? (f16_act ? "gemv_gate_up_swiglu_f16" : "gemv_gate_up_swiglu_f32")
                          : p.perm ? (f16_act ? "gemv_act_order_f16" : "gemv_act_order_f32")
                                   : (f16_act ? "gemv_f16" : "gemv_f32");
    if (f16_act) {
        return fused ? launch_a<__half, true>(L, p, waves, stream)
                     : launch_a<__half, false>(L, p, waves, stream);
    }
    return fused ? launch_a<float, true>(L, p, waves, stream)
                 : launch_a<float, false>(L, p, waves, stream);
}

}  // namespace mnb
