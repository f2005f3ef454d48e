// gemm_mfma.hip -- prefill GEMM (M > 16) on the gfx950 matrix cores.
//
// Method: onnx-runtime-ep-cuda 0.1.0-dev.6, src/kernels/marlin_gemm.rs
// (matmul_nbits_marlin_gemm_f16 and its module doc): weights enter the matrix
// multiply centred but unscaled, as exact fp16 (code - zp); each group's
// products accumulate in fp32 from zero and the group's scale multiplies that
// partial after the group's accumulate, so the accumulator never carries a
// scale that varies along K.
//
// gfx950 design.
// * v_mfma_f32_32x32x16_f16 (32x32 output, 16 k): it reaches the matrix
//   cores' full rate from one wave per SIMD, which the 16x16x32 shape does not.
// * Workgroup tile 128 (M) x 256 (N), 4 waves, one per SIMD; each wave owns
//   all 128 rows and 64 columns: 4 row blocks x 2 column pairs of 32x32
//   tiles.
// * Every operand of a 128-k chunk -- the A rows, the wave's four 1 KiB code
//   word blocks, and the scales and zero points of its tiles -- is copied
//   into LDS by buffer_load ... lds (no VGPR round trip) into a ring of
//   stages, ahead of the compute.  Rows and k outside the operand read as
//   zero through the buffer range check.  A's 16-byte segments are
//   XOR-swizzled by row, so fragment reads are bank-conflict free.
// * The repacked layout distributes a 16-column tile over the 64 lanes as 16
//   columns x 4 k-octets; two v_permlane*_swap instructions on the raw words
//   of two adjacent tiles give the 32 columns x 2 k-octets of the 32x32x16 B
//   operand before the unpack.
// * Each group accumulates from zero into one set of 32x32 accumulators; at
//   the group's end they are multiplied by the group's scales into the fp32
//   running total.
// * Workgroup ids are remapped so the tiles resident on one XCD at a time
//   share A rows and B columns in that XCD's L2.
#include "mnb_device.hpp"
#include "mnb_internal.hpp"

namespace mnb {

namespace {

constexpr int BM = 96;             // rows per workgroup
constexpr int BN = 256;            // columns per workgroup (16 tiles of 16)
constexpr int WAVES = 4;           // one per SIMD; wave w owns columns [64w, 64w+64)
constexpr int RB = BM / 32;        // 32-row blocks per wave
constexpr int PAIRS = 2;           // 32-column pairs of tiles per wave
constexpr int TPW = 2 * PAIRS;     // 16-column tiles per wave
constexpr int SEGS = kChunkK / 8;  // 16-byte segments per A row per chunk
constexpr int kGroupM = 4;         // m-blocks per XCD-local band
constexpr int kLdsBudget = 160 * 1024;
constexpr int ROWS_PER_WAVE = BM / WAVES;   // A rows each wave copies per chunk
constexpr int A_DMA = ROWS_PER_WAVE / 4;    // 1 KiB (4-row) DMAs per wave per chunk

typedef float f16v_t __attribute__((ext_vector_type(16)));

struct GemmParams {
    const uint8_t* w;      // repacked weight base
    int64_t scales_off, zp_off;
    uint32_t w_bytes;      // repacked size (buffer range)
    const _Float16* a;
    __half* y;
    int M, N, K, C;
    int T;                 // column tiles
    int num_m, num_n;      // workgroup grid
};

// LDS geometry of one pipeline stage for (Q, scale bytes, zero points).
template <int Q, int SS, bool HAS_ZP> struct StageGeom {
    static constexpr int kScaleDw = kTileN * Q * SS / 4;               // dwords per tile record
    static constexpr int kZpDw = HAS_ZP ? kTileN * Q / 8 : 0;          // 8Q bytes per tile record
    static constexpr int kMetaDw = TPW * (kScaleDw + kZpDw);           // per wave
    static constexpr int kMetaInstr = (kMetaDw + 63) / 64;             // dword DMAs per wave
    static constexpr int kMetaDwPad = kMetaInstr * 64;
    static constexpr int kA = BM * SEGS * 16;                          // bytes
    static constexpr int kB = WAVES * TPW * 1024;
    static constexpr int kMeta = WAVES * kMetaDwPad * 4;
    static constexpr int kBytes = kA + kB + kMeta;
    static constexpr int kStages = 3 * kBytes <= kLdsBudget ? 3 : 2;
    static constexpr int kDmaPerChunk = A_DMA + TPW + kMetaInstr;      // per wave
};

__device__ __forceinline__ f16v_t mfma32(const h8_t& a, const h8_t& b, const f16v_t& c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
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

// LDS destination pointers of buffer_load ... lds.  (Cast inline: a
// __device__ helper called from the kernel's lambdas would suppress the
// kernel's host-side launch stub.)
typedef void __attribute__((address_space(3))) * lds_ptr_t;

// Wait until at most N vector-memory operations of this wave are
// outstanding (gfx9 s_waitcnt encoding; expcnt and lgkmcnt left open).
template <int N> __device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup id -> (m-block, n-block).  Consecutive ids go to different XCDs
// (round-robin dispatch), so ids are first regrouped per XCD; within an XCD,
// tiles are ordered in bands of kGroupM m-blocks so the ~32 tiles resident at
// a time span few A rows and few B columns.
__device__ __forceinline__ void tile_of(int bid, int num_m, int num_n, int& mb, int& nb)
{
    const int total = num_m * num_n;
    constexpr int XCDS = 8;
    int g = bid;
    if (total % XCDS == 0) {
        const int per = total / XCDS;
        g = (bid % XCDS) * per + bid / XCDS;
    }
    const int in_group = kGroupM * num_n;
    const int group = g / in_group;
    const int first_m = group * kGroupM;
    const int gm = (num_m - first_m) < kGroupM ? (num_m - first_m) : kGroupM;
    const int r = g - group * in_group;
    mb = first_m + r % gm;
    nb = r / gm;
}

template <typename ST, int Q, bool HAS_ZP> struct KernelLds {
    typedef StageGeom<Q, (int)sizeof(ST), HAS_ZP> G;
    static constexpr int kBytes = G::kStages * G::kBytes;
};

template <typename ST, int Q, bool HAS_ZP>
__global__ __launch_bounds__(WAVES * 64, 1) void gemm_mfma_kernel(GemmParams p)
{
    typedef StageGeom<Q, (int)sizeof(ST), HAS_ZP> G;
    constexpr int NST = G::kStages;
    __shared__ __align__(16) unsigned char lds[KernelLds<ST, Q, HAS_ZP>::kBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int i = lane & 15;
    const int half = (lane >> 4) & 1;   // which tile of a pair holds this lane's column
    const int oct = lane >> 5;          // k-octet of a 16-k step (A and B operands)
    int mb, nb;
    tile_of(blockIdx.x, p.num_m, p.num_n, mb, nb);
    const int m0 = mb * BM;
    const int C = p.C;
    const int K = p.K;

    auto stage_a = [&](int st) { return reinterpret_cast<u4_t*>(lds + st * G::kBytes); };
    auto stage_b = [&](int st) { return reinterpret_cast<uint32_t*>(lds + st * G::kBytes + G::kA); };
    auto stage_m = [&](int st) {
        return reinterpret_cast<unsigned char*>(lds + st * G::kBytes + G::kA + G::kB) +
               wave * G::kMetaDwPad * 4;
    };

    // ---- DMA sources ------------------------------------------------------
    // A: rows m0 .. m0+BM as a buffer that ends at the last valid row, so
    // rows >= M read zero; k >= K uses an offset past the range.
    const int rows_here = (p.M - m0) < BM ? (p.M - m0) : BM;
    const uint32_t a_bytes = (uint32_t)rows_here * (uint32_t)K * 2u;
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.a + (int64_t)m0 * K), (short)0, (int)a_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t w_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.w, (short)0, (int)p.w_bytes, 0x00020000);

    // this wave's 4 tiles (clamped for loads; stores are masked by N)
    uint32_t tile_chunk0[TPW];   // chunk index of (tile, chunk 0)
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        int t = nb * (BN / 16) + wave * TPW + tt;
        if (t >= p.T) t = p.T - 1;
        tile_chunk0[tt] = (uint32_t)t * (uint32_t)C;
    }

    auto issue_chunk = [&](int c, int st) {
        // A rows [ROWS_PER_WAVE*wave, +ROWS_PER_WAVE): DMAs of 4 rows each
#pragma unroll
        for (int b = 0; b < A_DMA; ++b) {
            const int r = ROWS_PER_WAVE * wave + 4 * b + (lane >> 4);
            const int sg = (lane & 15) ^ (r & 15);          // logical segment at this slot
            const int k = c * kChunkK + 8 * sg;
            const uint32_t off = k < K ? ((uint32_t)r * (uint32_t)K + (uint32_t)k) * 2u : a_bytes;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr_t)(stage_a(st) + (ROWS_PER_WAVE * wave + 4 * b) * SEGS),
                                                     16, off, 0, 0, 0);
        }
        // code words: one 1 KiB block per tile
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const uint32_t off = (tile_chunk0[tt] + (uint32_t)c) * 1024u + (uint32_t)lane * 16u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (lds_ptr_t)(stage_b(st) + (wave * TPW + tt) * 256),
                                                     16, off, 0, 0, 0);
        }
        // scale records, then zero-point records, of the 4 tiles (dwords)
#pragma unroll
        for (int m = 0; m < G::kMetaInstr; ++m) {
            int d = m * 64 + lane;
            uint32_t off;
            if (d < TPW * G::kScaleDw) {
                const int tt = d / G::kScaleDw, o = d % G::kScaleDw;
                off = (uint32_t)p.scales_off + (tile_chunk0[tt] + (uint32_t)c) * (uint32_t)(G::kScaleDw * 4) + o * 4;
            } else if (HAS_ZP && d < G::kMetaDw) {
                constexpr int ZD = G::kZpDw > 0 ? G::kZpDw : 1;
                d -= TPW * G::kScaleDw;
                const int tt = d / ZD, o = d % ZD;
                off = (uint32_t)p.zp_off + (tile_chunk0[tt] + (uint32_t)c) * (uint32_t)(ZD * 4) + o * 4;
            } else {
                off = p.w_bytes;   // padding lanes read zero
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (lds_ptr_t)(stage_m(st) + m * 256), 4, off, 0, 0, 0);
        }
    };

    // ---- accumulators -----------------------------------------------------
    f16v_t total[RB][PAIRS];
    f16v_t grp[RB][PAIRS];
    f16v_t zero;
#pragma unroll
    for (int e = 0; e < 16; ++e) zero[e] = 0.f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
            total[rb][q] = zero;
            grp[rb][q] = zero;
        }

    constexpr int HS_PER_GROUP = 8 / Q;          // 16-k steps per group (group = 128/Q)

    // one 128-k chunk from stage st
    auto chunk = [&](int st) {
        const u4_t* As = stage_a(st);
        const uint32_t* Bs = stage_b(st) + wave * TPW * 256;
        const unsigned char* Ms = stage_m(st);
        // this lane's column lives in tile 2q + half of pair q
        float sc[PAIRS][Q];
        uint32_t zc[PAIRS][Q];
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
            const int tt = 2 * q + half;
            const ST* srec = reinterpret_cast<const ST*>(Ms + tt * G::kScaleDw * 4);
#pragma unroll
            for (int g = 0; g < Q; ++g) {
                const int s = slot_of(i, g, Q);
                sc[q][g] = to_f32(srec[s]);
                if (HAS_ZP) {
                    const unsigned char* zrec = Ms + (TPW * G::kScaleDw + tt * G::kZpDw) * 4;
                    zc[q][g] = (zrec[s >> 1] >> (4 * (s & 1))) & 15u;
                } else {
                    zc[q][g] = 8u;
                }
            }
        }
        // A fragments of 16-k step hs: row (rb*32 + lane%32), k-octet oct;
        // the XOR swizzle term depends on the lane only (rb*32 is a multiple
        // of 16), so rows of different blocks differ by a constant offset.
        auto load_afr = [&](h8_t (&afr)[RB], int hs) {
            const int sgi = (2 * hs + oct) ^ (lane & 15);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                afr[rb] = __builtin_bit_cast(h8_t, As[(rb * 32 + (lane & 31)) * SEGS + sgi]);
        };
        // raw code words of 32-k step j for the wave's 4 tiles
        auto load_words = [&](uint32_t (&w)[TPW], int j) {
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) w[tt] = Bs[tt * 256 + lane * 4 + j];
        };
        h8_t afr[RB], afr_next[RB];
        uint32_t wcur[TPW], wnext[TPW];
        load_afr(afr, 0);
        load_words(wcur, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {          // 32-k steps
            if (j < 3) load_words(wnext, j + 1);
            uint32_t bh[2][PAIRS];
#pragma unroll
            for (int q = 0; q < PAIRS; ++q) {
                const auto s1 = __builtin_amdgcn_permlane16_swap(wcur[2 * q], wcur[2 * q + 1], false, false);
                const auto s2 = __builtin_amdgcn_permlane32_swap(s1[0], s1[1], false, false);
                bh[0][q] = s2[0];
                bh[1][q] = s2[1];
            }
#pragma unroll
            for (int ph = 0; ph < 2; ++ph) {   // 16-k halves
                const int hs = 2 * j + ph;     // 16-k step within the chunk
                const int gq = hs / HS_PER_GROUP;               // group within the chunk
                const int t_in = hs % HS_PER_GROUP;             // step within the group
                if (hs < 7) load_afr(afr_next, hs + 1);         // one step ahead
#pragma unroll
                for (int q = 0; q < PAIRS; ++q) {
                    h2_t u[4];
                    unpack8(bh[ph][q], zp_const(zc[q][gq]), u);
                    const h8_t b = as_h8(u);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) grp[rb][q] = mfma32(afr[rb], b, t_in == 0 ? zero : grp[rb][q]);
                }
                if (t_in == HS_PER_GROUP - 1) {
                    // group complete: scale it into the running total
#pragma unroll
                    for (int q = 0; q < PAIRS; ++q)
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                            for (int e = 0; e < 16; ++e)
                                total[rb][q][e] = __builtin_fmaf(grp[rb][q][e], sc[q][gq], total[rb][q][e]);
                }
                if (hs < 7) {
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) afr[rb] = afr_next[rb];
                }
                // keep each step's reads one step ahead of their use: no
                // instruction moves across a 16-k step boundary
                __builtin_amdgcn_sched_barrier(0);
            }
            if (j < 3) {
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt) wcur[tt] = wnext[tt];
            }
        }
    };

    // ---- pipeline: chunks c+1 .. c+NST-1 are in flight while c computes ----
#pragma unroll
    for (int s = 0; s < NST - 1; ++s) {
        if (s < C) issue_chunk(s, s);
    }
    for (int c = 0; c < C; ++c) {
        // chunk c landed for this wave (later chunks may stay in flight) ...
        if (c + NST - 2 < C) wait_vm<(NST - 2) * G::kDmaPerChunk>();
        else wait_vm<0>();
        block_sync_lds();   // ... and for every wave; stage (c-1) % NST is free
        if (c + NST - 1 < C) issue_chunk(c + NST - 1, (c + NST - 1) % NST);
        chunk(c % NST);
    }

    // ---- epilogue: lane holds column (lane & 31) of each 32x32 block, rows
    // 8*(e/4) + 4*oct + e%4
#pragma unroll
    for (int q = 0; q < PAIRS; ++q) {
        const int n = nb * BN + wave * 64 + q * 32 + (lane & 31);
        if (n >= p.N) continue;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + rb * 32 + 8 * (e >> 2) + 4 * oct + (e & 3);
                if (m < p.M) p.y[(int64_t)m * p.N + n] = __float2half_rn(total[rb][q][e]);
            }
        }
    }
}

template <typename ST, int Q, bool HAS_ZP>
hipError_t launch_t(const GemmParams& p, hipStream_t s)
{
    const int blocks = p.num_m * p.num_n;
    gemm_mfma_kernel<ST, Q, HAS_ZP><<<dim3(blocks), dim3(WAVES * 64), 0, s>>>(p);
    return hipGetLastError();
}

template <typename ST, bool HAS_ZP>
hipError_t launch_q(const Layout& L, const GemmParams& p, hipStream_t s)
{
    switch (L.Q) {
    case 1: return launch_t<ST, 1, HAS_ZP>(p, s);
    case 2: return launch_t<ST, 2, HAS_ZP>(p, s);
    case 4: return launch_t<ST, 4, HAS_ZP>(p, s);
    default: return launch_t<ST, 8, HAS_ZP>(p, s);
    }
}

}  // namespace

int64_t gemm_mfma_max_repacked_bytes() { return (int64_t)0x7FFFFF00; }

hipError_t launch_gemm_mfma(const Layout& L, const WeightView& w, const void* a, int64_t m,
                            void* y, hipStream_t stream, const char** variant)
{
    GemmParams p;
    p.w = w.codes;   // the codes section starts the repacked buffer
    p.scales_off = L.scales_off;
    p.zp_off = L.zp_off;
    p.w_bytes = (uint32_t)L.total;
    p.a = static_cast<const _Float16*>(a);
    p.y = static_cast<__half*>(y);
    p.M = (int)m;
    p.N = (int)L.N;
    p.K = (int)L.K;
    p.C = (int)L.C;
    p.T = (int)L.T;
    p.num_m = (int)((m + BM - 1) / BM);
    p.num_n = (int)((L.N + BN - 1) / BN);
    if (variant) *variant = "gemm_mfma_32x32x16";
    if (L.ss == 2)
        return L.has_zp ? launch_q<__half, true>(L, p, stream) : launch_q<__half, false>(L, p, stream);
    return L.has_zp ? launch_q<float, true>(L, p, stream) : launch_q<float, false>(L, p, stream);
}

}  // namespace mnb
