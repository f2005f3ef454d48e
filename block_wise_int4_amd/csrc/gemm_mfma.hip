// gemm_mfma.hip -- prefill GEMM (M > 16) on the gfx950 matrix cores.
//
// Method: onnx-runtime-ep-cuda 0.1.0-dev.6, src/kernels/marlin_gemm.rs
// (matmul_nbits_marlin_gemm_f16 and its module doc): weights enter the matrix
// multiply centred but unscaled, as exact fp16 (code - zp); products
// accumulate in fp32 and each group's scale is applied in fp32 after that
// group's accumulate, never folded into the fp16 weights.
//
// gfx950 design.
// * v_mfma_f32_32x32x16_f16 (32x32 output, 16 k).
// * Workgroup tile 96 (M) x 256 (N), 4 waves; wave w owns columns
//   [64w, +64) of all 96 rows: 3 row blocks x 2 column pairs of 32x32 tiles.
//   Two workgroups share a CU (two waves per SIMD).  Groups of 32 or 16 k
//   (and fp32 scales with zero points at 64 k) use 64-row tiles (2 row
//   blocks): their per-chunk rescale factors and zero points would push a
//   96-row wave past 256 registers or its stages past half the LDS, one
//   wave per SIMD, which measured twice as slow.
// * Groups of 128 k also have a 128-row form (4 row blocks per wave): each
//   unpacked B operand then feeds four MFMAs instead of three, and only two
//   pipeline stages fit in the workgroup's half of the LDS.  Groups of 128
//   and 64 k also have a 64-row form, faster where every workgroup fits on
//   the chip at once.  The launcher picks the height per call from the
//   number of workgroup rounds each leaves on the chip's CUs, weighted by its
//   cost (a 64-row workgroup about 0.82 times a 96-row one, a 128-row one
//   about 1.23 times); all give the same bits, as every output adds the same
//   products in the same order.
// * A rows reach LDS by buffer_load ... lds (no VGPR round trip) into a ring
//   of as many stages as the workgroup's share of LDS holds (three for the
//   common record sizes); the DMAs of chunk c + stages - 1 are spread over the
//   matrix work of chunk c.  A's 16-byte segments are XOR-swizzled by row,
//   so fragment reads are conflict free.  Rows and k outside the operand read
//   as zero through the range check.
// * Code words are loaded straight into the lanes that use them, a chunk
//   ahead: the repacked 16-column tile (16 columns x 4 k-octets per 32 k)
//   holds, in one 16-byte lane record, the four 32-k steps of one column and
//   k-octet, which is exactly what a lane of the 32x32x16 B operand needs.
// * Per-group scaling with a single accumulator per output: while group g
//   accumulates, acc holds total / s_g; entering group g+1 it is multiplied
//   by s_g / s_{g+1}, and after the last group the output is acc * s_last.
//   For fp32 outputs (int8 activations) the ratio is a correctly rounded
//   division and each rescale adds two fp32 roundings (the ratio and the
//   product); for fp16 outputs it is the product with v_rcp_f32 (1 ulp), a
//   relative error of at most 2^-22 per rescale.  A group with
//   scale 0 gets all-zero B operands (it adds exactly nothing, NaN for
//   infinite activations as (c - z) * 0 * a does) and keeps the units; the
//   padding past K is such a group.  Half the registers of a separate group
//   accumulator are freed for deeper prefetch and for two waves per SIMD.
//   This needs the range class the repack records per tile: nonzero scales
//   in [2^-100, 2^100] and within 2^64 of each other per column, so that
//   total / s_g stays inside binary32 for any fp16 activations.  A workgroup
//   with a tile outside that class computes its whole tile the plain way
//   instead: a fresh fp32 partial per group, multiplied by the group's scale
//   into the total with an fma (slower, any scales).
// * Workgroup ids are remapped so the tiles resident on one XCD at a time
//   share A rows and code columns in that XCD's L2.
// * Epilogues: fp16 outputs (with an optional fp16 bias in either rounding of
//   matmul_nbits.rs fold_bias_f16), or, for int8 activation codes as A
//   (accuracy_level 4), fp32 outputs times the row's activation scale plus an
//   fp32 bias.
#include <atomic>
#include <type_traits>

#include "mnb_device.hpp"
#include "mnb_acc4.hpp"
#include "mnb_internal.hpp"

namespace mnb {

namespace {

constexpr int BN = 256;            // columns per workgroup (16 tiles of 16)
constexpr int WAVES = 4;           // one per SIMD; wave w owns columns [64w, 64w+64)
constexpr int PAIRS = 2;           // 32-column pairs of tiles per wave
constexpr int TPW = 2 * PAIRS;     // 16-column tiles per wave
constexpr int SEGS = kChunkK / 8;  // 16-byte segments per A row per chunk
constexpr int kGroupM = 4;         // m-blocks per XCD-local band
constexpr int kWgPerCu = 8 / WAVES;          // two waves per SIMD
constexpr int kLdsCu = 160 * 1024;
constexpr int kLdsBudget = kLdsCu / kWgPerCu;   // this workgroup's share
constexpr int kMaxStages = 6;
constexpr int kMaxBM = 96;         // rows of the three-stage form
constexpr int kTallBM = 128;       // rows of the two-stage form (groups of 128 k)
constexpr int kShortBM = 64;       // rows of the short form


typedef float f16v_t __attribute__((ext_vector_type(16)));

struct GemmParams {
    const uint8_t* w;      // repacked weight base
    int64_t scales_off, zp_off;
    uint32_t w_bytes;      // repacked size (buffer range)
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
    int T;                 // column tiles
    int num_m, num_n;      // workgroup grid
    int vec_store;         // 16-byte row stores: y (y32) 16-byte aligned, N % 8 (N % 4) == 0
    int64_t flags_off;     // the per-tile scale range classes
};

// Tile height and LDS geometry of one pipeline stage for (Q, scale bytes,
// zero points, requested height H).  Rows per workgroup: H when given (128:
// the two-stage form for groups of 128 k; 64: the short form); else 96 when
// a 96-row stage leaves room for three stages in the workgroup's half of the
// LDS and groups span 64 k or more; else 64 (groups of 32 or 16 k, whose
// per-chunk rescale factors and zero points would also push a 96-row wave
// past 256 registers).
template <int Q, int SS, bool HAS_ZP, int H> struct StageGeom {
    static constexpr int kScaleDw = kTileN * Q * SS / 4;               // dwords per tile record
    static constexpr int kZpDw = HAS_ZP ? kTileN * Q / 8 : 0;          // 8Q bytes per tile record
    // per wave: the scale records of its tiles, then (from a 64-dword
    // boundary) their zero-point records; one dword DMA per 64 dwords
    static constexpr int kScaleInstr = (TPW * kScaleDw + 63) / 64;
    static constexpr int kZpInstr = (TPW * kZpDw + 63) / 64;
    static constexpr int kMetaInstr = kScaleInstr + kZpInstr;
    static constexpr int kZpOffDw = kScaleInstr * 64;                  // zero points in the record
    static constexpr int kMetaDwPad = kMetaInstr * 64;
    static constexpr int kMeta = WAVES * kMetaDwPad * 4;
    static_assert(H == 0 || H == kShortBM || (H == kTallBM && Q == 1),
                  "the two-stage form serves groups of 128 k");
    static constexpr bool kFits96 = Q < 4 && kLdsBudget / (kMaxBM * SEGS * 16 + kMeta) >= 3;
    static constexpr int BM = H ? H : kFits96 ? kMaxBM : kShortBM;
    static constexpr int RB = BM / 32;                  // 32-row blocks per wave
    static constexpr int ROWS_PER_WAVE = BM / WAVES;    // A rows each wave copies per chunk
    static constexpr int A_DMA = ROWS_PER_WAVE / 4;     // 1 KiB (4-row) DMAs per wave per chunk
    static_assert(ROWS_PER_WAVE % 4 == 0, "A is copied in 4-row pieces");
    static constexpr int kA = BM * SEGS * 16;                          // bytes
    static constexpr int kB = 0;                                       // codes go to VGPRs
    static constexpr int kBytes = kA + kB + kMeta;
    // as many pipeline stages as the workgroup's share of LDS holds (up to
    // kMaxStages); when that is fewer than three (large scale records), three
    // or more in the whole LDS, leaving one workgroup per CU.  The 128-row
    // form keeps two.
    static constexpr int kMinStages = BM == kTallBM ? 2 : 3;
    static constexpr int kFit = kLdsBudget / kBytes >= kMinStages ? kLdsBudget / kBytes : kLdsCu / kBytes;
    static constexpr int kStages = kFit < kMaxStages ? kFit : kMaxStages;
    static constexpr int kDmaPerChunk = A_DMA + kMetaInstr;            // per wave
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

// unpack8 for the rescaled accumulator: (c - z) as exact fp16 pairs, or all
// zeros for a group whose scale is zero (bit 4 of zf), so such a group adds
// exactly nothing (NaN for infinite activations, as (c - z) * 0 * a does).
// Both nibble halves use one packed fma, (x | magic) * m + a, with m = 1 or
// 1/16 and a = -(1024 + z) or -(64 + z) for a live group and m = a = 0 for a
// dead one.  The two m and the two a sit in the halves of one register each
// (a is zp_pair's), and each fma takes its pair from one half (op_sel).
__device__ __forceinline__ void unpack8_scaled(uint32_t d, uint32_t zf, h2_t out[4])
{
    const uint32_t lo = 0x000F000Fu, hi = 0x00F000F0u, magic = 0x64006400u;
    const bool dead = zf >= 16u;
    const h2_t m = as_h2(dead ? 0u : 0x2C003C00u);          // 1/16 (high half), 1.0 (low half)
    const h2_t a = as_h2(dead ? 0u : zp_pair(zf & 15u));
    const h2_t m_lo = {m[0], m[0]}, m_hi = {m[1], m[1]};
    const h2_t a_lo = {a[0], a[0]}, a_hi = {a[1], a[1]};
    const uint32_t d8 = d >> 8;
    out[0] = as_h2(__builtin_amdgcn_bitop3_b32(d, lo, magic, 0xEA)) * m_lo + a_lo;
    out[1] = as_h2(__builtin_amdgcn_bitop3_b32(d, hi, magic, 0xEA)) * m_hi + a_hi;
    out[2] = as_h2(__builtin_amdgcn_bitop3_b32(d8, lo, magic, 0xEA)) * m_lo + a_lo;
    out[3] = as_h2(__builtin_amdgcn_bitop3_b32(d8, hi, magic, 0xEA)) * m_hi + a_hi;
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

// The pipeline's stages, or the epilogue's staging of the output block
// (BM rows of 144 bytes per wave), whichever is larger.
template <typename ST, int Q, bool HAS_ZP, int H> struct KernelLds {
    typedef StageGeom<Q, (int)sizeof(ST), HAS_ZP, H> G;
    static constexpr int kPipe = G::kStages * G::kBytes;
    static constexpr int kOut = WAVES * G::BM * 144;
    static constexpr int kBytes = kPipe > kOut ? kPipe : kOut;
};

// F32OUT: the int8-activation epilogue (fp32 output, row scale, fp32 bias),
// its own instantiation so that the fp16 kernel's code is not affected.
template <typename ST, int Q, bool HAS_ZP, bool KTAIL, bool F32OUT, int H>
__global__ __launch_bounds__(WAVES * 64, kWgPerCu) void gemm_mfma_kernel(GemmParams p)
{
    typedef StageGeom<Q, (int)sizeof(ST), HAS_ZP, H> G;
    constexpr int NST = G::kStages;
    constexpr int BM = G::BM, RB = G::RB, ROWS_PER_WAVE = G::ROWS_PER_WAVE, A_DMA = G::A_DMA;
    __shared__ __align__(16) unsigned char lds[KernelLds<ST, Q, HAS_ZP, H>::kBytes];

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
    // Every buffer starts at this workgroup's (or wave's) first row or first
    // tile, so offsets stay far inside 32 bits whatever the size of the
    // operands, and rows, tiles and k outside the operand read as zero
    // through the range check.  A: at most 32 rows from row r0 (the rows a
    // wave copies, or one 32-row block), ending at the last valid row; k >= K
    // uses an offset past the range.
    auto a_rows = [&](int r0, int rows) {
        int n = p.M - r0;
        n = n < rows ? n : rows;
        n = n > 0 ? n : 0;
        return __builtin_amdgcn_make_buffer_rsrc((void*)(p.a + (n > 0 ? (int64_t)r0 * K : 0)), (short)0,
                                                 (int)((uint32_t)n * (uint32_t)K * 2u), 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t a_rsrc = a_rows(m0 + ROWS_PER_WAVE * wave, ROWS_PER_WAVE);
    const int t0 = nb * (BN / 16);                         // first tile of the workgroup
    const int tiles_here = (p.T - t0) < BN / 16 ? (p.T - t0) : BN / 16;
    const uint32_t code_bytes = (uint32_t)tiles_here * (uint32_t)C * 1024u;
    const uint32_t scale_bytes = (uint32_t)tiles_here * (uint32_t)C * (uint32_t)(G::kScaleDw * 4);
    const uint32_t zp_bytes = (uint32_t)tiles_here * (uint32_t)C * (uint32_t)(G::kZpDw * 4);
    const __amdgpu_buffer_rsrc_t c_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.w + (int64_t)t0 * C * 1024), (short)0, (int)code_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.w + p.scales_off + (int64_t)t0 * C * (G::kScaleDw * 4)), (short)0, (int)scale_bytes,
        0x00020000);
    const __amdgpu_buffer_rsrc_t z_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.w + (HAS_ZP ? p.zp_off : 0) + (int64_t)t0 * C * (G::kZpDw * 4)), (short)0,
        (int)zp_bytes, 0x00020000);

    // The range classes of the workgroup's tiles (one byte each; the 16
    // bytes from t0 lie inside the flags section, whose size is rounded up to
    // 256), requested before any DMA so that they have landed when chunk 0
    // has.
    const u4_t tile_flags = *reinterpret_cast<const u4_t*>(p.w + p.flags_off + t0);

    // The LDS DMAs of one chunk, one "piece" (one instruction) at a time, so
    // they can be spread over the compute of an earlier chunk: pieces
    // 0 .. A_DMA-1 copy A rows, then the scale records and the zero-point
    // records of the wave's tiles.  Each lane's part of an offset is fixed
    // for the whole loop; the chunk's part is uniform and goes in the scalar
    // offset.  Padding lanes of the record DMAs use an offset past every
    // range, so they read zero.
    constexpr uint32_t kFar = 0x80000000u;
    uint32_t a_voff[A_DMA];
    uint32_t s_voff[G::kScaleInstr], z_voff[G::kZpInstr > 0 ? G::kZpInstr : 1];
    auto set_offsets = [&](int ln) __attribute__((always_inline)) {
#pragma unroll
        for (int idx = 0; idx < A_DMA; ++idx) {
            const int rw = 4 * idx + (ln >> 4);            // row among the wave's
            const int r = ROWS_PER_WAVE * wave + rw;       // row in the tile
            const int sg = (ln & 15) ^ (r & 15);           // logical segment at this slot
            a_voff[idx] = ((uint32_t)rw * (uint32_t)K + 8u * (uint32_t)sg) * 2u;
        }
#pragma unroll
        for (int m = 0; m < G::kScaleInstr; ++m) {
            const int d = m * 64 + ln;
            const int tt = d / G::kScaleDw, o = d % G::kScaleDw;
            s_voff[m] = d < TPW * G::kScaleDw
                ? (uint32_t)(wave * TPW + tt) * (uint32_t)C * (uint32_t)(G::kScaleDw * 4) + (uint32_t)o * 4u : kFar;
        }
#pragma unroll
        for (int m = 0; m < G::kZpInstr; ++m) {
            constexpr int ZD = G::kZpDw > 0 ? G::kZpDw : 1;
            const int d = m * 64 + ln;
            const int tt = d / ZD, o = d % ZD;
            z_voff[m] = d < TPW * G::kZpDw
                ? (uint32_t)(wave * TPW + tt) * (uint32_t)C * (uint32_t)(ZD * 4) + (uint32_t)o * 4u : kFar;
        }
    };
    set_offsets(lane);
    auto issue_piece = [&](int c, int st, int idx) {
        if (idx < A_DMA) {
            // A rows [ROWS_PER_WAVE*wave + 4*idx, +4); a chunk reaching past K
            // (K not a multiple of 128) sends its lanes past K out of range
            uint32_t voff = a_voff[idx];
            if (KTAIL) {
                const int r = ROWS_PER_WAVE * wave + 4 * idx + (lane >> 4);
                if (c * kChunkK + 8 * ((lane & 15) ^ (r & 15)) >= K) voff = kFar;
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr_t)(stage_a(st) + (ROWS_PER_WAVE * wave + 4 * idx) * SEGS),
                                                     16, voff, (uint32_t)c * (kChunkK * 2), 0, 0);
        } else if (idx < A_DMA + G::kScaleInstr) {
            const int m = idx - A_DMA;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lds_ptr_t)(stage_m(st) + m * 256), 4, s_voff[m],
                                                     (uint32_t)c * (uint32_t)(G::kScaleDw * 4), 0, 0);
        } else {
            constexpr int ZD = G::kZpDw > 0 ? G::kZpDw : 1;
            const int m = idx - A_DMA - G::kScaleInstr;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(z_rsrc, (lds_ptr_t)(stage_m(st) + (G::kScaleInstr + m) * 256), 4,
                                                     z_voff[m], (uint32_t)c * (uint32_t)(ZD * 4), 0, 0);
        }
    };

    // One fp32 accumulator per output, kept in units of the current
    // group's scale: acc = total / s_g while group g accumulates.  At a group
    // boundary acc is multiplied by s_g / s_{g+1}; after the last group the
    // output is acc * s_last.
    f16v_t acc[RB][PAIRS];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int q = 0; q < PAIRS; ++q)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[rb][q][e] = 0.f;

    constexpr int HS_PER_GROUP = 8 / Q;          // 16-k steps per group (group = 128/Q)
    constexpr int NP = G::kDmaPerChunk;           // DMA pieces per chunk and wave
    constexpr int NP_STEP = (NP + 5) / 6;         // pieces issued per step (steps 0..5)
    static_assert(NST >= 2, "the pipeline keeps at least two stages");
    static_assert((NST - 2) * NP + 2 * PAIRS < 64, "vmcnt range");
    // Wait until chunk j's DMAs (this wave's) have landed, with y later
    // chunks' DMAs and the next chunk's code words issued after them
    // (y <= NST - 2; a smaller y than the truth only waits longer).  With
    // two stages, chunk j's DMAs and code words are issued in the same chunk,
    // in no fixed order, and nothing later: wait for all of them.
    auto wait_landed = [&](int y) {
        if constexpr (NST == 2) { wait_vm<0>(); return; }
        if constexpr (NST - 2 >= 4) { if (y >= 4) { wait_vm<4 * NP + 2 * PAIRS>(); return; } }
        if constexpr (NST - 2 >= 3) { if (y >= 3) { wait_vm<3 * NP + 2 * PAIRS>(); return; } }
        if constexpr (NST - 2 >= 2) { if (y >= 2) { wait_vm<2 * NP + 2 * PAIRS>(); return; } }
        if (y >= 1) { wait_vm<NP + 2 * PAIRS>(); return; }
        wait_vm<2 * PAIRS>();
    };

    // units of acc per column pair: the scale of the last group with a
    // nonzero scale (groups past K have scale 0 and contribute exactly 0)
    float unit[PAIRS];
#pragma unroll
    for (int q = 0; q < PAIRS; ++q) unit[q] = 0.f;

    // per-chunk state: the rescale factor entering each group and the zero
    // points of the lane's columns, for the current and the next chunk
    float ratioA[PAIRS][Q], ratioB[PAIRS][Q];
    uint32_t zcA[PAIRS][Q], zcB[PAIRS][Q];
    auto read_meta = [&](int st, float (&rt)[PAIRS][Q], uint32_t (&z)[PAIRS][Q], bool live) {
        const unsigned char* Ms = stage_m(st);
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
            const int tt = 2 * q + half;   // this lane's column lives in tile 2q + half
            const ST* srec = reinterpret_cast<const ST*>(Ms + tt * G::kScaleDw * 4);
#pragma unroll
            for (int g = 0; g < Q; ++g) {
                const int sl = slot_of(i, g, Q);
                const float sg = to_f32(srec[sl]);
                // the int8-activation (fp32 output) form, whose bound counts
                // roundings, divides correctly rounded; the fp16 output's
                // bound (1e-3 of the magnitude sum) leaves room for the
                // reciprocal's 1-ulp error
                if constexpr (F32OUT)
                    rt[q][g] = sg != 0.f ? __fdiv_rn(unit[q], sg) : 1.f;
                else
                    rt[q][g] = sg != 0.f ? unit[q] * __builtin_amdgcn_rcpf(sg) : 1.f;
                unit[q] = (live && sg != 0.f) ? sg : unit[q];
                uint32_t zv = 8u;
                if (HAS_ZP) {
                    const unsigned char* zrec = Ms + (G::kZpOffDw + tt * G::kZpDw) * 4;
                    zv = (zrec[sl >> 1] >> (4 * (sl & 1))) & 15u;
                }
                // bit 4: the group's scale is zero, so its B operands are zero
                z[q][g] = zv | (sg == 0.f ? 16u : 0u);
            }
        }
    };
    // A fragments of 16-k step hs: row (rb*32 + lane%32), k-octet oct; the
    // XOR swizzle term depends on the lane only (rb*32 is a multiple of 16).
    auto load_afr = [&](int st, h8_t (&afr)[RB], int hs) {
        const u4_t* As = stage_a(st);
        const int sgi = (2 * hs + oct) ^ (lane & 15);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            afr[rb] = __builtin_bit_cast(h8_t, As[(rb * 32 + (lane & 31)) * SEGS + sgi]);
    };
    // Code words go straight from memory to the lanes that use them, in
    // the 32x32x16 B-operand distribution: lane l takes column l%32 (tile
    // 2q + (l/16)%2 of pair q, column l%16) and, for 16-k step hs, k-octet
    // 2*(hs%2) + l/32 of 32-k step hs/2.  The repacked chunk holds that
    // octet in word hs/2 of the tile's lane (k-octet*16 + column), so one
    // 16-byte load per (pair, hs%2) brings a lane all four 32-k steps.
    uint32_t b_voff[PAIRS][2];
#pragma unroll
    for (int q = 0; q < PAIRS; ++q)
#pragma unroll
        for (int ph = 0; ph < 2; ++ph) {
            const int src = (2 * ph + oct) * 16 + i;
            b_voff[q][ph] = (uint32_t)(wave * TPW + 2 * q + half) * (uint32_t)C * 1024u + (uint32_t)src * 16u;
        }
    auto load_b = [&](int c, u4_t (&bq)[PAIRS][2]) {
#pragma unroll
        for (int q = 0; q < PAIRS; ++q)
#pragma unroll
            for (int ph = 0; ph < 2; ++ph)
                bq[q][ph] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(
                    c_rsrc, b_voff[q][ph], (uint32_t)c * 1024u, 0));
    };
    auto load_bw = [&](const u4_t (&bq)[PAIRS][2], uint32_t (&w)[PAIRS], int hs) {
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) w[q] = bq[q][hs & 1][hs >> 1];
    };
    auto unpack_b = [&](const uint32_t (&w)[PAIRS], const uint32_t (&z)[PAIRS][Q], int hs, h8_t (&bop)[PAIRS]) {
        const int gq = hs / HS_PER_GROUP;
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
            h2_t u[4];
            unpack8_scaled(w[q], z[q][gq], u);
            bop[q] = as_h8(u);
        }
    };

    // A fragments: two sets indexed by the parity of the step, read one step
    // ahead (the other wave on the SIMD covers the LDS latency); the next
    // chunk's first step is read in step 7, after the barrier that makes
    // that chunk visible.  Code words: this chunk's and the next one's,
    // loaded a chunk ahead.  B operands: unpacked one step ahead.
    h8_t afr[2][RB];
    u4_t bqA[PAIRS][2], bqB[PAIRS][2];
    h8_t bop[2][PAIRS];

    // The plain per-group evaluation, for tiles outside the range class of
    // the rescaled accumulator: one 32x32 block at a time, A fragments and
    // code words straight from memory (rows and k outside the operand read
    // zero), a fresh fp32 partial per group, and the total += partial * scale
    // in fp32.  A group whose scale is 0 adds 0 (NaN for a non-finite
    // partial, as (c - z) * 0 * a does).
    auto fallback_tile = [&]() {
        constexpr int SREC = G::kScaleDw * 4, ZREC = G::kZpDw * 4;
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
            const int tt = wave * TPW + 2 * q + half;   // the lane's tile in the workgroup
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                f16v_t tot, grp;
#pragma unroll
                for (int e = 0; e < 16; ++e) tot[e] = 0.f;
                const __amdgpu_buffer_rsrc_t ab_rsrc = a_rows(m0 + 64 * (rb >> 1), 64);
                const uint32_t arow = (uint32_t)((rb & 1) * 32 + (lane & 31)) * (uint32_t)K * 2u;
                for (int c = 0; c < C; ++c) {
                    u4_t bq[2];
#pragma unroll
                    for (int ph = 0; ph < 2; ++ph)
                        bq[ph] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(
                            c_rsrc, b_voff[q][ph], (uint32_t)c * 1024u, 0));
                    float sg[Q];
                    uint32_t zg[Q];
#pragma unroll
                    for (int g = 0; g < Q; ++g) {
                        const int sl = slot_of(i, g, Q);
                        const uint32_t rec = (uint32_t)(tt * C + c);
                        if constexpr (sizeof(ST) == 2)
                            sg[g] = (float)__builtin_bit_cast(_Float16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(
                                s_rsrc, rec * SREC + sl * 2, 0, 0));
                        else
                            sg[g] = __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
                                s_rsrc, rec * SREC + sl * 4, 0, 0));
                        zg[g] = 8u;
                        if constexpr (HAS_ZP)
                            zg[g] = ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(z_rsrc, rec * ZREC + (sl >> 1), 0, 0) >>
                                     (4 * (sl & 1))) & 15u;
                    }
#pragma unroll
                    for (int hs = 0; hs < 8; ++hs) {
                        const int k = c * kChunkK + 16 * hs + 8 * oct;
                        h8_t a;
                        if (!KTAIL || k < K)
                            a = __builtin_bit_cast(h8_t, __builtin_amdgcn_raw_buffer_load_b128(
                                ab_rsrc, arow + (uint32_t)k * 2u, 0, 0));
                        else
                            a = h8_t{};
                        h2_t u[4];
                        unpack8(bq[hs & 1][hs >> 1], zp_const(zg[hs / HS_PER_GROUP]), u);
                        if (hs % HS_PER_GROUP == 0) {
#pragma unroll
                            for (int e = 0; e < 16; ++e) grp[e] = 0.f;
                        }
                        grp = mfma32(a, as_h8(u), grp);
                        if (hs % HS_PER_GROUP == HS_PER_GROUP - 1) {
                            const float sc = sg[hs / HS_PER_GROUP];
#pragma unroll
                            for (int e = 0; e < 16; ++e) tot[e] = __builtin_fmaf(grp[e], sc, tot[e]);
                        }
                    }
                }
                acc[rb][q] = tot;
            }
        }
    };

    // ---- prologue: chunks 0 .. NST-2 in flight, chunk 0 read in ----
    // Every chunk's loads and DMAs are issued whether or not the chunk
    // exists: one past the operand reads bytes that are never used (inside
    // the buffer range) or zeros (outside it), into a stage no wave still
    // reads.  So the pipeline has no branches and the same number of loads
    // in flight everywhere.
#pragma unroll
    for (int j = 0; j < NST - 1; ++j) {
#pragma unroll
        for (int k = 0; k < NP; ++k) issue_piece(j, j, k);
    }
    load_b(0, bqA);
    // chunk 0's DMAs landed for this wave (later issues may stay in flight)
    wait_landed(NST - 2);
    block_sync_lds();

    // every wave of the workgroup reads the same bytes: a uniform decision
    bool tiles_safe = true;
#pragma unroll
    for (int j = 0; j < BN / 16; ++j)
        if (j < tiles_here && ((tile_flags[j >> 2] >> (8 * (j & 3))) & 0xFFu) != 1u) tiles_safe = false;
    tiles_safe = uniform(tiles_safe ? 1 : 0) != 0;

    if (!tiles_safe) {
        // the plain way: let the prologue's DMAs land (the epilogue reuses
        // the LDS), then each 32x32 block of the wave on its own
        wait_vm<0>();
        fallback_tile();
    } else {
    // The DMA offsets once more, from an opaque copy of the lane: the
    // prologue's copies then end with the prologue's DMAs instead of living
    // across the fallback branch, which spilled them to scratch memory
    {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        set_offsets(ln);
    }
    read_meta(0, ratioA, zcA, true);
    load_afr(0, afr[0], 0);
    {
        uint32_t w[PAIRS];
        load_bw(bqA, w, 0);
        unpack_b(w, zcA, 0, bop[0]);
    }

    // One chunk.  The code words, rescale factors and zero points of the
    // chunk and of the next one alternate between two register sets (the
    // loop below runs two chunks per trip), so nothing is copied between
    // chunks.  st: pipeline stage of chunk c (wave-uniform).
    int st = 0;
    auto chunk = [&](auto par, int c, const u4_t (&bq)[PAIRS][2], u4_t (&bq_n)[PAIRS][2],
                     const float (&ratio)[PAIRS][Q], float (&ratio_n)[PAIRS][Q],
                     const uint32_t (&zc)[PAIRS][Q], uint32_t (&zc_n)[PAIRS][Q])
        __attribute__((always_inline)) {
        // two stages: the first chunk of a trip is always in stage 0, the
        // second in stage 1, so the stage offsets are constants
        if constexpr (NST == 2) st = decltype(par)::value;
        const int nst = st == NST - 1 ? 0 : st + 1;
        const int dst = st == 0 ? NST - 1 : st - 1;   // stage of chunk c + NST - 1
        const bool more = c + 1 < C;        // wave-uniform
        // one 16-k step; hs is a compile-time constant (the interleave
        // pattern needs constant counts)
        auto step = [&](auto hs_c) {
            constexpr int hs = decltype(hs_c)::value;
            constexpr int gq = hs / HS_PER_GROUP;   // group within the chunk
            constexpr int t_in = hs % HS_PER_GROUP; // step within the group
            // the next chunk's code words, a chunk ahead
            if (hs == 0) load_b(c + 1, bq_n);
            // LDS reads one step ahead (step 7 reads the next chunk's first)
            if (hs + 1 < 8) {
                load_afr(st, afr[(hs + 1) & 1], hs + 1);
            } else {
                read_meta(nst, ratio_n, zc_n, more);
                load_afr(nst, afr[0], 0);
            }
            // this chunk's share of the DMAs of chunk c + NST - 1
            if (hs < 6) {
#pragma unroll
                for (int k = hs * NP_STEP; k < (hs + 1) * NP_STEP && k < NP; ++k) issue_piece(c + NST - 1, dst, k);
            }
            // the matrix work, each group entered with its rescale (the
            // first group's factor is 0 or 1 and acc is still zero)
            constexpr bool rescale = t_in == 0;
#pragma unroll
            for (int q = 0; q < PAIRS; ++q) {
                const float r = ratio[q][gq];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    if (rescale) {
#pragma unroll
                        for (int e = 0; e < 16; ++e) acc[rb][q][e] *= r;
                    }
                    acc[rb][q] = mfma32(afr[hs & 1][rb], bop[hs & 1][q], acc[rb][q]);
                }
            }
            // the next step's B operands
            uint32_t w[PAIRS];
            if (hs + 1 < 8) {
                load_bw(bq, w, hs + 1);
                unpack_b(w, zc, hs + 1, bop[(hs + 1) & 1]);
            } else {
                load_bw(bq_n, w, 0);
                unpack_b(w, zc_n, 0, bop[0]);
            }
            // interleave: LDS reads first, then each MFMA followed by a share
            // of the VALU work and of the memory issue
            constexpr int kReads = RB;
            if (kReads > 0) __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);   // DS reads
#pragma unroll
            for (int k = 0; k < RB * PAIRS; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // 1 MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, t_in == 0 ? 19 : 3, 0); // VALU
                if (hs < 6 && k < NP_STEP + (hs == 0 ? 2 * PAIRS : 0))
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);             // VMEM
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        step(std::integral_constant<int, 0>());
        step(std::integral_constant<int, 1>());
        step(std::integral_constant<int, 2>());
        step(std::integral_constant<int, 3>());
        step(std::integral_constant<int, 4>());
        step(std::integral_constant<int, 5>());
        step(std::integral_constant<int, 6>());
        // chunk c+1's DMAs landed for this wave (later issues: chunk c+1's
        // code words and the DMAs of chunks c+2 .. c+NST-1, may stay in
        // flight) ...
        wait_landed(NST - 2);
        block_sync_lds();   // ... and for every wave
        step(std::integral_constant<int, 7>());
        st = nst;
    };
    for (int c = 0; c < C; c += 2) {
        chunk(std::integral_constant<int, 0>(), c, bqA, bqB, ratioA, ratioB, zcA, zcB);
        if (c + 1 < C) chunk(std::integral_constant<int, 1>(), c + 1, bqB, bqA, ratioB, ratioA, zcB, zcA);
    }

    // the DMAs of the chunks past the last are not waited for in the loop;
    // they land before the epilogue reuses the LDS
    wait_vm<0>();
    // back from units of the last group's scale
#pragma unroll
    for (int q = 0; q < PAIRS; ++q)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[rb][q][e] *= unit[q];
    }   // tiles_safe

    // ---- epilogue: lane holds column (lane & 31) of each 32x32 block, rows
    // 8*(e/4) + 4*oct + e%4
    if constexpr (F32OUT) {
        if (p.pair_rows) {
            // fp32 activations as (hi, lo) row pairs: rows 2m and 2m + 1 of
            // the block sit in the same lane (elements e and e + 1, e even,
            // since m0 and the other row offsets are even); each output is
            // stored on its own
#pragma unroll
            for (int q = 0; q < PAIRS; ++q) {
                const int n = nb * BN + wave * 64 + q * 32 + (lane & 31);
                if (n >= p.N) continue;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int e = 0; e < 16; e += 2) {
                        const int m = m0 + rb * 32 + 8 * (e >> 2) + 4 * oct + (e & 3);
                        if (m >= p.M) continue;
                        const int mo = m >> 1;
                        float v = (acc[rb][q][e] + acc[rb][q][e + 1]) * p.row_scale[mo];
                        if (p.bias32) v = v + p.bias32[(int64_t)mo * p.bias32_stride + n];
                        p.y32[(int64_t)mo * p.N + n] = v;
                    }
            }
            return;
        }
        // fp32 outputs: the accumulator times its row's activation scale (0
        // where that scale is 0), then the bias.  Each row scale is loaded
        // for the store of its row, so the lane's 64 row scales are never
        // live beside its 128 accumulators (held all at once they spilled)
        auto finish32 = [&](float a, float sc, float b) __attribute__((always_inline)) {
            float v = sc != 0.0f ? a * sc : 0.0f;
            if (p.bias32) v = v + b;
            return v;
        };
        if (p.vec_store) {
            // the raw accumulators staged as the fp16 output below, in two
            // passes of BM/2 rows (the fp32 block of a wave is twice the
            // size); 288-byte rows put the two row quads of one write
            // instruction in different banks.  With N % 4 == 0 a 16-byte
            // segment is all inside or all outside.  A lane then finishes
            // and stores 4 columns of one row at a time.
            constexpr int RS = 288, HALF = BM / 2, ROWS = HALF / 4;
            static_assert(WAVES * HALF * RS <= KernelLds<ST, Q, HAS_ZP, H>::kBytes, "half the fp32 block fits the LDS");
            const int n = nb * BN + wave * 64 + (lane & 15) * 4;
            float b4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) b4[j] = p.bias32 ? p.bias32[n + j < p.N ? n + j : p.N - 1] : 0.0f;
            block_sync_lds();   // every wave is past its last fragment reads
            unsigned char* ob = lds + wave * (HALF * RS);
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
                float rsv[ROWS];
#pragma unroll
                for (int i = 0; i < ROWS; ++i) {
                    const int m = m0 + hp * HALF + (lane >> 4) + 4 * i;
                    rsv[i] = p.row_scale[m < p.M ? m : p.M - 1];
                }
                // 8-row block rb*4 + e/4 of the wave's BM rows is in pass (rb*4 + e/4) / (HALF/8)
#pragma unroll
                for (int q = 0; q < PAIRS; ++q)
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            if ((rb * 4 + (e >> 2)) / (HALF / 8) != hp) continue;
                            const int row = rb * 32 + 8 * (e >> 2) + 4 * oct + (e & 3) - hp * HALF;
                            *reinterpret_cast<float*>(ob + row * RS + (q * 32 + (lane & 31)) * 4) = acc[rb][q][e];
                        }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int i = 0; i < ROWS; ++i) {
                    const int row = (lane >> 4) + 4 * i;
                    const int m = m0 + hp * HALF + row;
                    f4_t v = __builtin_bit_cast(f4_t, *reinterpret_cast<const u4_t*>(ob + row * RS + (lane & 15) * 16));
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = finish32(v[j], rsv[i], b4[j]);
                    if (m < p.M && n < p.N) *reinterpret_cast<u4_t*>(p.y32 + (int64_t)m * p.N + n) = __builtin_bit_cast(u4_t, v);
                }
                // the reads are done before the next pass writes
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
            return;
        }
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
            const int n = nb * BN + wave * 64 + q * 32 + (lane & 31);
            if (n >= p.N) continue;
            const float bn = p.bias32 ? p.bias32[n] : 0.0f;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int m = m0 + rb * 32 + 8 * (e >> 2) + 4 * oct + (e & 3);
                    if (m < p.M) p.y32[(int64_t)m * p.N + n] = finish32(acc[rb][q][e], p.row_scale[m], bn);
                }
        }
        return;
    }
    // fp16 outputs, value(rb, q, e) for each accumulator element.  With
    // vec_store (N % 8 == 0, y 16-byte aligned) each wave stages its BM x 64
    // block in LDS, row-major with 144-byte rows (the two row quads of one
    // store instruction fall in different banks), then writes 8 columns of
    // one row per lane: 96 rows in 12 full-line instructions instead of 96
    // two-byte ones.  A segment is then all inside the output or all
    // outside.  Otherwise every element is stored on its own.
    auto store_f16 = [&](auto value) __attribute__((always_inline)) {
        if (p.vec_store) {
            constexpr int RS = 144;
            static_assert(WAVES * BM * RS <= KernelLds<ST, Q, HAS_ZP, H>::kBytes, "the output block fits the LDS");
            block_sync_lds();   // every wave is past its last fragment reads
            unsigned char* ob = lds + wave * (BM * RS);
#pragma unroll
            for (int q = 0; q < PAIRS; ++q)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int row = rb * 32 + 8 * (e >> 2) + 4 * oct + (e & 3);
                        *reinterpret_cast<__half*>(ob + row * RS + (q * 32 + (lane & 31)) * 2) = value(rb, q, e);
                    }
            // the wave reads what its other lanes wrote: LDS keeps a wave's
            // operations in order; this keeps the compiler from moving them
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            const int n = nb * BN + wave * 64 + (lane & 7) * 8;
#pragma unroll
            for (int i = 0; i < BM / 8; ++i) {
                const int row = (lane >> 3) + 8 * i;
                const u4_t v = *reinterpret_cast<const u4_t*>(ob + row * RS + (lane & 7) * 16);
                if (m0 + row < p.M && n < p.N) *reinterpret_cast<u4_t*>(p.y + (int64_t)(m0 + row) * p.N + n) = v;
            }
            return;
        }
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
            const int n = nb * BN + wave * 64 + q * 32 + (lane & 31);
            if (n >= p.N) continue;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int m = m0 + rb * 32 + 8 * (e >> 2) + 4 * oct + (e & 3);
                    if (m < p.M) p.y[(int64_t)m * p.N + n] = value(rb, q, e);
                }
        }
    };
    if (p.bias && p.bias_stride == 0) {
        // one bias vector for every row: the lane's two columns only
        float bq[PAIRS];
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
            const int n = nb * BN + wave * 64 + q * 32 + (lane & 31);
            bq[q] = __half2float(p.bias[n < p.N ? n : p.N - 1]);
        }
        store_f16([&](int rb, int q, int e) { return finish_value(acc[rb][q][e], bq[q], p.bias_after_round); });
        return;
    }
    if (p.bias) {
        // a per-row bias.  With 16-byte stores the raw accumulators are
        // staged in LDS as fp32, in two passes of BM/2 rows as for the fp32
        // output, and a lane finishes 4 columns of one row at a time; a
        // pass's bias elements are requested before its staging, so their
        // latency hides behind it, and only that pass's 64 are live (all 128
        // of a lane held at once spilled).  Rows and columns outside the
        // output read an element inside it.  Otherwise each output element
        // reads its own bias element.
        if (p.vec_store) {
            constexpr int RS = 288, HALF = BM / 2, ROWS = HALF / 4;
            static_assert(WAVES * HALF * RS <= KernelLds<ST, Q, HAS_ZP, H>::kBytes, "half the fp32 block fits the LDS");
            const int n = nb * BN + wave * 64 + (lane & 15) * 4;
            const int nc = n < p.N ? n : p.N - 4;     // N % 8 == 0 here
            block_sync_lds();   // every wave is past its last fragment reads
            unsigned char* ob = lds + wave * (HALF * RS);
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
                __half bb[ROWS][4];
#pragma unroll
                for (int i = 0; i < ROWS; ++i) {
                    int m = m0 + hp * HALF + (lane >> 4) + 4 * i;
                    m = m < p.M ? m : p.M - 1;
#pragma unroll
                    for (int j = 0; j < 4; ++j) bb[i][j] = p.bias[(int64_t)m * p.bias_stride + nc + j];
                }
#pragma unroll
                for (int q = 0; q < PAIRS; ++q)
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            if ((rb * 4 + (e >> 2)) / (HALF / 8) != hp) continue;
                            const int row = rb * 32 + 8 * (e >> 2) + 4 * oct + (e & 3) - hp * HALF;
                            *reinterpret_cast<float*>(ob + row * RS + (q * 32 + (lane & 31)) * 4) = acc[rb][q][e];
                        }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int i = 0; i < ROWS; ++i) {
                    const int row = (lane >> 4) + 4 * i;
                    const int m = m0 + hp * HALF + row;
                    const f4_t v = __builtin_bit_cast(f4_t, *reinterpret_cast<const u4_t*>(ob + row * RS + (lane & 15) * 16));
                    uint32_t h[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        h[j] = __half_as_ushort(finish_value(v[j], __half2float(bb[i][j]), p.bias_after_round));
                    if (m < p.M && n < p.N)
                        *reinterpret_cast<uint2*>(p.y + (int64_t)m * p.N + n) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
                }
                // the reads are done before the next pass writes
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
            return;
        }
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
            const int n = nb * BN + wave * 64 + q * 32 + (lane & 31);
            if (n >= p.N) continue;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int m = m0 + rb * 32 + 8 * (e >> 2) + 4 * oct + (e & 3);
                    if (m < p.M)
                        p.y[(int64_t)m * p.N + n] = finish_value(
                            acc[rb][q][e], __half2float(p.bias[(int64_t)m * p.bias_stride + n]), p.bias_after_round);
                }
        }
        return;
    }
    store_f16([&](int rb, int q, int e) { return __float2half_rn(acc[rb][q][e]); });
}

template <typename ST, int Q, bool HAS_ZP, bool F32OUT, int H>
void launch_k(GemmParams p, hipStream_t s)
{
    constexpr int BM = StageGeom<Q, (int)sizeof(ST), HAS_ZP, H>::BM;
    p.num_m = (p.M + BM - 1) / BM;
    const int blocks = p.num_m * p.num_n;
    if (Q == 1 || p.K % kChunkK == 0) {
        // groups of 128 k: K is a multiple of the chunk
        gemm_mfma_kernel<ST, Q, HAS_ZP, false, F32OUT, H><<<dim3(blocks), dim3(WAVES * 64), 0, s>>>(p);
    } else {
        if constexpr (Q != 1)
            gemm_mfma_kernel<ST, Q, HAS_ZP, true, F32OUT, H><<<dim3(blocks), dim3(WAVES * 64), 0, s>>>(p);
    }
}

// Compute units of the current device (queried once per device).
int device_cus()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// A fixed tile height where the group size offers several (64, 96 or 128;
// one the group size does not offer leaves the default), or 0: per call.
std::atomic<int> g_prefill_rows{0};

// Tile height for groups of 128 or 64 k: the one whose workgroup rounds,
// weighted by its cost, are fewest (128 rows only for groups of 128 k).  A
// round here is one workgroup per CU (a CU holds two; one alone runs
// faster).  Costs relative to a 96-row workgroup: 64 rows 18/22, 128 rows
// 27/22 (measured on MI355X at M = 32 .. 4096, N = 14336, K = 4096, groups
// of 128 and 64 k).  Ties go to the taller tile.
int pick_rows(const GemmParams& p, bool tall)
{
    const int64_t cus = device_cus();
    auto cost = [&](int bm, int64_t w) { return w * ((((int64_t)p.M + bm - 1) / bm * p.num_n + cus - 1) / cus); };
    int best = kMaxBM;
    int64_t c = cost(kMaxBM, 22);
    if (tall && cost(kTallBM, 27) <= c) { best = kTallBM; c = cost(kTallBM, 27); }
    if (cost(kShortBM, 18) < c) best = kShortBM;
    return best;
}

template <typename ST, int Q, bool HAS_ZP, bool F32OUT>
void launch_h(const GemmParams& p, hipStream_t s)
{
    if constexpr (Q <= 2 && StageGeom<Q, (int)sizeof(ST), HAS_ZP, 0>::BM == kMaxBM) {
        int rows = g_prefill_rows.load(std::memory_order_relaxed);
        if (rows == 0) rows = pick_rows(p, Q == 1);
        if constexpr (Q == 1) {
            if (rows == kTallBM) { launch_k<ST, Q, HAS_ZP, F32OUT, kTallBM>(p, s); return; }
        }
        if (rows == kShortBM) { launch_k<ST, Q, HAS_ZP, F32OUT, kShortBM>(p, s); return; }
    }
    launch_k<ST, Q, HAS_ZP, F32OUT, 0>(p, s);
}

template <typename ST, int Q, bool HAS_ZP>
hipError_t launch_t(const GemmParams& p, hipStream_t s)
{
    if (p.row_scale)
        launch_h<ST, Q, HAS_ZP, true>(p, s);
    else
        launch_h<ST, Q, HAS_ZP, false>(p, s);
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

int set_prefill_rows(int rows)
{
    if (rows != 0 && rows != kShortBM && rows != kMaxBM && rows != kTallBM) return -1;
    return g_prefill_rows.exchange(rows);
}

// Largest K the kernel's 32-bit buffer ranges and offsets cover: the rows
// of A behind one buffer resource (at most 32 * K * 2 bytes) and the code
// bytes of a workgroup's BN / 16 tiles (BN / 16 * C * 1024) each stay below
// 2^31.
int64_t gemm_mfma_max_k()
{
    const int64_t lim = (int64_t(1) << 31) - 1;
    const int64_t by_a = lim / (2 * 32);
    const int64_t by_codes = lim / ((BN / 16) * 1024) * kChunkK;
    return by_a < by_codes ? by_a : by_codes;
}

hipError_t launch_gemm_mfma(const Layout& L, const WeightView& w, const void* a, int64_t m,
                            const Bias& bias, void* y, hipStream_t stream, const char** variant)
{
    GemmParams p;
    p.y32 = nullptr;
    p.row_scale = nullptr;
    p.bias32 = nullptr;
    p.bias32_stride = 0;
    p.pair_rows = 0;
    p.w = w.codes;   // the codes section starts the repacked buffer
    p.scales_off = L.scales_off;
    p.zp_off = L.zp_off;
    p.w_bytes = (uint32_t)L.total;
    p.a = static_cast<const _Float16*>(a);
    p.y = static_cast<__half*>(y);
    p.bias = static_cast<const __half*>(bias.ptr);
    p.bias_stride = bias.row_stride;
    p.bias_after_round = bias.after_round;
    p.M = (int)m;
    p.N = (int)L.N;
    p.K = (int)L.K;
    p.C = (int)L.C;
    p.T = (int)L.T;
    p.num_m = 0;   // set per tile height in launch_t
    p.num_n = (int)((L.N + BN - 1) / BN);
    p.vec_store = (L.N % 8 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0) ? 1 : 0;
    p.flags_off = L.flags_off;
    if (variant) *variant = "gemm_mfma_32x32x16";
    if (L.ss == 2)
        return L.has_zp ? launch_q<__half, true>(L, p, stream) : launch_q<__half, false>(L, p, stream);
    return L.has_zp ? launch_q<float, true>(L, p, stream) : launch_q<float, false>(L, p, stream);
}

hipError_t launch_gemm_mfma_f32(const Layout& L, const WeightView& w, const void* a16, int64_t m,
                                const float* row_scale, const float* bias, float* y, hipStream_t stream,
                                const char** variant, int pair_rows, int64_t bias_stride)
{
    GemmParams p;
    p.w = w.codes;
    p.scales_off = L.scales_off;
    p.zp_off = L.zp_off;
    p.w_bytes = (uint32_t)L.total;
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
    p.T = (int)L.T;
    p.num_m = 0;   // set per tile height in launch_t
    p.num_n = (int)((L.N + BN - 1) / BN);
    p.vec_store = (L.N % 4 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0) ? 1 : 0;
    p.flags_off = L.flags_off;
    if (variant) *variant = pair_rows ? "gemm_mfma_32x32x16_f32act" : "gemm_mfma_32x32x16_accuracy4";
    if (L.ss == 2)
        return L.has_zp ? launch_q<__half, true>(L, p, stream) : launch_q<__half, false>(L, p, stream);
    return L.has_zp ? launch_q<float, true>(L, p, stream) : launch_q<float, false>(L, p, stream);
}

}  // namespace mnb
