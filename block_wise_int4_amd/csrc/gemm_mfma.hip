// gemm_mfma.hip -- prefill GEMM (M > 16) on the gfx950 matrix cores.
//
// Method: onnx-runtime-ep-cuda 0.1.0-dev.6, src/kernels/marlin_gemm.rs
// (matmul_nbits_marlin_gemm_f16 and its module doc): weights enter the matrix
// multiply centred but unscaled, as exact fp16 (code - zp); each group's
// products accumulate in fp32 from zero and the group's scale multiplies that
// partial after the group's accumulate, so the accumulator never carries a
// scale that varies along K.
//
// gfx950 design.  Workgroup tile 128 (M) x 256 (N), 4 waves, each wave
// 128 x 64 (8 x 4 tiles of v_mfma_f32_16x16x32_f16).  A streams through LDS
// in 128-k chunks, double-buffered, stored with a 16-byte-segment XOR swizzle
// so fragment reads are bank-conflict free.  B never touches LDS: each lane
// loads one 16-byte code word per 16-column tile per chunk (already in the
// MFMA B-operand distribution), unpacks it to fp16 in registers and feeds
// eight MFMAs with it.  Workgroup ids are remapped so that the tiles resident
// on one XCD at a time share A rows and B columns in that XCD's L2.
#include "mnb_device.hpp"
#include "mnb_internal.hpp"

namespace mnb {

namespace {

constexpr int BN = 256;            // columns per workgroup (16 tiles)
constexpr int WAVES = 4;           // each wave: all BM rows x 64 columns
constexpr int TW = 4;              // 16-column tiles per wave
constexpr int SEGS = kChunkK / 8;  // 16-byte segments per A row per chunk
constexpr int kGroupM = 4;         // m-blocks per XCD-local group

struct GemmParams {
    const u4_t* codes;
    const void* scales;
    const uint8_t* zp;
    const _Float16* a;
    __half* y;
    int M, N, K, C;
    int T;                 // column tiles
    int num_m, num_n;      // workgroup grid
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

// RB row blocks of 16 per wave: BM = 16 * RB rows per workgroup.
template <typename ST, int Q, bool HAS_ZP, int RB>
__global__ __launch_bounds__(WAVES * 64, 1) void gemm_mfma_kernel(GemmParams p)
{
    constexpr int BM = RB * 16;
    __shared__ u4_t As[2][BM * SEGS];   // 2 x BM x 256 bytes

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int i = lane & 15;
    const int h = lane >> 4;
    int mb, nb;
    tile_of(blockIdx.x, p.num_m, p.num_n, mb, nb);
    const int m0 = mb * BM;
    const int C = p.C;
    const int K = p.K;

    // this wave's 4 tiles (clamped for loads; stores are masked by N)
    int64_t tile_base[TW];
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
        int t = nb * (BN / 16) + wave * TW + tt;
        if (t >= p.T) t = p.T - 1;
        tile_base[tt] = (int64_t)t * C;
    }

    // A staging: thread -> (row = tid/16 + 16*it, segment = tid%16)
    const int seg = tid & 15;
    const int row0 = tid >> 4;
    u4_t stage[BM / 16];
    auto load_a = [&](int c) {
#pragma unroll
        for (int it = 0; it < BM / 16; ++it) {
            const int r = row0 + 16 * it;
            const int m = m0 + r;
            const int k = c * kChunkK + seg * 8;
            if (m < p.M && k < K)
                stage[it] = *reinterpret_cast<const u4_t*>(p.a + (int64_t)m * K + k);
            else
                stage[it] = u4_t{0u, 0u, 0u, 0u};
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int it = 0; it < BM / 16; ++it) {
            const int r = row0 + 16 * it;
            As[buf][r * SEGS + (seg ^ (r & 15))] = stage[it];
        }
    };

    // B operands and per-group constants of one chunk
    constexpr int NSC = Q <= 4 ? Q : 8;
    u4_t bw[TW];
    float sc[TW][NSC];
    uint32_t zw[TW];
    auto load_b = [&](int c) {
#pragma unroll
        for (int tt = 0; tt < TW; ++tt) {
            const int64_t chunk = tile_base[tt] + c;
            bw[tt] = __builtin_nontemporal_load(p.codes + chunk * 64 + lane);
            const ST* sp = static_cast<const ST*>(p.scales) + chunk * kTileN * Q;
#pragma unroll
            for (int q = 0; q < NSC; ++q) sc[tt][q] = to_f32(sp[slot_of(i, q, Q)]);
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
    };

    f4_t total[RB][TW];
    f4_t grp[RB][TW];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int tt = 0; tt < TW; ++tt) {
            total[rb][tt] = f4_t{0.f, 0.f, 0.f, 0.f};
            grp[rb][tt] = f4_t{0.f, 0.f, 0.f, 0.f};
        }

    load_a(0);
    load_b(0);
    store_a(0);
    __syncthreads();

    for (int c = 0; c < C; ++c) {
        const int buf = c & 1;
        // current chunk's B state; next chunk's loads go in flight
        u4_t bcur[TW];
        float scur[TW][NSC];
        uint32_t zcur[TW];
#pragma unroll
        for (int tt = 0; tt < TW; ++tt) {
            bcur[tt] = bw[tt];
            zcur[tt] = zw[tt];
#pragma unroll
            for (int q = 0; q < NSC; ++q) scur[tt][q] = sc[tt][q];
        }
        if (c + 1 < C) {
            load_a(c + 1);
            load_b(c + 1);
        }

#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h8_t afr[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int r = rb * 16 + i;
                const int sgi = 4 * j + h;
                afr[rb] = __builtin_bit_cast(h8_t, As[buf][r * SEGS + (sgi ^ (r & 15))]);
            }
#pragma unroll
            for (int tt = 0; tt < TW; ++tt) {
                const uint32_t dw = j == 0 ? bcur[tt].x : j == 1 ? bcur[tt].y : j == 2 ? bcur[tt].z : bcur[tt].w;
                const int zs = Q == 1 ? 0 : (Q == 2 ? (j >> 1) : j);
                const uint32_t z = HAS_ZP ? (zcur[tt] >> (4 * zs)) & 15u : 8u;
                h2_t q[4];
                unpack8(dw, zp_const(z), q);
                const h8_t b = make_b(q);
                if (Q <= 4) {
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) grp[rb][tt] = mfma16(afr[rb], b, grp[rb][tt]);
                    constexpr int steps = 4 / (Q <= 4 ? Q : 1);
                    if ((j + 1) % steps == 0) {
                        const float s = scur[tt][Q == 1 ? 0 : (Q == 2 ? (j >> 1) : j)];
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                total[rb][tt][r] = __builtin_fmaf(grp[rb][tt][r], s, total[rb][tt][r]);
                            grp[rb][tt] = f4_t{0.f, 0.f, 0.f, 0.f};
                        }
                    }
                } else {
                    h8_t zero;
#pragma unroll
                    for (int e = 0; e < 8; ++e) zero[e] = (_Float16)0.0f;
                    const h8_t be = (h < 2) ? b : zero;
                    const h8_t bo = (h < 2) ? zero : b;
                    const float se = scur[tt][2 * j], so = scur[tt][2 * j + 1];
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        const f4_t ge = mfma16(afr[rb], be, f4_t{0.f, 0.f, 0.f, 0.f});
                        const f4_t go = mfma16(afr[rb], bo, f4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            total[rb][tt][r] = __builtin_fmaf(ge[r], se, total[rb][tt][r]);
                            total[rb][tt][r] = __builtin_fmaf(go[r], so, total[rb][tt][r]);
                        }
                    }
                }
            }
        }

        if (c + 1 < C) store_a(buf ^ 1);
        __syncthreads();
    }

    // epilogue: D lane layout row 4h + r, column i of each 16x16 tile
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
        const int n = nb * BN + wave * 64 + tt * 16 + i;
        if (n >= p.N) continue;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + rb * 16 + 4 * h + r;
                if (m < p.M) p.y[(int64_t)m * p.N + n] = __float2half_rn(total[rb][tt][r]);
            }
        }
    }
}

// Row blocks per wave: 8 (128-row tiles) for one group per chunk; groups
// smaller than a chunk keep more per-group state live, so they use 64 rows.
constexpr int rb_for(int Q) { return Q == 1 ? 8 : 4; }

template <typename ST, int Q, bool HAS_ZP>
hipError_t launch_t(GemmParams p, hipStream_t s)
{
    constexpr int RB = rb_for(Q);
    p.num_m = (p.M + RB * 16 - 1) / (RB * 16);
    const int blocks = p.num_m * p.num_n;
    gemm_mfma_kernel<ST, Q, HAS_ZP, RB><<<dim3(blocks), dim3(WAVES * 64), 0, s>>>(p);
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

hipError_t launch_gemm_mfma(const Layout& L, const WeightView& w, const void* a, int64_t m,
                            void* y, hipStream_t stream, const char** variant)
{
    GemmParams p;
    p.codes = reinterpret_cast<const u4_t*>(w.codes);
    p.scales = w.scales;
    p.zp = w.zp;
    p.a = static_cast<const _Float16*>(a);
    p.y = static_cast<__half*>(y);
    p.M = (int)m;
    p.N = (int)L.N;
    p.K = (int)L.K;
    p.C = (int)L.C;
    p.T = (int)L.T;
    p.num_m = 0;  // set per row-tile height in launch_t
    p.num_n = (int)((L.N + BN - 1) / BN);
    if (variant) *variant = L.Q == 1 ? "gemm_mfma_128x256" : "gemm_mfma_64x256";
    if (L.ss == 2)
        return L.has_zp ? launch_q<__half, true>(L, p, stream) : launch_q<__half, false>(L, p, stream);
    return L.has_zp ? launch_q<float, true>(L, p, stream) : launch_q<float, false>(L, p, stream);
}

}  // namespace mnb
