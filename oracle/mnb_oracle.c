/*
 * mnb_oracle.c -- plain, slow, obviously-correct CPU oracle for the block-wise
 * int4 weight-only matmul in the ONNX MatMulNBits layout.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant with the HIP library under block_wise_int4_amd/,
 * and the product path never calls it.
 *
 * Everything is computed in IEEE-754 binary64, in the order the definitions
 * state, with no blocking, fusion or reordering.
 *
 * Sources (web pages, cited by title and item):
 *  [FMT]  onnx-runtime-ep-cuda 0.1.0-dev.6, src/kernels/marlin_gemm.rs --
 *         module doc, section "ONNX MatMulNBits int4 format (input to the
 *         repack)": Y[M,N] = A[M,K] . dequant(B)^T with
 *         dequant(B)[n,k] = (code[n,k] - zp[n,k/group]) * scale[n,k/group];
 *         packed [N, k_blocks, group/2], low nibble for even k; zero points
 *         [N, ceil(k_blocks/2)], low nibble for even block; default zp 8.
 *  [DQ]   onnx-runtime-ep-cuda 0.1.0-dev.3, src/kernels/matmul_nbits.rs --
 *         kernel matmul_nbits_dequant_f32 (the same indexing written as a
 *         dequantize-to-dense step) and the f64 dequant-and-matmul oracle
 *         loop of test fp16_gemv_matches_dequant_reference.
 *  [SILU] ferrox-cuda gpu.rs -- kernel silu_mul_f32: silu(g) * u with
 *         silu(x) = x / (1 + e^-x); matmul_nbits.rs (dev.3) --
 *         gate_up_silu_f32 states the same function in a two-branch form.
 *  [GIDX] onnx-runtime-ep-cuda 0.1.0-dev.3, src/kernels/matmul_nbits.rs --
 *         kernel matmul_nbits_dequant_f32 with group_indices, and the
 *         g_idx checks of MatMulNBitsFactory (optional input 4, int32 [K],
 *         every value in 0..k_blocks-1): the code of (n,k) stays where the
 *         format puts it, the scale and zero point are those of group
 *         g_idx[k] instead of k/group; a group outside the range dequantizes
 *         to 0.
 *  [BIAS] onnx-runtime-ep-cuda 0.1.0-dev.3, src/kernels/matmul_nbits.rs --
 *         the fp16 GEMV bias epilogue (fold_bias_f16) and the bias stage
 *         records of the GEMV dispatch; marlin_gemm.rs (dev.6) -- the same
 *         epilogue (fold_bias) with a per-row bias stride.  An optional fp16
 *         bias b[n] (or, with a row stride, b[m*stride + n]) is added to the
 *         fp32 accumulator in one of two ways: added in fp32 and rounded once
 *         to fp16 (the operator's own bias), or rounded to fp16 first and then
 *         added in fp32 and rounded again (a folded elementwise Add, which
 *         must stay byte-identical to the two-operator path).
 *  [ACC4] onnx-runtime-ep-cuda 0.1.0-dev.3, src/kernels/matmul_nbits.rs --
 *         the accuracy_level=4 path of the fp32 operator (fp32 A, fp32
 *         scales, fp32 Y): kernel matmul_nbits_accuracy4 (any M, block size,
 *         zero points) and the M=1 pair matmul_nbits_quantize_accuracy4_block32
 *         / matmul_nbits_gemv_accuracy4_block32.  Each row of A is quantized
 *         to int8 with one scale, max|a|/127 in binary32; a code is a*(1/scale)
 *         in binary32, clamped to [-127, 127] and rounded half away from
 *         zero; the integer dot of each block, sum q*(code - zp), is scaled
 *         by that block's weight scale and the row's activation scale; a row
 *         whose max is 0 gives the bias (or 0).
 *
 * Parity pins for every function live in tests/test_oracle.py (worked
 * examples, exhaustive nibble decode, pack/unpack identity, code==zp gives
 * zero, exact-rational brute force, integer special case, fp16 decode against
 * numpy for all 65536 bit patterns, silu against scipy's expit, binary16
 * rounding against numpy's conversion at every value and every tie, the bias
 * epilogue against numpy binary32 arithmetic and hand-worked cases).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- scalar decoding --------------------------------------------------- */

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exponent 0 = zero/subnormal (fraction * 2^-24), exponent 31 =
 * infinity (fraction 0) or NaN. */
double oracle_f16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 31;
    const int frac = h & 1023;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);
    } else if (expo == 31) {
        v = frac == 0 ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25);
    }
    return sign ? -v : v;
}

void oracle_decode_f16(const uint16_t* h, int64_t count, double* out)
{
    for (int64_t i = 0; i < count; ++i) out[i] = oracle_f16_to_f64(h[i]);
}

void oracle_decode_f32(const float* f, int64_t count, double* out)
{
    for (int64_t i = 0; i < count; ++i) out[i] = (double)f[i];
}

/* ---- the format [FMT] -------------------------------------------------- */

static int64_t k_blocks_of(int64_t K, int64_t g) { return (K + g - 1) / g; }
static int64_t zp_row_bytes_of(int64_t kb) { return (kb + 1) / 2; }

/* code[n,k]: byte (n*k_blocks + k/g) * (g/2) + (k mod g)/2, low nibble for
 * even (k mod g), high nibble for odd. */
int oracle_code(const uint8_t* packed, int64_t n, int64_t k, int64_t K, int64_t g)
{
    const int64_t kb = k_blocks_of(K, g);
    const int64_t blob = g / 2;
    const int64_t block = k / g;
    const int64_t within = k % g;
    const uint8_t byte = packed[(n * kb + block) * blob + within / 2];
    return (within % 2 == 0) ? (byte & 15) : (byte >> 4);
}

/* zp[n,b]: 8 when no zero points are given; otherwise byte n*zrb + b/2, low
 * nibble for even b, high nibble for odd b. */
int oracle_zero_point(const uint8_t* zero_points, int64_t n, int64_t b, int64_t kb)
{
    if (zero_points == NULL) return 8;
    const uint8_t byte = zero_points[n * zp_row_bytes_of(kb) + b / 2];
    return (b % 2 == 0) ? (byte & 15) : (byte >> 4);
}

/* codes u8[N,K] in plain row-major order. */
void oracle_unpack_codes(const uint8_t* packed, int64_t N, int64_t K, int64_t g, uint8_t* codes)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            codes[n * K + k] = (uint8_t)oracle_code(packed, n, k, K, g);
}

/* zero points u8[N,kb] in plain row-major order (8 everywhere when absent). */
void oracle_unpack_zero_points(const uint8_t* zero_points, int64_t N, int64_t kb, uint8_t* z)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < kb; ++b)
            z[n * kb + b] = (uint8_t)oracle_zero_point(zero_points, n, b, kb);
}

/* dequant(B)[n,k] = (code[n,k] - zp[n,k/g]) * scale[n,k/g], in fp64.  The
 * scales arrive already decoded to fp64 ([N, k_blocks]).  The product is
 * exact: a 5-bit integer times a scale of at most 24 significant bits. */
void oracle_dequant(const uint8_t* packed, const double* scales, const uint8_t* zero_points,
                    int64_t N, int64_t K, int64_t g, double* w)
{
    const int64_t kb = k_blocks_of(K, g);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            const int64_t b = k / g;
            const int code = oracle_code(packed, n, k, K, g);
            const int zp = oracle_zero_point(zero_points, n, b, kb);
            w[n * K + k] = ((double)code - (double)zp) * scales[n * kb + b];
        }
    }
}

/* Y[m,n] = sum_{k=0}^{K-1} A[m,k] * W[n,k], k ascending, in fp64; alongside,
 * Bnd[m,n] = sum_k |A[m,k] * W[n,k]| (the magnitude the tolerance scales
 * with).  Naive loop over output elements; threads > 0 sets the OpenMP team. */
void oracle_matmul(const double* A, const double* W, int64_t M, int64_t N, int64_t K,
                   double* Y, double* Bnd, int threads)
{
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#pragma omp parallel for collapse(2) schedule(static)
#endif
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = A[m * K + k] * W[n * K + k];
                acc += p;
                mag += fabs(p);
            }
            Y[m * N + n] = acc;
            if (Bnd) Bnd[m * N + n] = mag;
        }
    }
}

/* The whole method for a chosen set of output elements (m_i, n_i): each
 * weight is decoded from the packed bytes on the fly, as in [DQ]'s f32
 * GEMV, so no dense [N,K] matrix is built.  Used where the full product is
 * too large for a CPU check. */
void oracle_matmul_nbits_at(const double* A, const uint8_t* packed, const double* scales,
                            const uint8_t* zero_points, int64_t N, int64_t K, int64_t g,
                            const int64_t* ms, const int64_t* ns, int64_t count,
                            double* Y, double* Bnd, int threads)
{
    const int64_t kb = k_blocks_of(K, g);
    (void)N;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#pragma omp parallel for schedule(dynamic, 16)
#endif
    for (int64_t i = 0; i < count; ++i) {
        const int64_t m = ms[i], n = ns[i];
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const int64_t b = k / g;
            const int code = oracle_code(packed, n, k, K, g);
            const int zp = oracle_zero_point(zero_points, n, b, kb);
            const double w = ((double)code - (double)zp) * scales[n * kb + b];
            const double p = A[m * K + k] * w;
            acc += p;
            mag += fabs(p);
        }
        Y[i] = acc;
        if (Bnd) Bnd[i] = mag;
    }
}

/* All M x N outputs of the method, decoding weights on the fly (no dense
 * matrix): the CPU baseline times this over a bounded sample of rows. */
void oracle_matmul_nbits(const double* A, const uint8_t* packed, const double* scales,
                         const uint8_t* zero_points, int64_t M, int64_t N, int64_t K, int64_t g,
                         double* Y, double* Bnd, int threads)
{
    const int64_t kb = k_blocks_of(K, g);
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#pragma omp parallel for collapse(2) schedule(static)
#endif
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t b = k / g;
                const int code = oracle_code(packed, n, k, K, g);
                const int zp = oracle_zero_point(zero_points, n, b, kb);
                const double w = ((double)code - (double)zp) * scales[n * kb + b];
                const double p = A[m * K + k] * w;
                acc += p;
                mag += fabs(p);
            }
            Y[m * N + n] = acc;
            if (Bnd) Bnd[m * N + n] = mag;
        }
    }
}

/* [SILU]: S = silu(G) * U with silu(x) = x / (1 + e^-x). */
void oracle_swiglu(const double* G, const double* U, int64_t count, double* S)
{
    for (int64_t i = 0; i < count; ++i) {
        const double x = G[i];
        S[i] = (x / (1.0 + exp(-x))) * U[i];
    }
}

/* ---- the inverse direction, for fixtures ------------------------------- */

/* Pack codes u8[N,K] (values 0..15) into [N, k_blocks, g/2] per [FMT];
 * nibbles past K in the last block are written as 0. */
void oracle_pack_codes(const uint8_t* codes, int64_t N, int64_t K, int64_t g, uint8_t* packed)
{
    const int64_t kb = k_blocks_of(K, g);
    const int64_t blob = g / 2;
    for (int64_t i = 0; i < N * kb * blob; ++i) packed[i] = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            const int64_t within = k % g;
            const int64_t at = (n * kb + k / g) * blob + within / 2;
            const uint8_t c = codes[n * K + k] & 15;
            packed[at] |= (within % 2 == 0) ? c : (uint8_t)(c << 4);
        }
    }
}

/* Pack zero points u8[N,kb] (0..15) into [N, ceil(kb/2)] per [FMT]; the high
 * nibble of the last byte of a row with odd kb is written as 0. */
void oracle_pack_zero_points(const uint8_t* z, int64_t N, int64_t kb, uint8_t* zero_points)
{
    const int64_t zrb = zp_row_bytes_of(kb);
    for (int64_t i = 0; i < N * zrb; ++i) zero_points[i] = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < kb; ++b) {
            const uint8_t v = z[n * kb + b] & 15;
            zero_points[n * zrb + b / 2] |= (b % 2 == 0) ? v : (uint8_t)(v << 4);
        }
    }
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- output rounding and the bias epilogue [BIAS] ------------------------ */

/* The binary16 value nearest to x, ties to the even significand (the
 * standard's default rounding); beyond the largest finite value (65504) the
 * result is infinity when x is at least 65520 (the tie between 65504 and
 * 2^16 goes to the even 2^16, which overflows); NaN gives a quiet NaN; the sign
 * of zero is kept.  Returns the bit pattern. */
uint16_t oracle_round_f16(double x)
{
    if (isnan(x)) return 0x7E00;
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    const double a = fabs(x);
    if (isinf(a)) return sign | 0x7C00;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                      /* a = f * 2^e, f in [0.5, 1) */
    /* spacing of binary16 values around a: 2^(e-11) in a normal binade,
     * 2^-24 among the subnormals and in the lowest normal binade */
    int ulp = e - 11;
    if (ulp < -24) ulp = -24;
    const double q = ldexp(a, -ulp);   /* a in units of that spacing, exact */
    const double lo = floor(q);
    const double rest = q - lo;        /* exact */
    double n = lo;
    if (rest > 0.5 || (rest == 0.5 && fmod(lo, 2.0) != 0.0)) n = lo + 1.0;
    const double v = ldexp(n, ulp);    /* the rounded magnitude */
    if (v > 65504.0) return sign | 0x7C00;
    if (v < ldexp(1.0, -14)) return sign | (uint16_t)(v * ldexp(1.0, 24));   /* subnormal */
    int ev;
    frexp(v, &ev);                     /* v = f * 2^ev: exponent field ev + 14 */
    const double frac = ldexp(v, 11 - ev) - 1024.0;
    return sign | (uint16_t)((ev + 14) << 10) | (uint16_t)frac;
}

void oracle_round_f16_array(const double* x, int64_t count, uint16_t* out)
{
    for (int64_t i = 0; i < count; ++i) out[i] = oracle_round_f16(x[i]);
}

/* One fp16 output with a bias: acc is the binary32 accumulator, b the bias
 * (binary16 bits).  after_round 0: acc + b in binary32, rounded once to
 * binary16.  after_round 1: acc rounded to binary16, then + b in binary32,
 * rounded to binary16 again. */
uint16_t oracle_bias_f16(float acc, uint16_t b, int after_round)
{
    const float bf = (float)oracle_f16_to_f64(b);   /* exact: binary16 is a subset of binary32 */
    float base = acc;
    if (after_round) base = (float)oracle_f16_to_f64(oracle_round_f16((double)acc));
    const float sum = base + bf;                     /* one binary32 addition */
    return oracle_round_f16((double)sum);
}

void oracle_bias_f16_array(const float* acc, const uint16_t* b, int64_t count, int after_round,
                           uint16_t* out)
{
    for (int64_t i = 0; i < count; ++i) out[i] = oracle_bias_f16(acc[i], b[i], after_round);
}

/* ---- act-order group indices [GIDX] -------------------------------------- */

/* dequant(B)[n,k] = (code[n,k] - zp[n,g_idx[k]]) * scale[n,g_idx[k]] in fp64,
 * and 0 for a group index outside 0..k_blocks-1. */
void oracle_dequant_gidx(const uint8_t* packed, const double* scales, const uint8_t* zero_points,
                         const int32_t* g_idx, int64_t N, int64_t K, int64_t g, double* w)
{
    const int64_t kb = k_blocks_of(K, g);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            const int64_t grp = g_idx[k];
            if (grp < 0 || grp >= kb) {
                w[n * K + k] = 0.0;
                continue;
            }
            const int code = oracle_code(packed, n, k, K, g);
            const int zp = oracle_zero_point(zero_points, n, grp, kb);
            w[n * K + k] = ((double)code - (double)zp) * scales[n * kb + grp];
        }
    }
}

/* ---- int8 activations, accuracy_level 4 [ACC4] --------------------------- */

/* The int8 activation codes of accuracy_level 4 (the quantize kernel of
 * onnx-runtime-ep-cuda 0.1.0-dev.3, src/kernels/matmul_nbits.rs,
 * matmul_nbits_quantize_accuracy4_block32), from the rule it implements:
 * one binary32 scale per row, the largest magnitude over 127, and each code
 * the binary32 value a * (1/scale) clamped to [-127, 127] and rounded to the
 * nearest integer, halves away from zero.  The binary32 operations are
 * evaluated exactly in binary64 and rounded once to binary32 (exact for a
 * product of two binary32 values; for a quotient, rounding binary64 to
 * binary32 is innocuous since 53 >= 2*24 + 2), so every step below is the
 * correctly rounded binary32 result.  Readings: a NaN takes no part in the
 * maximum, and the clamp sends it to -127; a row whose largest magnitude is 0
 * has scale 0 and codes 0; an overflowing reciprocal is +inf and the codes
 * follow from it (nonzero values +-127, zeros -127 since 0 * inf is NaN). */

static float b32_quotient(float x, float y) { return (float)((double)x / (double)y); }
static float b32_product(float x, float y) { return (float)((double)x * (double)y); }

/* nearest integer, halves away from zero; |x| <= 127 here, so x + 0.5 is
 * exact in binary64 */
static int nearest_away(float x)
{
    const double m = floor(fabs((double)x) + 0.5);
    return x < 0 ? -(int)m : (int)m;
}

static float largest_magnitude(const float* a, int64_t K)
{
    float best = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        const float v = a[k] < 0 ? -a[k] : a[k];
        if (v == v && v > best) best = v;   /* NaN compares false */
    }
    return best;
}

void oracle_acc4_quantize_row(const float* a, int64_t K, int8_t* q, float* scale)
{
    const float top = largest_magnitude(a, K);
    if (top == 0.0f) {
        for (int64_t k = 0; k < K; ++k) q[k] = 0;
        *scale = 0.0f;
        return;
    }
    const float s = b32_quotient(top, 127.0f);
    const float inv = b32_quotient(1.0f, s);
    for (int64_t k = 0; k < K; ++k) {
        float x = b32_product(a[k], inv);
        if (!(x >= -127.0f)) x = -127.0f;   /* below the range, or NaN */
        if (x > 127.0f) x = 127.0f;
        q[k] = (int8_t)nearest_away(x);
    }
    *scale = s;
}

void oracle_acc4_quantize(const float* a, int64_t M, int64_t K, int8_t* q, float* scale)
{
    for (int64_t m = 0; m < M; ++m) oracle_acc4_quantize_row(a + m * K, K, q + m * K, scale + m);
}

/* Y[m,n] = scale_a[m] * (sum_b scale[n,b] * dot[m,n,b]) + bias[n] in fp64,
 * with dot[m,n,b] = sum over k in block b of q[m,k] * (code[n,k] - zp[n,b]),
 * an exact integer; a row with scale_a 0 gives bias[n] (or 0).  The
 * activation scale multiplies the sum over blocks, as in the M=1 kernel of
 * the pages (for finite values the same number as scaling every block; for
 * an infinite activation, whose scale is infinite, the result is an
 * infinity of the sum's sign).  bias may be NULL; scales are the decoded
 * weight scales [N, k_blocks].  Bnd[m,n] is the error scale of a binary32
 * evaluation: |scale_a| * sum_b |scale[n,b] * dot| + |bias[n]|.  q and
 * scale_a (the quantized rows, [M,K] and [M]) are written too. */
void oracle_acc4_matmul(const float* a, int64_t M, int64_t K, const uint8_t* packed,
                        const double* scales, const uint8_t* zero_points, int64_t N, int64_t g,
                        const float* bias, double* Y, double* Bnd, int8_t* q, float* scale_a)
{
    const int64_t kb = k_blocks_of(K, g);
    oracle_acc4_quantize(a, M, K, q, scale_a);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            const double b = bias ? (double)bias[n] : 0.0;
            const double sa = (double)scale_a[m];
            double inner = 0.0, mag = 0.0;
            if (sa != 0.0) {
                for (int64_t blk = 0; blk < kb; ++blk) {
                    const int zp = oracle_zero_point(zero_points, n, blk, kb);
                    int64_t dot = 0;
                    const int64_t end = (blk + 1) * g < K ? (blk + 1) * g : K;
                    for (int64_t k = blk * g; k < end; ++k)
                        dot += (int64_t)q[m * K + k] * (oracle_code(packed, n, k, K, g) - zp);
                    const double term = scales[n * kb + blk] * (double)dot;
                    inner += term;
                    mag += fabs(term);
                }
            }
            const double y = sa != 0.0 ? sa * inner : 0.0;
            Y[m * N + n] = y + b;
            Bnd[m * N + n] = (sa != 0.0 ? fabs(sa) * mag : 0.0) + fabs(b);
        }
    }
}
