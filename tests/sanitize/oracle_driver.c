/* The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every
 * function on small operands, including the edge cases its pins use (K not a
 * multiple of the group, an odd number of blocks, group indices out of range,
 * NaN, infinite and subnormal activations, binary16 boundaries).  Results are
 * checked by the pins; this run checks memory and arithmetic safety only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_f16_to_f64(uint16_t h);
void oracle_decode_f16(const uint16_t* h, int64_t count, double* out);
void oracle_decode_f32(const float* f, int64_t count, double* out);
int oracle_code(const uint8_t* packed, int64_t n, int64_t k, int64_t K, int64_t g);
int oracle_zero_point(const uint8_t* zero_points, int64_t n, int64_t b, int64_t kb);
void oracle_unpack_codes(const uint8_t* packed, int64_t N, int64_t K, int64_t g, uint8_t* codes);
void oracle_unpack_zero_points(const uint8_t* zero_points, int64_t N, int64_t kb, uint8_t* z);
void oracle_dequant(const uint8_t* packed, const double* scales, const uint8_t* zero_points, int64_t N,
                    int64_t K, int64_t g, double* w);
void oracle_matmul(const double* A, const double* W, int64_t M, int64_t N, int64_t K, double* Y, double* B,
                   int threads);
void oracle_matmul_nbits(const double* A, const uint8_t* packed, const double* scales,
                         const uint8_t* zero_points, int64_t M, int64_t N, int64_t K, int64_t g, double* Y,
                         double* B, int threads);
void oracle_matmul_nbits_at(const double* A, const uint8_t* packed, const double* scales,
                            const uint8_t* zero_points, int64_t N, int64_t K, int64_t g,
                            const int64_t* ms, const int64_t* ns, int64_t count, double* Y, double* B,
                            int threads);
void oracle_swiglu(const double* G, const double* U, int64_t count, double* S);
void oracle_pack_codes(const uint8_t* codes, int64_t N, int64_t K, int64_t g, uint8_t* packed);
void oracle_pack_zero_points(const uint8_t* z, int64_t N, int64_t kb, uint8_t* zero_points);
uint16_t oracle_round_f16(double x);
uint16_t oracle_bias_f16(float acc, uint16_t b, int after_round);
void oracle_dequant_gidx(const uint8_t* packed, const double* scales, const uint8_t* zero_points,
                         const int32_t* g_idx, int64_t N, int64_t K, int64_t g, double* w);
void oracle_acc4_quantize(const float* a, int64_t M, int64_t K, int8_t* q, float* scale);
void oracle_acc4_matmul(const float* a, int64_t M, int64_t K, const uint8_t* packed, const double* scales,
                        const uint8_t* zero_points, int64_t N, int64_t g, const float* bias, double* Y,
                        double* Bnd, int8_t* q, float* scale_a);

static uint32_t rnd_state = 2463534242u;
static uint32_t rnd(void)
{
    rnd_state ^= rnd_state << 13;
    rnd_state ^= rnd_state >> 17;
    rnd_state ^= rnd_state << 5;
    return rnd_state;
}

static void run_shape(int64_t M, int64_t N, int64_t K, int64_t g)
{
    const int64_t kb = (K + g - 1) / g, zrb = (kb + 1) / 2;
    uint8_t* codes = malloc((size_t)(N * K));
    uint8_t* packed = malloc((size_t)(N * kb * (g / 2)));
    uint8_t* z = malloc((size_t)(N * kb));
    uint8_t* zp = malloc((size_t)(N * zrb));
    double* s = malloc(sizeof(double) * (size_t)(N * kb));
    double* A = malloc(sizeof(double) * (size_t)(M * K));
    float* Af = malloc(sizeof(float) * (size_t)(M * K));
    double* W = malloc(sizeof(double) * (size_t)(N * K));
    double* Y = malloc(sizeof(double) * (size_t)(M * N));
    double* B = malloc(sizeof(double) * (size_t)(M * N));
    int32_t* gi = malloc(sizeof(int32_t) * (size_t)K);
    int8_t* q = malloc((size_t)(M * K));
    float* sa = malloc(sizeof(float) * (size_t)M);
    float* bias = malloc(sizeof(float) * (size_t)N);
    for (int64_t i = 0; i < N * K; ++i) codes[i] = (uint8_t)(rnd() & 15u);
    for (int64_t i = 0; i < N * kb; ++i) {
        z[i] = (uint8_t)(rnd() & 15u);
        s[i] = 0.005 + (rnd() % 1000) * 1e-5;
    }
    for (int64_t i = 0; i < M * K; ++i) {
        Af[i] = (float)((int)(rnd() % 2001) - 1000) / 300.0f;
        A[i] = Af[i];
    }
    for (int64_t n = 0; n < N; ++n) bias[n] = (float)n * 0.25f;
    /* edge rows of the int8 quantization: NaN, infinity, subnormal, zero */
    if (M >= 4) {
        Af[0 * K + 1] = NAN;
        Af[1 * K + 0] = INFINITY;
        for (int64_t k = 0; k < K; ++k) Af[2 * K + k] = k % 3 ? 1e-40f : 0.0f;
        for (int64_t k = 0; k < K; ++k) Af[3 * K + k] = 0.0f;
    }
    for (int64_t k = 0; k < K; ++k) gi[k] = (int32_t)(k % 5 == 0 ? kb : (int64_t)(rnd() % (uint32_t)kb));
    gi[0] = -1;
    oracle_pack_codes(codes, N, K, g, packed);
    oracle_pack_zero_points(z, N, kb, zp);
    oracle_unpack_codes(packed, N, K, g, codes);
    oracle_unpack_zero_points(zp, N, kb, z);
    (void)oracle_code(packed, N - 1, K - 1, K, g);
    (void)oracle_zero_point(zp, N - 1, kb - 1, kb);
    (void)oracle_zero_point(NULL, 0, 0, kb);
    oracle_dequant(packed, s, zp, N, K, g, W);
    oracle_dequant(packed, s, NULL, N, K, g, W);
    oracle_dequant_gidx(packed, s, zp, gi, N, K, g, W);
    oracle_matmul(A, W, M, N, K, Y, B, 2);
    oracle_matmul_nbits(A, packed, s, zp, M, N, K, g, Y, B, 2);
    {
        int64_t ms[3] = {0, M - 1, M / 2}, ns[3] = {N - 1, 0, N / 2};
        double y3[3], b3[3];
        oracle_matmul_nbits_at(A, packed, s, zp, N, K, g, ms, ns, 3, y3, b3, 1);
    }
    oracle_swiglu(Y, B, M * N, W);
    oracle_acc4_quantize(Af, M, K, q, sa);
    oracle_acc4_matmul(Af, M, K, packed, s, zp, N, g, bias, Y, B, q, sa);
    oracle_acc4_matmul(Af, M, K, packed, s, NULL, N, g, NULL, Y, B, q, sa);
    free(codes); free(packed); free(z); free(zp); free(s); free(A); free(Af); free(W); free(Y); free(B);
    free(gi); free(q); free(sa); free(bias);
}

int main(void)
{
    const double edges[] = {0.0, -0.0, 1.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 5.96e-8, 2.98e-8,
                            6.1e-5, NAN, INFINITY, -INFINITY, 1.0 + 1.0 / 2048, 3.0 / 2048};
    for (size_t i = 0; i < sizeof(edges) / sizeof(edges[0]); ++i) {
        const uint16_t h = oracle_round_f16(edges[i]);
        (void)oracle_f16_to_f64(h);
        (void)oracle_bias_f16((float)edges[i], h, 0);
        (void)oracle_bias_f16((float)edges[i], h, 1);
    }
    uint16_t all[65536];
    double dec[65536];
    for (int i = 0; i < 65536; ++i) all[i] = (uint16_t)i;
    oracle_decode_f16(all, 65536, dec);
    float f[4] = {1.0f, -2.5f, NAN, 1e-45f};
    double fd[4];
    oracle_decode_f32(f, 4, fd);
    run_shape(5, 7, 64, 16);     /* four blocks */
    run_shape(4, 9, 80, 32);     /* K not a multiple of the group: three blocks, odd */
    run_shape(6, 33, 384, 128);  /* three blocks, odd: a padded zero-point nibble */
    run_shape(1, 1, 16, 16);
    printf("ok\n");
    return 0;
}
