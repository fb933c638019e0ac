/*
 * Host sanitizer driver for the CPU oracle (test infrastructure; built with
 * -fsanitize=address,undefined by tests/test_host_sanitizers.py and run on the CPU).
 *
 * Calls every function of oracle/convrot_oracle.c on small inputs held in buffers of exactly
 * the size each function may touch (so any read or write past them is reported), on its
 * argument-error paths, and at its edge cases: zero rows, an all-zero row, int32 overflow of a
 * dot product, every fp16 bit pattern.  A few results are checked as well, so a driver that
 * stopped calling the code would fail too.  Exit status 0 = every check held.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_num_threads(void);
int oracle_hadamard_entry(int i, int j);
int oracle_rotate(const double *x, int64_t rows, int64_t K, int g, double *y);
int oracle_quantize_rows_i8(const double *y, int64_t rows, int64_t K, float *scale, int8_t *q);
uint16_t oracle_f16_from_double(double d);
double oracle_f16_to_double(uint16_t h);
int oracle_quantize_groups_i4(const double *y, int64_t rows, int64_t K, int g, uint16_t *scale, int8_t *codes);
int oracle_pack_i4(const int8_t *codes, int64_t rows, int64_t K, uint8_t *packed);
int oracle_unpack_i4(const uint8_t *packed, int64_t rows, int64_t K, int8_t *codes);
int oracle_gemm_i32(const int8_t *a, const int8_t *b, int64_t M, int64_t N, int64_t K, int32_t *acc);
int oracle_gemm_i32_pairs(const int8_t *a, const int8_t *b, int64_t K, const int64_t *ms, const int64_t *ns,
                          int64_t count, int32_t *out);
int oracle_dequant(const int32_t *acc, const float *sx, const float *sw, const float *bias, int64_t M, int64_t N,
                   double *y);
int oracle_linear_i4(const int8_t *cx, const uint16_t *sx, const int8_t *cw, const uint16_t *sw, const float *bias,
                     int64_t M, int64_t N, int64_t K, int g, double *y);
int oracle_linear_w4a8(const int8_t *qx, const float *sx, const int8_t *cw, const uint16_t *sw, const float *bias,
                       int64_t M, int64_t N, int64_t K, int g, double *y);

enum { OK = 0, ERR_ARG = 1, ERR_RANGE = 2 };

static int failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double unif(void)   /* xorshift64*, in [-1, 1) */
{
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return (double)((rng * 2685821657736338717ull) >> 11) / 4503599627370496.0 - 1.0;
}

static void *exact(size_t n) { return malloc(n ? n : 1); }

int main(void)
{
    CHECK(oracle_num_threads() >= 1);

    /* Sylvester Hadamard rows are orthogonal: sum_j H[i,j] H[k,j] = 16 [i == k] */
    for (int i = 0; i < 16; ++i)
        for (int k = 0; k < 16; ++k) {
            int s = 0;
            for (int j = 0; j < 16; ++j) s += oracle_hadamard_entry(i, j) * oracle_hadamard_entry(k, j);
            CHECK(s == (i == k ? 16 : 0));
        }

    const int64_t R = 3, K = 512;
    double *x = exact(sizeof(double) * R * K), *y = exact(sizeof(double) * R * K);
    for (int64_t i = 0; i < R * K; ++i) x[i] = 4.0 * unif();
    for (int64_t k = 0; k < K; ++k) x[2 * K + k] = 0.0;             /* an all-zero row */
    const int groups[] = {1, 2, 128, 256, 512};
    for (unsigned gi = 0; gi < sizeof groups / sizeof groups[0]; ++gi) {
        CHECK(oracle_rotate(x, R, K, groups[gi], y) == OK);
        /* the rotation is orthonormal: row norms are kept */
        for (int64_t r = 0; r < R; ++r) {
            double a = 0.0, b = 0.0;
            for (int64_t k = 0; k < K; ++k) { a += x[r * K + k] * x[r * K + k]; b += y[r * K + k] * y[r * K + k]; }
            CHECK(fabs(a - b) <= 1e-9 * (a + 1.0));
        }
    }
    CHECK(oracle_rotate(x, 0, K, 256, y) == OK);
    CHECK(oracle_rotate(x, R, K, 3, y) == ERR_ARG);
    CHECK(oracle_rotate(x, R, 500, 256, y) == ERR_ARG);
    CHECK(oracle_rotate(NULL, R, K, 256, y) == ERR_ARG);
    CHECK(oracle_rotate(x, -1, K, 256, y) == ERR_ARG);

    /* INT8 rows: codes within [-127, 127], the row maximum maps to +-127, the zero row to 0 */
    CHECK(oracle_rotate(x, R, K, 256, y) == OK);
    float *s8 = exact(sizeof(float) * R);
    int8_t *q8 = exact((size_t)(R * K));
    CHECK(oracle_quantize_rows_i8(y, R, K, s8, q8) == OK);
    for (int64_t r = 0; r < R; ++r) {
        int top = 0;
        for (int64_t k = 0; k < K; ++k) {
            CHECK(q8[r * K + k] >= -127 && q8[r * K + k] <= 127);
            if (abs(q8[r * K + k]) == 127) top = 1;
        }
        CHECK(r == 2 ? (s8[r] == 0.0f && !top) : (s8[r] > 0.0f && top));
    }
    CHECK(oracle_quantize_rows_i8(y, R, 0, s8, q8) == ERR_ARG);
    CHECK(oracle_quantize_rows_i8(NULL, R, K, s8, q8) == ERR_ARG);

    /* fp16: every finite pattern survives the round trip; halfway cases round to even */
    for (uint32_t h = 0; h < 65536; ++h) {
        if (((h >> 10) & 31) == 31) continue;
        const double d = oracle_f16_to_double((uint16_t)h);
        CHECK(oracle_f16_from_double(d) == (uint16_t)h || (h == 0x8000u && d == 0.0));
    }
    CHECK(oracle_f16_from_double(1.0 + ldexp(1.0, -11)) == 0x3c00u);
    CHECK(oracle_f16_from_double(1.0 + 3.0 * ldexp(1.0, -11)) == 0x3c02u);
    CHECK(oracle_f16_from_double(70000.0) == 0x7c00u);
    CHECK(isnan(oracle_f16_to_double(oracle_f16_from_double(NAN))));

    /* INT4 groups, packing both ways */
    for (int g = 128; g <= 256; g *= 2) {
        const int64_t G = K / g;
        uint16_t *s4 = exact(sizeof(uint16_t) * R * G);
        int8_t *c4 = exact((size_t)(R * K)), *c4b = exact((size_t)(R * K));
        uint8_t *p4 = exact((size_t)(R * K / 2));
        CHECK(oracle_quantize_groups_i4(y, R, K, g, s4, c4) == OK);
        for (int64_t i = 0; i < R * K; ++i) CHECK(c4[i] >= -7 && c4[i] <= 7);
        CHECK(oracle_pack_i4(c4, R, K, p4) == OK);
        CHECK(oracle_unpack_i4(p4, R, K, c4b) == OK);
        CHECK(memcmp(c4, c4b, (size_t)(R * K)) == 0);
        CHECK(oracle_quantize_groups_i4(y, R, K, 96, s4, c4) == ERR_ARG);
        CHECK(oracle_pack_i4(c4, R, 511, p4) == ERR_ARG);
        CHECK(oracle_unpack_i4(p4, R, 511, c4b) == ERR_ARG);

        /* W4A4 and W4A8 outputs from these codes, with and without bias */
        const int64_t M = 2, N = 3;
        double *yo = exact(sizeof(double) * M * N);
        float *bias = exact(sizeof(float) * N), *sx = exact(sizeof(float) * M);
        for (int64_t n = 0; n < N; ++n) bias[n] = (float)unif();
        for (int64_t m = 0; m < M; ++m) sx[m] = 0.01f;
        /* rows 0..1 as tokens, rows 0..2 as weights: [M, G] / [N, G] scale blocks */
        CHECK(oracle_linear_i4(c4, s4, c4, s4, bias, M, N, K, g, yo) == OK);
        CHECK(oracle_linear_i4(c4, s4, c4, s4, NULL, M, N, K, g, yo) == OK);
        CHECK(oracle_linear_w4a8(q8, sx, c4, s4, bias, M, N, K, g, yo) == OK);
        CHECK(oracle_linear_w4a8(q8, sx, c4, s4, NULL, M, N, K, g, yo) == OK);
        CHECK(oracle_linear_i4(c4, s4, c4, s4, bias, M, N, K, 3, yo) == ERR_ARG);
        CHECK(oracle_linear_w4a8(q8, sx, c4, s4, bias, M, N, 500, g, yo) == ERR_ARG);
        free(yo); free(bias); free(sx); free(s4); free(c4); free(c4b); free(p4);
    }

    /* integer GEMM, the listed pairs, dequantization; int32 overflow is refused */
    {
        const int64_t M = 3, N = 5, KK = 96;
        int8_t *a = exact((size_t)(M * KK)), *b = exact((size_t)(N * KK));
        for (int64_t i = 0; i < M * KK; ++i) a[i] = (int8_t)(127.0 * unif());
        for (int64_t i = 0; i < N * KK; ++i) b[i] = (int8_t)(127.0 * unif());
        int32_t *acc = exact(sizeof(int32_t) * M * N);
        CHECK(oracle_gemm_i32(a, b, M, N, KK, acc) == OK);
        int64_t ms[4] = {0, 2, 1, 2}, ns[4] = {4, 0, 3, 2};
        int32_t *out = exact(sizeof(int32_t) * 4);
        CHECK(oracle_gemm_i32_pairs(a, b, KK, ms, ns, 4, out) == OK);
        for (int i = 0; i < 4; ++i) CHECK(out[i] == acc[ms[i] * N + ns[i]]);
        float sxv[3] = {0.5f, 0.25f, 2.0f}, swv[5] = {1.0f, 2.0f, 3.0f, 4.0f, 5.0f}, bv[5] = {1, 1, 1, 1, 1};
        double *yd = exact(sizeof(double) * M * N);
        CHECK(oracle_dequant(acc, sxv, swv, bv, M, N, yd) == OK);
        CHECK(yd[1 * N + 2] == (double)acc[1 * N + 2] * 0.25 * 3.0 + 1.0);
        CHECK(oracle_dequant(acc, sxv, swv, NULL, M, N, yd) == OK);
        CHECK(oracle_gemm_i32(a, b, -1, N, KK, acc) == ERR_ARG);
        free(a); free(b); free(acc); free(out); free(yd);

        /* 127 * 127 * 133200 > 2^31 - 1 */
        const int64_t KB = 133200;
        int8_t *big = exact((size_t)KB);
        memset(big, 127, (size_t)KB);
        int32_t one;
        int64_t z = 0;
        CHECK(oracle_gemm_i32(big, big, 1, 1, KB, &one) == ERR_RANGE);
        CHECK(oracle_gemm_i32_pairs(big, big, KB, &z, &z, 1, &one) == ERR_RANGE);
        free(big);
    }
    free(x); free(y); free(s8); free(q8);
    if (failures) fprintf(stderr, "%d checks failed\n", failures);
    else printf("oracle sanitizer driver: all checks held\n");
    return failures ? 1 : 0;
}
