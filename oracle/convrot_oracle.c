/*
 * convrot_oracle.c -- plain, slow CPU oracle for the ConvRot quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path loads, links or calls this
 * library: only the test-suite, the package smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header, table or constant with the HIP library.
 *
 * What the method computes, and where the pages say so:
 *  - ConvRot is a grouped Hadamard rotation: before quantizing, the weight is rotated by a
 *    Hadamard transform over fixed-size groups, which spreads outlier energy so that INT8
 *    can represent it ("minimax-h3-nvfp4-convrot核心原理", section 四 "核心原理 3：INT8 ConvRot").
 *  - The group size is 256 channels of in_features (same section, engineering detail 3, and
 *    the converter flag --convrot-group-size 256 in "Qwen3-VL-32B-...-INT8-ConvRot部署优化",
 *    section "量化转换过程").
 *  - INT8 weights use one FP32 scale per output row (--scaling_mode row, same converter
 *    command; "INT8 row-scale + ConvRot metadata" in section 四 of the nvfp4-convrot page;
 *    "FP32缩放因子" in the 部署优化 page, section "INT8 ConvRot量化技术细节").
 *  - The W4A4 variant rotates BOTH activations and weights with the grouped Hadamard and then
 *    quantizes them to 4 bits with round-to-nearest (nvfp4-convrot page, section 五
 *    "INT4 W4A4 ConvRot", bullets on W4A4 and --simple RTN).
 *
 * Where the pages are silent this file takes the plainest reading:
 *  - Hadamard in Sylvester (natural) order, H[i][j] = (-1)^popcount(i & j), scaled by 1/sqrt(g)
 *    so the rotation is orthonormal; groups are contiguous blocks of g channels along K.
 *  - Activations are rotated with the same R and quantized per token, dynamically.
 *  - Symmetric RTN (ties to even) with qmax 127 (INT8) or 7 (INT4); a zero row/group gets
 *    scale 0 and codes 0.
 *  - A quantized code is a decision taken in floating point, so it is taken in fp32, the
 *    precision of the GPU kernel: the rotated value is rounded to fp32, the scale is the fp32
 *    (INT8) or fp16 (INT4) rounding of max|v|/qmax, and the code is rint of the correctly
 *    rounded fp32 quotient v / scale.  Everything else (rotation sums, dequantization) is fp64.
 *  - INT4 scales are per (row, group of g channels), stored as fp16; two codes per byte,
 *    the even channel in the low nibble.
 *
 * Every loop is the definition written out: the rotation is the explicit matrix product with
 * the Hadamard entries (no fast transform), the GEMM is a scalar int64 dot product.
 * OpenMP only splits independent rows across threads; it changes no arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum {
    ORACLE_OK = 0,
    ORACLE_ERR_ARG = 1,      /* bad size, group, NULL pointer */
    ORACLE_ERR_RANGE = 2     /* an int32 accumulator would overflow */
};

static int is_pow2_upto(int g, int gmax) { return g >= 1 && g <= gmax && (g & (g - 1)) == 0; }

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Entry (i, j) of the unnormalised Sylvester Hadamard matrix: (-1)^popcount(i & j). */
int oracle_hadamard_entry(int i, int j)
{
    return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1;
}

/*
 * y = x . R  with  R = blockdiag(H_g / sqrt(g), ..., H_g / sqrt(g))  (K/g blocks along K).
 * x, y: fp64 [rows, K] row-major.  Row-vector convention; H is symmetric so x.R = (R.x^T)^T.
 */
int oracle_rotate(const double *x, int64_t rows, int64_t K, int g, double *y)
{
    if (!x || !y || rows < 0 || K <= 0 || !is_pow2_upto(g, 1 << 15) || K % g) return ORACLE_ERR_ARG;
    const double root = sqrt((double)g);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * K;
        double *yr = y + r * K;
        for (int64_t b = 0; b < K; b += g) {
            for (int i = 0; i < g; ++i) {
                double s = 0.0;
                for (int j = 0; j < g; ++j) s += (double)oracle_hadamard_entry(j, i) * xr[b + j];
                yr[b + i] = s / root;
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Symmetric per-row INT8 quantization of already-rotated values (one scale per row over all K):
 *   a = max_k |fp32(y[r,k])|,  s[r] = fp32(a / 127),
 *   q[r,k] = clamp(rint(fp32(fp32(y[r,k]) / s[r])), -127, 127),   s == 0 -> q = 0.
 * Used for weight rows (one scale per output channel) and activation rows (one per token).
 * fp32 division is computed in double and rounded once to float; for operands that are
 * themselves fp32 this equals the correctly rounded fp32 quotient.
 */
int oracle_quantize_rows_i8(const double *y, int64_t rows, int64_t K, float *scale, int8_t *q)
{
    if (!y || !scale || !q || rows < 0 || K <= 0) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *yr = y + r * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf((float)yr[k]);
            if (v > amax) amax = v;
        }
        const float s = (float)((double)amax / 127.0);
        scale[r] = s;
        for (int64_t k = 0; k < K; ++k) {
            if (s == 0.0f) { q[r * K + k] = 0; continue; }
            const float t = (float)((double)(float)yr[k] / (double)s);
            double c = rint((double)t);
            if (c > 127.0) c = 127.0;
            if (c < -127.0) c = -127.0;
            q[r * K + k] = (int8_t)c;
        }
    }
    return ORACLE_OK;
}

/* IEEE binary16 round-to-nearest-even from a double (finite or not). */
uint16_t oracle_f16_from_double(double d)
{
    uint16_t sign = signbit(d) ? 0x8000u : 0u;
    double a = fabs(d);
    if (isnan(d)) return (uint16_t)(sign | 0x7e00u);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u);           /* rounds past 65504 -> inf */
    if (a < ldexp(1.0, -14)) {                                       /* subnormal: units of 2^-24 */
        double u = rint(ldexp(a, 24));                               /* exact scaling, one rounding */
        return (uint16_t)(sign | (uint16_t)u);                       /* u == 1024 is the min normal */
    }
    int e2;
    (void)frexp(a, &e2);            /* a = m * 2^e2, m in [0.5, 1) */
    int E = e2 - 1;                 /* a = (1.f) * 2^E */
    double frac = rint((ldexp(a, -E) - 1.0) * 1024.0);
    if (frac >= 1024.0) { frac = 0.0; E += 1; }
    if (E > 15) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)frac);
}

double oracle_f16_to_double(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)f, -24);
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp(1024.0 + f, e - 25);
    return s ? -v : v;
}

/*
 * Symmetric INT4 quantization per (row, group of g channels) of already-rotated values:
 *   a = max_{k in group} |fp32(y)|,  s = fp16(a / 7),
 *   c = clamp(rint(fp32(fp32(y) / s)), -7, 7),   s == 0 -> c = 0.
 * codes: int8 [rows, K] (one code per byte, unpacked); scale: fp16 bits [rows, K/g].
 */
int oracle_quantize_groups_i4(const double *y, int64_t rows, int64_t K, int g, uint16_t *scale, int8_t *codes)
{
    if (!y || !scale || !codes || rows < 0 || K <= 0 || !is_pow2_upto(g, 1 << 15) || K % g) return ORACLE_ERR_ARG;
    const int64_t G = K / g;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < G; ++j) {
            const double *yg = y + r * K + j * g;
            float amax = 0.0f;
            for (int i = 0; i < g; ++i) {
                float v = fabsf((float)yg[i]);
                if (v > amax) amax = v;
            }
            const uint16_t sh = oracle_f16_from_double((double)amax / 7.0);
            scale[r * G + j] = sh;
            const float s = (float)oracle_f16_to_double(sh);
            for (int i = 0; i < g; ++i) {
                int8_t *c = codes + r * K + j * g + i;
                if (s == 0.0f) { *c = 0; continue; }
                const float t = (float)((double)(float)yg[i] / (double)s);
                double v = rint((double)t);
                if (v > 7.0) v = 7.0;
                if (v < -7.0) v = -7.0;
                *c = (int8_t)v;
            }
        }
    }
    return ORACLE_OK;
}

/* Two INT4 codes per byte: byte i of a row = (c[2i] & 0xF) | ((c[2i+1] & 0xF) << 4). */
int oracle_pack_i4(const int8_t *codes, int64_t rows, int64_t K, uint8_t *packed)
{
    if (!codes || !packed || rows < 0 || K <= 0 || K % 2) return ORACLE_ERR_ARG;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t i = 0; i < K / 2; ++i) {
            unsigned lo = (unsigned)(uint8_t)codes[r * K + 2 * i] & 0xFu;
            unsigned hi = (unsigned)(uint8_t)codes[r * K + 2 * i + 1] & 0xFu;
            packed[r * (K / 2) + i] = (uint8_t)(lo | (hi << 4));
        }
    return ORACLE_OK;
}

/* Inverse of oracle_pack_i4: each nibble is a two's-complement 4-bit integer. */
int oracle_unpack_i4(const uint8_t *packed, int64_t rows, int64_t K, int8_t *codes)
{
    if (!codes || !packed || rows < 0 || K <= 0 || K % 2) return ORACLE_ERR_ARG;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t i = 0; i < K / 2; ++i) {
            int lo = packed[r * (K / 2) + i] & 0xF;
            int hi = (packed[r * (K / 2) + i] >> 4) & 0xF;
            codes[r * K + 2 * i] = (int8_t)(lo >= 8 ? lo - 16 : lo);
            codes[r * K + 2 * i + 1] = (int8_t)(hi >= 8 ? hi - 16 : hi);
        }
    return ORACLE_OK;
}

/*
 * acc[m,n] = sum_k a[m,k] * b[n,k]   (a: [M,K], b: [N,K], both K-contiguous; acc int32 [M,N]).
 * Accumulates in int64 and refuses (ORACLE_ERR_RANGE) a result outside int32.
 */
int oracle_gemm_i32(const int8_t *a, const int8_t *b, int64_t M, int64_t N, int64_t K, int32_t *acc)
{
    if (!a || !b || !acc || M < 0 || N < 0 || K < 0) return ORACLE_ERR_ARG;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int64_t)a[m * K + k] * (int64_t)b[n * K + k];
            if (s > INT32_MAX || s < INT32_MIN) { bad = 1; s = 0; }
            acc[m * N + n] = (int32_t)s;
        }
    }
    return bad ? ORACLE_ERR_RANGE : ORACLE_OK;
}

/* Same dot products, but only for the listed (m, n) pairs: out[i] = sum_k a[ms[i],k] * b[ns[i],k]. */
int oracle_gemm_i32_pairs(const int8_t *a, const int8_t *b, int64_t K, const int64_t *ms, const int64_t *ns,
                          int64_t count, int32_t *out)
{
    if (!a || !b || !ms || !ns || !out || K < 0 || count < 0) return ORACLE_ERR_ARG;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t i = 0; i < count; ++i) {
        int64_t s = 0;
        for (int64_t k = 0; k < K; ++k) s += (int64_t)a[ms[i] * K + k] * (int64_t)b[ns[i] * K + k];
        if (s > INT32_MAX || s < INT32_MIN) { bad = 1; s = 0; }
        out[i] = (int32_t)s;
    }
    return bad ? ORACLE_ERR_RANGE : ORACLE_OK;
}

/* Dequantization: y[m,n] = acc[m,n] * sx[m] * sw[n] + bias[n]   (fp64; bias may be NULL). */
int oracle_dequant(const int32_t *acc, const float *sx, const float *sw, const float *bias, int64_t M, int64_t N,
                   double *y)
{
    if (!acc || !sx || !sw || !y || M < 0 || N < 0) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = (double)acc[m * N + n] * (double)sx[m] * (double)sw[n] + (bias ? (double)bias[n] : 0.0);
    return ORACLE_OK;
}

/*
 * W4A4 output:  y[m,n] = sum_j ( sum_{k in group j} cx[m,k] cw[n,k] ) * sx[m,j] * sw[n,j] + bias[n]
 * cx: int8 codes [M,K], cw: int8 codes [N,K], sx: fp16 bits [M,K/g], sw: fp16 bits [N,K/g].
 * Group sums are exact integers; the sum over groups runs in increasing j, in fp64.
 */
int oracle_linear_i4(const int8_t *cx, const uint16_t *sx, const int8_t *cw, const uint16_t *sw, const float *bias,
                     int64_t M, int64_t N, int64_t K, int g, double *y)
{
    if (!cx || !sx || !cw || !sw || !y || M < 0 || N < 0 || K <= 0 || !is_pow2_upto(g, 1 << 15) || K % g)
        return ORACLE_ERR_ARG;
    const int64_t G = K / g;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t j = 0; j < G; ++j) {
                int64_t s = 0;
                for (int i = 0; i < g; ++i) s += (int64_t)cx[m * K + j * g + i] * (int64_t)cw[n * K + j * g + i];
                acc += (double)s * oracle_f16_to_double(sx[m * G + j]) * oracle_f16_to_double(sw[n * G + j]);
            }
            y[m * N + n] = acc + (bias ? (double)bias[n] : 0.0);
        }
    return ORACLE_OK;
}


/*
 * W4A8 linear: INT4 weights with one fp16 scale per (row, group) against INT8 activations with
 * one fp32 scale per token, both rotated by the same grouped Hadamard (the W4A8 variant of the
 * ConvRot checkpoints, "MiniMax-H3-W4A8-ConvRot" pages: 4-bit weights, 8-bit activations).
 *   y[m,n] = sx[m] * sum_j sw[n,j] * (sum_{k in group j} qx[m,k] * cw[n,k]) + bias[n]
 * Each group's dot product is an exact integer; groups are scaled and summed in fp64 in
 * increasing j.  sw is [N, K/g] (row-major, this file's layout).
 */
int oracle_linear_w4a8(const int8_t *qx, const float *sx, const int8_t *cw, const uint16_t *sw, const float *bias,
                       int64_t M, int64_t N, int64_t K, int g, double *y)
{
    if (!qx || !sx || !cw || !sw || !y || M < 0 || N < 0 || K <= 0 || !is_pow2_upto(g, 1 << 15) || K % g)
        return ORACLE_ERR_ARG;
    const int64_t G = K / g;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t j = 0; j < G; ++j) {
                int64_t s = 0;
                for (int i = 0; i < g; ++i) s += (int64_t)qx[m * K + j * g + i] * (int64_t)cw[n * K + j * g + i];
                acc += (double)s * oracle_f16_to_double(sw[n * G + j]);
            }
            y[m * N + n] = acc * (double)sx[m] + (bias ? (double)bias[n] : 0.0);
        }
    return ORACLE_OK;
}
