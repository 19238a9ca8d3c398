/*
 * CPU oracle for the group-quantised int4-weight x bf16-activation matmul.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code, header, table or
 * helper with the HIP library: every conversion below is written out from its definition.
 *
 * What it computes (the plain definition, no blocking or reordering):
 *   q[k][n]  = code of row k, column n            (4-bit field of the packed weight word)
 *   z[gi][n] = zero point of group gi, column n   (4-bit field, or 8 when no zeros are given)
 *   s[gi][n] = fp16 scale, widened to float exactly
 *   w[k][n]  = (float)(q - z) * s                 exact in fp32 (a 5-bit integer times an
 *                                                 11-bit significand fits in 24 bits)
 *   y[m][n]  = sum over k ascending of (double)A[m][k] * (double)w[k][n]
 *   bound[m][n] = sum over k of |(double)A[m][k] * (double)w[k][n]|
 * with gi = k / g.
 * The affine form w = s * q + b of MLX checkpoints (codes of 1 to 8 bits, bf16 scales and
 * biases) has its own unpacking and matmul at the end of the file.
 *
 * Sources. The dequantisation is the exact (q - z) * scale form that the GRIMOIRE v1.7
 * release notes ('What changed') keep for their int4 single-user GEMV, with int4 weights and
 * bf16 activations for both the one-row GEMV and the 2-16-row matrix-engine GEMM. The group
 * sizes are those of the GPTQ-Int4 group-128 and W4A16 group-64 checkpoints in the same
 * section. The packing is the GPTQ storage convention: nibble j of qweight word [i][n] holds
 * row 8i+j, nibble j of qzeros word [gi][c] holds column 8c+j; no stored offset on the zero.
 * The fp64 accumulation and the |a*w| bound follow the practice in TensorFold PR #859
 * (commit messages) of measuring a GPU product against a float64 bound.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC w4a16_oracle.c -o libw4a16_oracle.so
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- scalar conversions, from the IEEE-754 binary16 and bfloat16 definitions ---------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
float w4o_fp16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)               /* zero or subnormal: f * 2^-24 */
        v = ldexp((double)f, -24);
    else if (e == 31)         /* infinity or NaN */
        v = f ? NAN : INFINITY;
    else                      /* normal: (1024 + f) * 2^(e - 25) */
        v = ldexp((double)(1024 + f), e - 25);
    return (float)(sign ? -v : v);   /* every binary16 value is exact in binary32 */
}

/* bfloat16 is the upper half of a binary32: same sign and exponent, 7 fraction bits. */
float w4o_bf16_to_f32(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float v;
    memcpy(&v, &bits, sizeof v);
    return v;
}

/* ---- unpacking ------------------------------------------------------------------------- */

static inline int code_of(const uint32_t *qweight, int64_t N, int64_t k, int64_t n)
{
    uint32_t word = qweight[(k / 8) * N + n];
    return (int)((word >> (4 * (k % 8))) & 0xFu);
}

static inline int zero_of(const uint32_t *qzeros, int64_t N, int64_t gi, int64_t n)
{
    if (!qzeros)
        return 8;
    uint32_t word = qzeros[gi * (N / 8) + n / 8];
    return (int)((word >> (4 * (n % 8))) & 0xFu);
}

/* q[k*N + n] = code of row k, column n. */
int w4o_unpack_qweight(const uint32_t *qweight, int64_t K, int64_t N, uint8_t *q)
{
    if (!qweight || !q || K <= 0 || N <= 0 || K % 8)
        return -1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            q[k * N + n] = (uint8_t)code_of(qweight, N, k, n);
    return 0;
}

/* z[gi*N + n] = zero of group gi, column n (8 everywhere when qzeros is NULL). */
int w4o_unpack_qzeros(const uint32_t *qzeros, int64_t G, int64_t N, uint8_t *z)
{
    if (!z || G <= 0 || N <= 0 || N % 8)
        return -1;
    for (int64_t gi = 0; gi < G; ++gi)
        for (int64_t n = 0; n < N; ++n)
            z[gi * N + n] = (uint8_t)zero_of(qzeros, N, gi, n);
    return 0;
}

/* ---- dequantisation -------------------------------------------------------------------- */

static inline float weight_of(const uint32_t *qweight, const uint16_t *scales,
                              const uint32_t *qzeros, int64_t g, int64_t N, int64_t k, int64_t n)
{
    int64_t gi = k / g;
    int d = code_of(qweight, N, k, n) - zero_of(qzeros, N, gi, n);
    float s = w4o_fp16_to_f32(scales[gi * N + n]);
    return (float)d * s;
}

/* w[k*N + n] = (q - z) * s in fp32. */
int w4o_dequant(const uint32_t *qweight, const uint16_t *scales, const uint32_t *qzeros,
                int64_t g, int64_t K, int64_t N, float *w)
{
    if (!qweight || !scales || !w || g <= 0 || K <= 0 || N <= 0 || K % 8 || K % g || N % 8)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            w[k * N + n] = weight_of(qweight, scales, qzeros, g, N, k, n);
    return 0;
}

/* ---- the matmul ------------------------------------------------------------------------ */

/*
 * y[m*C + c] and bound[m*C + c] for the C output columns cols[0..C-1] (all N columns, in
 * order, when cols is NULL; then C = N). A is bf16 [M, K] row-major.
 */
int w4o_gemm(const uint16_t *A, const uint32_t *qweight, const uint16_t *scales,
             const uint32_t *qzeros, int64_t g, int64_t M, int64_t N, int64_t K,
             const int64_t *cols, int64_t C, double *y, double *bound)
{
    if (!A || !qweight || !scales || !y || g <= 0 || M <= 0 || N <= 0 || K <= 0 ||
        K % 8 || K % g || N % 8)
        return -1;
    if (!cols)
        C = N;
    if (C <= 0)
        return -1;
    for (int64_t c = 0; cols && c < C; ++c)
        if (cols[c] < 0 || cols[c] >= N)
            return -1;

    double *a = (double *)malloc(sizeof(double) * (size_t)(M * K));
    if (!a)
        return -2;
    for (int64_t i = 0; i < M * K; ++i)
        a[i] = (double)w4o_bf16_to_f32(A[i]);

#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        int64_t n = cols ? cols[c] : c;
        for (int64_t m = 0; m < M; ++m) {
            y[m * C + c] = 0.0;
            if (bound)
                bound[m * C + c] = 0.0;
        }
        for (int64_t k = 0; k < K; ++k) {
            double w = (double)weight_of(qweight, scales, qzeros, g, N, k, n);
            for (int64_t m = 0; m < M; ++m) {
                double p = a[m * K + k] * w;
                y[m * C + c] += p;
                if (bound)
                    bound[m * C + c] += fabs(p);
            }
        }
    }
    free(a);
    return 0;
}

/* ---- greedy selection ------------------------------------------------------------------ */

/*
 * idx[m] = smallest n with v[m][n] equal to the row maximum, decided in fp32: the precision
 * the logits leave the GPU in (lucebox PR #823 moves this greedy choice onto the device).
 * NaN entries are never selected unless the whole row is NaN (then idx = 0).
 */
int w4o_argmax_rows_f32(const float *v, int64_t M, int64_t N, int64_t *idx)
{
    if (!v || !idx || M <= 0 || N <= 0)
        return -1;
    for (int64_t m = 0; m < M; ++m) {
        int64_t best = -1;
        for (int64_t n = 0; n < N; ++n) {
            float x = v[m * N + n];
            if (isnan(x))
                continue;
            if (best < 0 || x > v[m * N + best])
                best = n;
        }
        idx[m] = best < 0 ? 0 : best;
    }
    return 0;
}

/*
 * The k best candidates of each row, best first: repeat the greedy selection above k times,
 * each time over the entries not yet chosen. idx[m * k + r] = the r-th choice of row m (largest
 * fp32 value first, equal values by smallest column, -0 equal to +0, NaN never chosen), or -1
 * once the row has no entry left to choose. The pages move only the greedy choice onto the
 * device (lucebox PR #823); the k best are that choice extended to the next candidates in the
 * same order, so the first of them is the greedy one.
 */
int w4o_topk_rows_f32(const float *v, int64_t M, int64_t N, int64_t k, int64_t *idx)
{
    if (!v || !idx || M <= 0 || N <= 0 || k <= 0)
        return -1;
    unsigned char *taken = (unsigned char *)malloc((size_t)N);
    if (!taken)
        return -2;
    for (int64_t m = 0; m < M; ++m) {
        memset(taken, 0, (size_t)N);
        for (int64_t r = 0; r < k; ++r) {
            int64_t best = -1;
            for (int64_t n = 0; n < N; ++n) {
                float x = v[m * N + n];
                if (taken[n] || isnan(x))
                    continue;
                if (best < 0 || x > v[m * N + best])
                    best = n;
            }
            idx[m * k + r] = best;
            if (best >= 0)
                taken[best] = 1;
        }
    }
    free(taken);
    return 0;
}

/* ---- gated feed-forward input: SiLU(gate) * up ------------------------------------------ */

/*
 * The GRIMOIRE v1.8 release notes ('What changed', INT4 prompt processing) fuse the
 * feed-forward gate into the int4 matmul path. The pages do not name the gate's nonlinearity;
 * the Qwen-family feed-forward they run is the SiLU-gated one, so the gated product is
 *   h[i] = silu(g[i]) * u[i],   silu(x) = x / (1 + e^-x),
 * here with g = A x W_gate and u = A x W_up, both the fp64 products of w4o_gemm.
 */
double w4o_silu(double x) { return x / (1.0 + exp(-x)); }

int w4o_silu_mul(const double *g, const double *u, int64_t n, double *h)
{
    if (!g || !u || !h || n < 0)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        h[i] = w4o_silu(g[i]) * u[i];
    return 0;
}

/* ---- affine codes: w = s * q + b (MLX affine quantisation) ------------------------------ */

/*
 * The format of the MLX checkpoints in TensorFold PR #859 (commit messages: the affine-4
 * checkpoint, mixed-width checkpoints of 2 to 8 bits in groups of 64): every code q of `bits`
 * bits keeps its own value, and the weight is w = s * q + b with a scale s and a bias b per
 * group of rows and column, both bf16.
 *
 * Storage read here: for column n, the codes of rows k = 0, 1, 2, ... form one little-endian
 * bit stream, row k at stream bits [k*bits, (k+1)*bits); stream bit i is bit i % 32 of word
 * [i / 32][n] of an array [K*bits/32, N]. At bits = 4 this is the GPTQ nibble layout above.
 */
static inline int affine_code_of(const uint32_t *packed, int bits, int64_t N, int64_t k, int64_t n)
{
    int code = 0;
    for (int b = 0; b < bits; ++b) {           /* one stream bit at a time */
        int64_t i = k * bits + b;
        uint32_t word = packed[(i / 32) * N + n];
        code |= (int)((word >> (i % 32)) & 1u) << b;
    }
    return code;
}

static int affine_shape_ok(int bits, int64_t K, int64_t N)
{
    return bits >= 1 && bits <= 8 && K > 0 && N > 0 && (K * bits) % 32 == 0;
}

/* q[k*N + n] = code of row k, column n. */
int w4o_affine_unpack(const uint32_t *packed, int bits, int64_t K, int64_t N, uint8_t *q)
{
    if (!packed || !q || !affine_shape_ok(bits, K, N))
        return -1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            q[k * N + n] = (uint8_t)affine_code_of(packed, bits, N, k, n);
    return 0;
}

/*
 * y[m*C + c] = sum over k ascending of a[m][k] * w[k][n], w = s * q + b in fp64 (exact: an
 * 8-bit significand times an 8-bit code, plus an 8-bit significand), and
 * bound[m*C + c] = sum over k of |a[m][k]| * (|s * q| + |b|): the sizes of the two terms a
 * kernel that applies scale and bias to separate sums rounds. Columns as in w4o_gemm.
 */
int w4o_affine_gemm(const uint16_t *A, const uint32_t *packed, int bits, const uint16_t *scales,
                    const uint16_t *biases, int64_t g, int64_t M, int64_t N, int64_t K,
                    const int64_t *cols, int64_t C, double *y, double *bound)
{
    if (!A || !packed || !scales || !biases || !y || g <= 0 || M <= 0 || K % g ||
        !affine_shape_ok(bits, K, N))
        return -1;
    if (!cols)
        C = N;
    if (C <= 0)
        return -1;
    for (int64_t c = 0; cols && c < C; ++c)
        if (cols[c] < 0 || cols[c] >= N)
            return -1;

    double *a = (double *)malloc(sizeof(double) * (size_t)(M * K));
    if (!a)
        return -2;
    for (int64_t i = 0; i < M * K; ++i)
        a[i] = (double)w4o_bf16_to_f32(A[i]);

#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        int64_t n = cols ? cols[c] : c;
        for (int64_t m = 0; m < M; ++m) {
            y[m * C + c] = 0.0;
            if (bound)
                bound[m * C + c] = 0.0;
        }
        for (int64_t k = 0; k < K; ++k) {
            int64_t gi = k / g;
            double s = (double)w4o_bf16_to_f32(scales[gi * N + n]);
            double b = (double)w4o_bf16_to_f32(biases[gi * N + n]);
            double sq = s * (double)affine_code_of(packed, bits, N, k, n);
            double w = sq + b;
            for (int64_t m = 0; m < M; ++m) {
                y[m * C + c] += a[m * K + k] * w;
                if (bound)
                    bound[m * C + c] += fabs(a[m * K + k]) * (fabs(sq) + fabs(b));
            }
        }
    }
    free(a);
    return 0;
}
