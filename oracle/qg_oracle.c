/*
 * qg_oracle.c -- plain, slow, obviously correct CPU oracle for the
 * dequantize-fused low-bit weight matrix-vector product, its matrix-matrix
 * (prefill) form, and greedy selection (argmax) over the output-head matvec.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library. The GPU product
 * path never calls it, and the two share no code, header, table or helper.
 *
 * What is computed is the plain definition, written out:
 *
 *   w[m][k]  = exact real value of weight (m,k) decoded from its format
 *   y[n][m]  = sum over k of w[m][k] * x[n][k]          (double accumulation)
 *   a[n][m]  = sum over k of |w[m][k] * x[n][k]|        (scale of the bound)
 *   idx[n]   = lowest m such that y[n][m] equals max over m' of y[n][m']
 *
 * The matrix-vector product and the prefill product are the same formula:
 * a matrix-vector product over N activation rows is N independent matvecs
 * (I Built an LLM Inference Engine on a 15 year old GPU..., "Two Numbers
 * That Tell the Whole Story": prefill runs the same weights against many
 * token rows; "The Baseline": the product is a plain triple loop).
 *
 * Weight formats (W is M x K: M outputs, K inputs; every array row-major):
 *
 *  1  INT8 per-row symmetric.  codes int8 [M][K], scales fp32 [M].
 *     w = scale[m] * q, q read as two's complement, no clamping.
 *     (MiniCPM-V-4.6 on a Tesla C2075, academ.us 2607.14568, section 2.3
 *     "Quantization and residency": symmetric 8-bit weights with an FP32
 *     scale; the per-row grouping is the reading this library takes.)
 *
 *  2  4-bit affine, group of 64 along k.  codes uint8 [M][K/2],
 *     scales bf16 [M][K/64], biases bf16 [M][K/64].
 *     Byte j of row m holds k = 2j in bits 0..3 and k = 2j+1 in bits 4..7.
 *     w = scale[m][k/64] * q + bias[m][k/64],  q in 0..15.
 *     (Pushing the limits of legacy hardware, "Start with the machine that
 *     actually exists": group-64 affine 4-bit codes with bf16 scale and bias;
 *     I Built an LLM Inference Engine..., "Quantization: The Model Doesn't
 *     Run on INT4": a code is turned back into a number as code times scale
 *     plus the block minimum, code 0 giving the minimum and code 15 the
 *     maximum.)
 *
 *  3  1-bit sign, group of 128 along k.  codes uint8 [M][K/8],
 *     scales fp16 [M][K/128].  Bit (k mod 8) of byte k/8 (least significant
 *     bit first) holds weight k; bit 1 means +scale, bit 0 means -scale.
 *     (A 27B model on two 4GB Maxwell GPUs, "Why this machine is awkward":
 *     binary weights with FP16 scales.)
 *
 *  4  INT8 symmetric, group of 64 along k.  codes int8 [M][K],
 *     scales fp32 [M][K/64].  w = scale[m][k/64] * q, q two's complement,
 *     no clamping.  (MiniCPM-V-4.6 on a Tesla C2075, section 2.3
 *     "Quantization and residency": symmetric 8-bit weights, each run of 64
 *     sharing an FP32 factor.)
 *
 * bf16 is the upper half of an IEEE binary32; fp16 is IEEE binary16
 * (subnormals included). Both are decoded here bit by bit, on purpose
 * without any half-precision type of the compiler.
 *
 * Every decoded weight is exact in double. Each product w*x is exact or
 * within one double rounding; the sum over K carries a relative error of
 * at most about K * 2^-53 of a[n][m], far below any tolerance applied.
 *
 * Embedding rows (4-bit format only): e[t][k] = the decoded weight of row
 * ids[t], input k, as a float32 the way the pages' decoder produces it: the
 * affine operations done separately in float32 (scale * code, exact, then
 * + bias, rounded to nearest even), the result rounded to an IEEE binary16
 * (nearest even, subnormals and signed zero kept) and widened back to
 * float32. (Pushing the limits of legacy hardware, "Half a billion values,
 * and one negative zero": that decoder multiplies and adds in two steps and
 * passes each value through FP16 on its way to FP32, and its GPU version had
 * to reproduce denormals, the sign of zero and round-to-nearest-even
 * exactly.) Rows of
 * ids outside [0, M) come out as quiet NaN. The float32 operations are
 * plain C float arithmetic (IEEE binary32 on this host; ISO C mode, so no
 * contraction); the binary16 rounding is written out bit by bit below.
 *
 * Threads: the (n, m) loop runs under OpenMP when built with -fopenmp;
 * nothing else is parallel, tiled or reordered.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_I8_ROW = 1, OR_U4_G64 = 2, OR_B1_G128 = 3, OR_I8_G64 = 4 };
enum { OR_OK = 0, OR_BAD_FORMAT = -1, OR_BAD_SHAPE = -2 };

/* ---- scalar decoders ------------------------------------------------- */

/* bf16 bit pattern -> its exact value: the 16 bits are the top half of an
 * IEEE binary32 whose low half is zero. */
double oracle_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* fp16 (IEEE binary16) bit pattern -> its exact value. 1 sign bit,
 * 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_fp16_value(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1f;
    int f = bits & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);              /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);  /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* float32 -> IEEE binary16 bit pattern, rounding to nearest, ties to even;
 * subnormal results and the sign of zero kept; overflow to infinity; NaN to
 * a quiet NaN. The float32 value is sig * 2^E with an integer significand;
 * the binary16 quantum at its magnitude is 2^max(L - 10, -24), L the
 * exponent of its leading bit. */
uint16_t oracle_f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    const int e = (int)((u >> 23) & 0xffu);
    const uint32_t man = u & 0x7fffffu;
    if (e == 0xff)
        return (uint16_t)(sign | (man ? 0x7e00u : 0x7c00u));
    if (e == 0 && man == 0)
        return sign;
    uint64_t sig = e ? (man | 0x800000u) : man;
    const int E = e ? e - 150 : -149;
    int L = E;
    for (uint64_t t = sig; t > 1; t >>= 1)
        ++L;                                   /* L = floor(log2(sig)) + E */
    int qe = L - 10 > -24 ? L - 10 : -24;      /* exponent of the quantum */
    const int shift = qe - E;                  /* low bits to drop, >= 0 here */
    uint64_t r;
    if (shift <= 0) {
        r = sig << (-shift);
    } else if (shift > 40) {
        r = 0;                                 /* below half the quantum */
    } else {
        r = sig >> shift;
        const uint64_t rem = sig & ((1ull << shift) - 1), half = 1ull << (shift - 1);
        if (rem > half || (rem == half && (r & 1)))
            ++r;
    }
    if (r >= 2048) {                           /* rounding carried into the next binade */
        r >>= 1;
        ++qe;
    }
    if (r < 1024)                              /* subnormal (qe == -24) or zero */
        return (uint16_t)(sign | r);
    const int e16 = qe + 25;                   /* value = r * 2^qe = (r/1024) * 2^(e16-15) */
    if (e16 >= 31)
        return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | ((uint32_t)e16 << 10) | (uint32_t)(r - 1024));
}

/* ---- the weight ------------------------------------------------------ */

struct qmat {
    int fmt;
    const void *codes;
    const void *scales;
    const void *biases;
    int64_t M, K;
};

static int shape_ok(int fmt, int64_t M, int64_t K)
{
    if (M < 1 || K < 1)
        return 0;
    if (fmt == OR_U4_G64 || fmt == OR_I8_G64)
        return K % 64 == 0;
    if (fmt == OR_B1_G128)
        return K % 128 == 0;
    return fmt == OR_I8_ROW;
}

/* Exact real value of weight (m, k). */
static double weight(const struct qmat *A, int64_t m, int64_t k)
{
    const int64_t K = A->K;
    if (A->fmt == OR_I8_ROW) {
        const int8_t *q = (const int8_t *)A->codes;
        const float *s = (const float *)A->scales;
        return (double)s[m] * (double)q[m * K + k];
    }
    if (A->fmt == OR_I8_G64) {
        const int8_t *code = (const int8_t *)A->codes;
        const float *gs = (const float *)A->scales;
        return (double)gs[m * (K / 64) + k / 64] * (double)code[m * K + k];
    }
    if (A->fmt == OR_U4_G64) {
        const uint8_t *c = (const uint8_t *)A->codes;
        const uint16_t *s = (const uint16_t *)A->scales;
        const uint16_t *b = (const uint16_t *)A->biases;
        uint8_t byte = c[m * (K / 2) + k / 2];
        int q = (k % 2 == 0) ? (byte & 0x0f) : (byte >> 4);
        int64_t g = m * (K / 64) + k / 64;
        return oracle_bf16_value(s[g]) * (double)q + oracle_bf16_value(b[g]);
    }
    /* OR_B1_G128 */
    {
        const uint8_t *c = (const uint8_t *)A->codes;
        const uint16_t *s = (const uint16_t *)A->scales;
        uint8_t byte = c[m * (K / 8) + k / 8];
        int bit = (byte >> (k % 8)) & 1;
        double sc = oracle_fp16_value(s[m * (K / 128) + k / 128]);
        return bit ? sc : -sc;
    }
}

/* One output: y = sum_k w[m][k] x[n][k], a = sum_k |w[m][k] x[n][k]|. */
static void dot_one(const struct qmat *A, const float *x, int64_t n, int64_t m,
                    double *y, double *a)
{
    double sum = 0.0, mag = 0.0;
    for (int64_t k = 0; k < A->K; ++k) {
        double p = weight(A, m, k) * (double)x[n * A->K + k];
        sum += p;
        mag += fabs(p);
    }
    *y = sum;
    *a = mag;
}

/* ---- exported entry points ------------------------------------------- */

/* Decode the whole matrix into w[M][K] (double). */
int oracle_decode(int fmt, const void *codes, const void *scales,
                  const void *biases, int64_t M, int64_t K, double *w)
{
    if (fmt < OR_I8_ROW || fmt > OR_I8_G64)
        return OR_BAD_FORMAT;
    if (!shape_ok(fmt, M, K))
        return OR_BAD_SHAPE;
    struct qmat A = {fmt, codes, scales, biases, M, K};
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            w[m * K + k] = weight(&A, m, k);
    return OR_OK;
}

/* y[n][m] and a[n][m] for all N activation rows and M outputs.
 * x is float32 [N][K]; y and a are double [N][M]. */
int oracle_qgemv(int fmt, const void *codes, const void *scales,
                 const void *biases, const float *x, int64_t M, int64_t K,
                 int64_t N, double *y, double *a)
{
    if (fmt < OR_I8_ROW || fmt > OR_I8_G64)
        return OR_BAD_FORMAT;
    if (!shape_ok(fmt, M, K) || N < 1)
        return OR_BAD_SHAPE;
    struct qmat A = {fmt, codes, scales, biases, M, K};
    int64_t total = N * M;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < total; ++t) {
        int64_t n = t / M, m = t % M;
        dot_one(&A, x, n, m, &y[t], &a[t]);
    }
    return OR_OK;
}

/* The same outputs for `count` chosen (n, m) pairs only: out[i] is
 * y[n_idx[i]][m_idx[i]]. Used where the full product is too large for the
 * oracle to finish in seconds. */
int oracle_qgemv_sample(int fmt, const void *codes, const void *scales,
                        const void *biases, const float *x, int64_t M,
                        int64_t K, int64_t N, const int64_t *n_idx,
                        const int64_t *m_idx, int64_t count, double *y,
                        double *a)
{
    if (fmt < OR_I8_ROW || fmt > OR_I8_G64)
        return OR_BAD_FORMAT;
    if (!shape_ok(fmt, M, K) || N < 1)
        return OR_BAD_SHAPE;
    for (int64_t i = 0; i < count; ++i)
        if (n_idx[i] < 0 || n_idx[i] >= N || m_idx[i] < 0 || m_idx[i] >= M)
            return OR_BAD_SHAPE;
    struct qmat A = {fmt, codes, scales, biases, M, K};
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        dot_one(&A, x, n_idx[i], m_idx[i], &y[i], &a[i]);
    return OR_OK;
}

/* Greedy selection over each row of y[N][M] (double): idx[n] is the lowest
 * index holding the maximum value, so ties go to the lowest index; -0 and
 * +0 compare equal. gap[n] is the maximum minus the largest value at any
 * other index (0 when the maximum is tied).
 * (Pushing the limits of legacy hardware, "Build the execution path, then
 * share the weights": greedy decoding needs only the winning vocabulary
 * index.) */
int oracle_argmax(const double *y, int64_t M, int64_t N, int32_t *idx,
                  double *gap)
{
    if (M < 1 || N < 1 || M > INT32_MAX)
        return OR_BAD_SHAPE;
    for (int64_t n = 0; n < N; ++n) {
        const double *row = y + n * M;
        int64_t best = 0;
        for (int64_t m = 1; m < M; ++m)
            if (row[m] > row[best])
                best = m;
        double second = -INFINITY;
        for (int64_t m = 0; m < M; ++m)
            if (m != best && row[m] > second)
                second = row[m];
        idx[n] = (int32_t)best;
        gap[n] = (M > 1) ? row[best] - second : INFINITY;
    }
    return OR_OK;
}

/* Embedding rows of the 4-bit format (see the header comment). */
int oracle_embed(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                 const int32_t *ids, int64_t M, int64_t K, int64_t n, float *out)
{
    if (!shape_ok(OR_U4_G64, M, K) || n < 0)
        return OR_BAD_SHAPE;
    for (int64_t t = 0; t < n; ++t) {
        const int64_t id = ids[t];
        for (int64_t k = 0; k < K; ++k) {
            float v = NAN;
            if (id >= 0 && id < M) {
                const uint8_t byte = codes[id * (K / 2) + k / 2];
                const int q = (k & 1) ? byte >> 4 : byte & 15;
                const float s = (float)oracle_bf16_value(scales[id * (K / 64) + k / 64]);
                const float b = (float)oracle_bf16_value(biases[id * (K / 64) + k / 64]);
                const float prod = s * (float)q;   /* exact: 8 x 4 significant bits */
                const float a = prod + b;          /* one float32 rounding */
                v = (float)oracle_fp16_value(oracle_f32_to_f16(a));
            }
            out[t * K + k] = v;
        }
    }
    return OR_OK;
}

/* Threads the (n, m) loops use (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the threads of the (n, m) loops (no effect without OpenMP); used to
 * time the oracle on one core and on all of them. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
