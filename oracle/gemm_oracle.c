/*
 * CPU oracle for the fp16 GEMM  D = A·Bᵀ  (test infrastructure only).
 *
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline
 * leg may load this file's library.  It shares no code, header or table with
 * the GPU library and never calls into it.
 *
 * What it computes (the plain definition, no blocking or reordering):
 *   - "TIRx 与高性能GEMM (上)", section "从 GEMM 公式到数据路径": D = A·Bᵀ with
 *     A of shape M×K, B of shape N×K (weight storage, so the transpose moves
 *     no data) and D of shape M×N.
 *   - "TIRx 基础", the closing 128×128×64 reference kernel: fp16 operands and
 *     output with a float32 accumulator type; "TIRx Compiler Foundation",
 *     section "Example: A GEMM Kernel": the epilogue converts with cvt.rn,
 *     i.e. round-to-nearest-even to binary16.
 * The oracle sums the exact fp16 products in float64 in increasing k and
 * rounds that float64 sum straight to binary16 (never through float32, which
 * would round twice).  Alongside it returns bound[i,j] = Σ_k |A_ik|·|B_jk|,
 * the scale of the accumulation error any fp32 summation order can make.
 *
 * Layout: A[i,k] = A[i*lda + k], B[j,k] = B[j*ldb + k], row-major, leading
 * dimensions in elements.  Outputs are dense (rows × N).
 *
 * bfloat16 variant ("从编译器能力到公开算子", section "SM90a 支持具体补了什么":
 * the matrix-multiply path takes FP16 or BF16 inputs with FP32
 * accumulation): the same definition with bfloat16 operands and output.  The
 * pages do not name the output rounding for BF16; the reading taken is the
 * fp16 one, round-to-nearest-even, applied directly from the float64 sum.
 *
 * Block-scaled FP8 variant (oracle_gemm_mx and oracle_gemm_mxf8, at the end
 * of this file): FP8 E4M3 or E5M2 operands with one 8-bit power-of-two scale
 * per 32 K elements of a row, fp16 output; its definition and readings are
 * written out there.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* binary16 → float64, exact.  Sign bit 15, exponent bits 14..10 (bias 15),
 * fraction bits 9..0; exponent 0 is the subnormal range f·2^-24. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25);
    return sign ? -v : v;
}

/* float64 → binary16 with round-to-nearest, ties to even, taken directly
 * from the float64 value.  Overflow goes to ±inf (RNE rounds 65520 and above
 * up to infinity), NaN stays NaN, subnormals are kept. */
uint16_t oracle_double_to_half(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return (uint16_t)(sign | 0x7e00);
    double a = fabs(x);
    if (isinf(a))
        return (uint16_t)(sign | 0x7c00);
    if (a == 0.0)
        return sign;
    int e;
    (void)frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
    int E = e - 1;                      /* unbiased exponent of a */
    int qexp = (E >= -14) ? E - 10 : -24; /* exponent of one fp16 ulp at a */
    double scaled = ldexp(a, -qexp);    /* exact: power-of-two scaling */
    double fl = floor(scaled);
    double frac = scaled - fl;          /* exact */
    uint64_t n = (uint64_t)fl;
    if (frac > 0.5 || (frac == 0.5 && (n & 1)))
        n += 1;
    if (E >= -14) {
        /* normal binade: n in [1024, 2048] */
        if (n == 2048) {
            n = 1024;
            qexp += 1;
        }
        int biased = qexp + 10 + 15;
        if (biased >= 31)
            return (uint16_t)(sign | 0x7c00);
        return (uint16_t)(sign | (biased << 10) | (uint16_t)(n - 1024));
    }
    /* subnormal range: n in [0, 1024]; n == 1024 is the smallest normal,
     * whose bit pattern is exactly 0x0400. */
    return (uint16_t)(sign | n);
}

/* bfloat16 → float64, exact.  Sign bit 15, exponent bits 14..7 (bias 127,
 * the binary32 range), fraction bits 6..0; exponent 0 is the subnormal
 * range f·2^-133. */
double oracle_bf16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x80), e - 134);
    return sign ? -v : v;
}

/* float64 → bfloat16, round-to-nearest, ties to even, directly from the
 * float64 value (the same construction as the binary16 one: scale to the
 * ulp at |x|, round the integer, renormalize).  Overflow to ±inf at and
 * above 2^128·(1 − 2^-9), NaN stays NaN, subnormals are kept. */
uint16_t oracle_double_to_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return (uint16_t)(sign | 0x7fc0);
    double a = fabs(x);
    if (isinf(a))
        return (uint16_t)(sign | 0x7f80);
    if (a == 0.0)
        return sign;
    int e;
    (void)frexp(a, &e);
    int E = e - 1;
    int qexp = (E >= -126) ? E - 7 : -133; /* exponent of one bf16 ulp at a */
    double scaled = ldexp(a, -qexp);
    double fl = floor(scaled);
    double frac = scaled - fl;
    uint64_t n = (uint64_t)fl;
    if (frac > 0.5 || (frac == 0.5 && (n & 1)))
        n += 1;
    if (E >= -126) {
        /* normal binade: n in [128, 256] */
        if (n == 256) {
            n = 128;
            qexp += 1;
        }
        int biased = qexp + 7 + 127;
        if (biased >= 255)
            return (uint16_t)(sign | 0x7f80);
        return (uint16_t)(sign | (biased << 7) | (uint16_t)(n - 128));
    }
    /* subnormal range: n in [0, 128]; 128 is the smallest normal, 0x0080 */
    return (uint16_t)(sign | n);
}

void oracle_bf16_to_double_array(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_to_double(h[i]);
}

void oracle_double_to_bf16_array(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_double_to_bf16(x[i]);
}

void oracle_half_to_double_array(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_half_to_double(h[i]);
}

void oracle_double_to_half_array(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_double_to_half(x[i]);
}

struct job {
    const uint16_t *A, *B;
    uint16_t *D;
    double *bound, *sum;
    int64_t N, K, lda, ldb;
    const int64_t *rows;
    int64_t nrows;
    int64_t r_begin, r_end;
    const double *lut;
    uint16_t (*encode)(double);
};

static void *run_rows(void *p)
{
    struct job *jb = (struct job *)p;
    for (int64_t r = jb->r_begin; r < jb->r_end; ++r) {
        int64_t i = jb->rows ? jb->rows[r] : r;
        const uint16_t *a = jb->A + i * jb->lda;
        for (int64_t j = 0; j < jb->N; ++j) {
            const uint16_t *b = jb->B + j * jb->ldb;
            double s = 0.0, bnd = 0.0;
            for (int64_t k = 0; k < jb->K; ++k) {
                double x = jb->lut[a[k]];
                double y = jb->lut[b[k]];
                s += x * y;           /* fp16·fp16 is exact in fp64 */
                bnd += fabs(x) * fabs(y);
            }
            int64_t o = r * jb->N + j;
            if (jb->D)
                jb->D[o] = jb->encode(s);
            if (jb->sum)
                jb->sum[o] = s;
            if (jb->bound)
                jb->bound[o] = bnd;
        }
    }
    return NULL;
}

/*
 * Reference GEMM.  Computes rows `rows[0..nrows)` of D (all M rows, in order,
 * when rows == NULL, in which case nrows must equal M).  Output row r goes to
 * D[r*N .. r*N+N), likewise for bound and sum (each may be NULL).  Work is
 * split over `nthreads` POSIX threads by output row; each element's sum is
 * taken in increasing k, so results do not depend on the thread count.
 * Returns 0, or -1 on invalid arguments.
 */
static int gemm16(const uint16_t *A, const uint16_t *B, uint16_t *D, double *bound,
                  double *sum, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                  const int64_t *rows, int64_t nrows, int nthreads,
                  double (*decode)(uint16_t), uint16_t (*encode)(double))
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || nrows < 0)
        return -1;
    if (!rows && nrows != M)
        return -1;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= M)
                return -1;
    if (nrows == 0 || N == 0)
        return 0;

    double *lut = (double *)malloc(65536 * sizeof(double));
    if (!lut)
        return -1;
    for (uint32_t h = 0; h < 65536; ++h)
        lut[h] = decode((uint16_t)h);

    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > nrows)
        nthreads = (int)nrows;
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    struct job *jobs = (struct job *)calloc((size_t)nthreads, sizeof(struct job));
    if (!th || !jobs) {
        free(lut);
        free(th);
        free(jobs);
        return -1;
    }
    int64_t per = nrows / nthreads, extra = nrows % nthreads, start = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t cnt = per + (t < extra ? 1 : 0);
        struct job jb = {A, B, D, bound, sum, N, K, lda, ldb, rows, nrows,
                         start, start + cnt, lut, encode};
        jobs[t] = jb;
        start += cnt;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, run_rows, &jobs[t]) != 0)
            break;
        started = t;
    }
    run_rows(&jobs[0]);
    for (int t = 1; t <= started; ++t)
        pthread_join(th[t], NULL);
    /* any job whose thread could not start runs here */
    for (int t = started + 1; t < nthreads; ++t)
        run_rows(&jobs[t]);
    free(lut);
    free(th);
    free(jobs);
    return 0;
}

int oracle_gemm_f16(const uint16_t *A, const uint16_t *B, uint16_t *D,
                    double *bound, double *sum,
                    int64_t M, int64_t N, int64_t K,
                    int64_t lda, int64_t ldb,
                    const int64_t *rows, int64_t nrows, int nthreads)
{
    return gemm16(A, B, D, bound, sum, M, N, K, lda, ldb, rows, nrows, nthreads,
                  oracle_half_to_double, oracle_double_to_half);
}

/* The same GEMM on bfloat16 operands and output (products exact in fp64). */
int oracle_gemm_bf16(const uint16_t *A, const uint16_t *B, uint16_t *D,
                     double *bound, double *sum,
                     int64_t M, int64_t N, int64_t K,
                     int64_t lda, int64_t ldb,
                     const int64_t *rows, int64_t nrows, int nthreads)
{
    return gemm16(A, B, D, bound, sum, M, N, K, lda, ldb, rows, nrows, nthreads,
                  oracle_bf16_to_double, oracle_double_to_bf16);
}

/*
 * Block-scaled FP8 GEMM ("TIRx Layout API", section "Scale Factor 布局":
 * block-scaled MMA, where the K elements of a row come in groups that share
 * one 8-bit scale factor; the same page's TMEM section names the
 * block-scaled FP8 GEMM).  The pages fix neither the element encoding nor the
 * group length.  The reading taken is OCP MX: elements are FP8 E4M3 (sign,
 * 4 exponent bits with bias 7, 3 fraction bits; no infinities, S.1111.111 is
 * NaN, largest finite 448); every 32 consecutive K elements of a row share
 * one UE8M0 scale byte s worth 2^(s-127) (s = 255 is NaN); the product is
 * accumulated and rounded to binary16 like the fp16 GEMM:
 *
 *   D[i,j] = RNE16( Σ_k (SA[i,k/32]·A[i,k]) · (SB[j,k/32]·B[j,k]) )
 *
 * with A[i,k] = A[i*lda+k], SA[i,b] = SA[i*ldsa+b] (bytes), likewise B, SB.
 * Every term is exact in float64 (two 4-bit significands and powers of two
 * within float64's range); the sum is taken in increasing k.
 *
 * OCP MX also defines the FP8 element encoding E5M2 (sign, 5 exponent bits
 * with bias 15, 2 fraction bits, with infinities: exponent 31 is ±infinity
 * for fraction 0 and NaN otherwise; largest finite 57344).  oracle_gemm_mx
 * takes the encoding of A and of B separately (0 E4M3, 1 E5M2); an infinite
 * element times a zero one gives NaN and infinities propagate through the
 * sum as IEEE float64 arithmetic has them, and the result rounds to a signed
 * infinity when it exceeds binary16's range, as for the fp16 GEMM.
 */

/* E4M3 → float64, exact: exponent 0 is the subnormal range f·2^-9, otherwise
 * (8+f)·2^(e-10). */
double oracle_e4m3_to_double(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 15;
    int f = b & 7;
    double v;
    if (e == 15 && f == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)f, -9);
    else
        v = ldexp((double)(8 | f), e - 10);
    return sign ? -v : v;
}

/* E5M2 → float64, exact: exponent 31 is ±infinity (fraction 0) or NaN,
 * exponent 0 the subnormal range f·2^-16, otherwise (4+f)·2^(e-17). */
double oracle_e5m2_to_double(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int e = (b >> 2) & 31;
    int f = b & 3;
    double v;
    if (e == 31)
        v = f == 0 ? INFINITY : NAN;
    else if (e == 0)
        v = ldexp((double)f, -16);
    else
        v = ldexp((double)(4 | f), e - 17);
    return sign ? -v : v;
}

/* UE8M0 scale byte → float64: 2^(s-127), NaN for 255. */
double oracle_e8m0_to_double(uint8_t s)
{
    return s == 255 ? NAN : ldexp(1.0, (int)s - 127);
}

void oracle_e4m3_to_double_array(const uint8_t *b, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_to_double(b[i]);
}

void oracle_e5m2_to_double_array(const uint8_t *b, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e5m2_to_double(b[i]);
}

struct mx_job {
    const uint8_t *A, *SA, *B, *SB;
    uint16_t *D;
    double *bound, *sum;
    int64_t N, K, lda, ldsa, ldb, ldsb;
    const int64_t *rows;
    int64_t r_begin, r_end;
    const double *alut, *blut, *slut;
};

static void *run_rows_mx(void *p)
{
    struct mx_job *jb = (struct mx_job *)p;
    for (int64_t r = jb->r_begin; r < jb->r_end; ++r) {
        int64_t i = jb->rows ? jb->rows[r] : r;
        const uint8_t *a = jb->A + i * jb->lda;
        const uint8_t *sa = jb->SA + i * jb->ldsa;
        for (int64_t j = 0; j < jb->N; ++j) {
            const uint8_t *b = jb->B + j * jb->ldb;
            const uint8_t *sb = jb->SB + j * jb->ldsb;
            double s = 0.0, bnd = 0.0;
            for (int64_t k = 0; k < jb->K; ++k) {
                double x = jb->slut[sa[k / 32]] * jb->alut[a[k]];
                double y = jb->slut[sb[k / 32]] * jb->blut[b[k]];
                s += x * y;
                bnd += fabs(x) * fabs(y);
            }
            int64_t o = r * jb->N + j;
            if (jb->D)
                jb->D[o] = oracle_double_to_half(s);
            if (jb->sum)
                jb->sum[o] = s;
            if (jb->bound)
                jb->bound[o] = bnd;
        }
    }
    return NULL;
}

/* Reference block-scaled GEMM; rows, outputs, threads and the return value as
 * for oracle_gemm_f16.  ldsa and ldsb count scale bytes per row and must
 * cover ceil(K/32) blocks; a_fmt and b_fmt are the element encodings of A
 * and B (0 E4M3, 1 E5M2). */
int oracle_gemm_mx(const uint8_t *A, const uint8_t *SA, const uint8_t *B, const uint8_t *SB,
                   uint16_t *D, double *bound, double *sum,
                   int64_t M, int64_t N, int64_t K,
                   int64_t lda, int64_t ldsa, int64_t ldb, int64_t ldsb, int a_fmt, int b_fmt,
                   const int64_t *rows, int64_t nrows, int nthreads)
{
    const int64_t blocks = (K + 31) / 32;
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || ldsa < blocks || ldsb < blocks || nrows < 0)
        return -1;
    if (a_fmt < 0 || a_fmt > 1 || b_fmt < 0 || b_fmt > 1)
        return -1;
    if (!rows && nrows != M)
        return -1;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= M)
                return -1;
    if (nrows == 0 || N == 0)
        return 0;

    double alut[256], blut[256], slut[256];
    for (int v = 0; v < 256; ++v) {
        alut[v] = a_fmt ? oracle_e5m2_to_double((uint8_t)v) : oracle_e4m3_to_double((uint8_t)v);
        blut[v] = b_fmt ? oracle_e5m2_to_double((uint8_t)v) : oracle_e4m3_to_double((uint8_t)v);
        slut[v] = oracle_e8m0_to_double((uint8_t)v);
    }
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > nrows)
        nthreads = (int)nrows;
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    struct mx_job *jobs = (struct mx_job *)calloc((size_t)nthreads, sizeof(struct mx_job));
    if (!th || !jobs) {
        free(th);
        free(jobs);
        return -1;
    }
    int64_t per = nrows / nthreads, extra = nrows % nthreads, start = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t cnt = per + (t < extra ? 1 : 0);
        struct mx_job jb = {A, SA, B, SB, D, bound, sum, N, K, lda, ldsa, ldb, ldsb, rows,
                            start, start + cnt, alut, blut, slut};
        jobs[t] = jb;
        start += cnt;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, run_rows_mx, &jobs[t]) != 0)
            break;
        started = t;
    }
    run_rows_mx(&jobs[0]);
    for (int t = 1; t <= started; ++t)
        pthread_join(th[t], NULL);
    for (int t = started + 1; t < nthreads; ++t)
        run_rows_mx(&jobs[t]);
    free(th);
    free(jobs);
    return 0;
}

/* E4M3 on both operands. */
int oracle_gemm_mxf8(const uint8_t *A, const uint8_t *SA, const uint8_t *B, const uint8_t *SB,
                     uint16_t *D, double *bound, double *sum,
                     int64_t M, int64_t N, int64_t K,
                     int64_t lda, int64_t ldsa, int64_t ldb, int64_t ldsb,
                     const int64_t *rows, int64_t nrows, int nthreads)
{
    return oracle_gemm_mx(A, SA, B, SB, D, bound, sum, M, N, K, lda, ldsa, ldb, ldsb, 0, 0, rows, nrows,
                          nthreads);
}
