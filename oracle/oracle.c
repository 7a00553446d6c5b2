/*
 * oracle.c -- plain, slow CPU reference for the FP16 x INT4 (grouped) linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this
 * file: only the test suite, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no code, header, table or helper with the GPU library.
 *
 * What it computes (each step is cited to the pages it follows):
 *
 *   C[M x N] = A[M x K] * Bhat[K x N]
 *     -- MARLIN paper (arXiv 2408.11743) sec. 3.2, problem statement "multiplying an
 *        M x K matrix A with a K x N matrix B"; Marlin deep-dive page ("Marlin 完全拆解"),
 *        section "Marlin 要解决的精确问题", formula C = A B.
 *
 *   Bhat[k][n] = s[g][n] * (q[k][n] - z[g][n]),   g = floor(k / group),  q, z in {0..15}
 *     -- deep-dive page, same section, the dequantisation formula s_{g,n}(q_{k,n} - z_{g,n});
 *        the main path is symmetric with z = 8 (section "INT4 只是存储类型", where the zero
 *        point 8 is folded into the subtraction constant, giving q - 8), and the general
 *        affine form takes a zero point per group and column (an integer code 0..15 here,
 *        like q: the page leaves its type open).  MARLIN paper sec. 3.4 "Kernel Design":
 *        symmetric INT4, one FP16 scale per G consecutive weights in each column; sec. 2.2:
 *        groups of 128 contiguous values.  group = K is one scale per column (deep-dive
 *        page, section "scale 为什么有时在内环乘，有时在末尾乘": AB = (AQ) diag(s)).
 *
 *   Accumulation in FP32, FP16 only when C is written
 *     -- deep-dive page, section "让多个 warp 计算同一个输出 tile 的部分和": the FP32
 *        accumulators are converted to FP16 only at the final write-out.
 *
 * The fp32 oracle takes k in ascending order, multiplies then adds (the file must be
 * compiled with -ffp-contract=off so no FMA is formed), and rounds the fp32 sum to fp16
 * with round-to-nearest-even.  s*(q-z) is exact in fp32 (11-bit by 5-bit significands), so
 * the only roundings are the product a*w, each addition, and the final fp16 rounding.
 *
 * The fp64 variant is a diagnostic "truth": a*w is exact in fp64 (26 significant bits) and
 * only the additions round; the result is rounded once from fp64 to fp16.
 *
 * Half-precision conversions are this file's own bit-level routines (normals, subnormals,
 * signed zero, infinity, NaN; round-to-nearest-even; overflow to infinity).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <unistd.h>

/* ---------------------------------------------------------------- fp16 <-> fp64 */

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);  /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Correctly rounded (nearest, ties to even) conversion of a double to binary16. */
uint16_t oracle_double_to_half(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return sign | 0x7e00;
    double a = fabs(x);
    if (isinf(a))
        return sign | 0x7c00;
    if (a == 0.0)
        return sign;

    int e;
    frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
    int ex = e - 1;
    if (ex < -14)
        ex = -14;                 /* below the normal range the spacing is fixed at 2^-24 */
    double ulp = ldexp(1.0, ex - 10);
    double r = rint(a / ulp);     /* a/ulp is exact; rint rounds half to even */
    double v = r * ulp;

    if (v > 65504.0)
        return sign | 0x7c00;     /* overflow (includes the tie at 65520) */
    if (v < ldexp(1.0, -14))
        return sign | (uint16_t)(v * 16777216.0);   /* subnormal: v / 2^-24 */
    frexp(v, &e);
    ex = e - 1;
    uint32_t frac = (uint32_t)(ldexp(v, 10 - ex) - 1024.0);
    return sign | (uint16_t)((ex + 15) << 10) | (uint16_t)frac;
}

uint16_t oracle_float_to_half(float x)
{
    /* float -> double is exact, so this is a single rounding of x. */
    return oracle_double_to_half((double)x);
}

/* ---------------------------------------------------------------- dequantisation */

/* One dequantised weight, exactly: s * (q - 8). */
double oracle_dequant(uint8_t q, uint16_t s_bits)
{
    return oracle_half_to_double(s_bits) * (double)((int)q - 8);
}

/* The same with a zero point z: s * (q - z). */
double oracle_dequant_zp(uint8_t q, uint16_t s_bits, uint8_t z)
{
    return oracle_half_to_double(s_bits) * (double)((int)q - (int)z);
}

/* ---------------------------------------------------------------- GEMM */

typedef struct {
    const float *a32;        /* A converted to fp32 (exact), M x K */
    const double *a64;       /* A converted to fp64 (exact), M x K */
    const uint8_t *q;        /* codes, K x N row-major */
    const uint16_t *s;       /* scales (fp16 bits), (K/group) x N row-major */
    const uint8_t *z;        /* zero points, (K/group) x N row-major, or NULL for 8 */
    uint16_t *C;             /* output fp16 bits, M x N row-major */
    int M, K, N, group;
    int n0, n1;              /* this worker's column range */
    int wide;                /* 0: fp32 accumulation, 1: fp64 accumulation */
} oracle_job;

static void *oracle_worker(void *arg)
{
    const oracle_job *j = (const oracle_job *)arg;
    const int M = j->M, K = j->K, N = j->N;
    float *w32 = NULL;
    double *w64 = NULL;
    if (j->wide)
        w64 = (double *)malloc((size_t)K * sizeof(double));
    else
        w32 = (float *)malloc((size_t)K * sizeof(float));
    if (!w32 && !w64)
        return (void *)1;

    for (int n = j->n0; n < j->n1; ++n) {
        /* Column n of Bhat: s[floor(k/group)][n] * (q[k][n] - z[floor(k/group)][n]). */
        for (int k = 0; k < K; ++k) {
            int g = k / j->group;
            uint16_t sb = j->s[(size_t)g * N + n];
            int zp = j->z ? (int)j->z[(size_t)g * N + n] : 8;
            int qmz = (int)j->q[(size_t)k * N + n] - zp;
            if (j->wide)
                w64[k] = oracle_half_to_double(sb) * (double)qmz;
            else
                w32[k] = (float)oracle_half_to_double(sb) * (float)qmz;
        }
        /* C[m][n] = sum_k A[m][k] * Bhat[k][n], k ascending. */
        for (int m = 0; m < M; ++m) {
            if (j->wide) {
                const double *a = j->a64 + (size_t)m * K;
                double acc = 0.0;
                for (int k = 0; k < K; ++k)
                    acc = acc + a[k] * w64[k];
                j->C[(size_t)m * N + n] = oracle_double_to_half(acc);
            } else {
                const float *a = j->a32 + (size_t)m * K;
                float acc = 0.0f;
                for (int k = 0; k < K; ++k) {
                    float p = a[k] * w32[k];
                    acc = acc + p;
                }
                j->C[(size_t)m * N + n] = oracle_float_to_half(acc);
            }
        }
    }
    free(w32);
    free(w64);
    return NULL;
}

static int oracle_gemm_impl(const uint16_t *A, const uint8_t *q, const uint16_t *s,
                            const uint8_t *z, int M, int K, int N, int group, uint16_t *C,
                            int nthreads, int wide)
{
    if (!A || !q || !s || !C || M <= 0 || K <= 0 || N <= 0 || group <= 0 || K % group)
        return -1;
    for (size_t i = 0; i < (size_t)K * N; ++i)
        if (q[i] > 15)
            return -1;
    if (z)
        for (size_t i = 0; i < (size_t)(K / group) * N; ++i)
            if (z[i] > 15)
                return -1;

    size_t na = (size_t)M * K;
    float *a32 = NULL;
    double *a64 = NULL;
    if (wide)
        a64 = (double *)malloc(na * sizeof(double));
    else
        a32 = (float *)malloc(na * sizeof(float));
    if (!a32 && !a64)
        return -2;
    for (size_t i = 0; i < na; ++i) {
        double v = oracle_half_to_double(A[i]);
        if (wide)
            a64[i] = v;
        else
            a32[i] = (float)v;
    }

    if (nthreads <= 0)
        nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > N)
        nthreads = N;

    oracle_job *jobs = (oracle_job *)calloc((size_t)nthreads, sizeof(oracle_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    int rc = 0;
    if (!jobs || !tids) {
        rc = -2;
        goto done;
    }
    /* Threads split the columns; each (m, n) is summed by one thread in the same order,
     * so the thread count never changes a result. */
    for (int t = 0; t < nthreads; ++t) {
        oracle_job *j = &jobs[t];
        j->a32 = a32;
        j->a64 = a64;
        j->q = q;
        j->s = s;
        j->z = z;
        j->C = C;
        j->M = M;
        j->K = K;
        j->N = N;
        j->group = group;
        j->n0 = (int)((long long)N * t / nthreads);
        j->n1 = (int)((long long)N * (t + 1) / nthreads);
        j->wide = wide;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, oracle_worker, &jobs[t]) != 0) {
            rc = -2;
            break;
        }
        started = t;
    }
    if (rc == 0 && oracle_worker(&jobs[0]) != NULL)
        rc = -2;
    for (int t = 1; t <= started; ++t) {
        void *res = NULL;
        pthread_join(tids[t], &res);
        if (res != NULL)
            rc = -2;
    }
done:
    free(jobs);
    free(tids);
    free(a32);
    free(a64);
    return rc;
}

/* fp32 accumulation, k ascending, fp16 RNE output.  Returns 0, or -1 on bad arguments
 * (null pointer, non-positive size, K not a multiple of group, a code above 15), or -2
 * when memory or threads cannot be obtained. */
int oracle_gemm_f32(const uint16_t *A, const uint8_t *q, const uint16_t *s,
                    int M, int K, int N, int group, uint16_t *C, int nthreads)
{
    return oracle_gemm_impl(A, q, s, NULL, M, K, N, group, C, nthreads, 0);
}

/* fp64 accumulation (diagnostic truth), fp16 RNE output from fp64. */
int oracle_gemm_f64(const uint16_t *A, const uint8_t *q, const uint16_t *s,
                    int M, int K, int N, int group, uint16_t *C, int nthreads)
{
    return oracle_gemm_impl(A, q, s, NULL, M, K, N, group, C, nthreads, 1);
}

/* The same two with a zero point per group and column (z codes 0..15; NULL means 8). */
int oracle_gemm_zp_f32(const uint16_t *A, const uint8_t *q, const uint16_t *s, const uint8_t *z,
                       int M, int K, int N, int group, uint16_t *C, int nthreads)
{
    return oracle_gemm_impl(A, q, s, z, M, K, N, group, C, nthreads, 0);
}

int oracle_gemm_zp_f64(const uint16_t *A, const uint8_t *q, const uint16_t *s, const uint8_t *z,
                       int M, int K, int N, int group, uint16_t *C, int nthreads)
{
    return oracle_gemm_impl(A, q, s, z, M, K, N, group, C, nthreads, 1);
}

/* The M = 1 case written out on its own: one activation row against every column.
 * Same operation order as oracle_gemm_f32, so its output equals row 0 of the GEMM
 * bit for bit. */
int oracle_gemv_f32(const uint16_t *a, const uint8_t *q, const uint16_t *s,
                    int K, int N, int group, uint16_t *c)
{
    if (!a || !q || !s || !c || K <= 0 || N <= 0 || group <= 0 || K % group)
        return -1;
    for (int n = 0; n < N; ++n) {
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) {
            uint8_t code = q[(size_t)k * N + n];
            if (code > 15)
                return -1;
            float w = (float)oracle_half_to_double(s[(size_t)(k / group) * N + n]) *
                      (float)((int)code - 8);
            float p = (float)oracle_half_to_double(a[k]) * w;
            acc = acc + p;
        }
        c[n] = oracle_float_to_half(acc);
    }
    return 0;
}
