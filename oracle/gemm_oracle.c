/*
 * CPU oracle for C = A . B with FP16, BF16 or FP8 (E4M3) operands
 * -- TEST INFRASTRUCTURE.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this file's library.  It shares no code, header or table with the GPU
 * path and must never be called by the product.
 *
 * What it computes (the plain definition of the product the tiled GEMM on
 * "Two Waves, One Stage Apart: Warp-Pipelining Triton GEMMs on AMD Instinct"
 * evaluates; opening section: compute on one operand-tile pair while the next
 * is prepared, i.e. a dense C = A.B, with throughput counted as 2MNK / time
 * under its Table 1):
 *
 *     Cref[i][j] = sum_{k=0}^{K-1} a(i,k) * b(k,j)
 *     Sabs[i][j] = sum_{k=0}^{K-1} |a(i,k) * b(k,j)|
 *
 *   a(i,k) = A[i*lda + k]
 *   b(k,j) = B[k*ldb + j]   if trans_b == 0   (B stored K x N, row-major)
 *          = B[j*ldb + k]   if trans_b == 1   (B stored N x K, row-major)
 *
 * Every operand is widened exactly to double (binary16, bfloat16 and FP8 E4M3
 * values are all representable in binary64), products are exact in binary64
 * (at most 2 x 11 significant bits), and the sum runs over increasing k from
 * +0.0 in binary64.  FP8 operands are one byte per element, the others two.  Rows of C are split across threads; each element is one thread's
 * plain loop, so the result does not depend on the thread count.
 *
 * The output-rounding helpers implement round-to-nearest-even from the
 * IEEE 754-2008 binary16 / bfloat16 formats (bfloat16 = binary32 with the low
 * 16 fraction bits dropped).
 *
 * Compile with -ffp-contract=off and without -ffast-math.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- operand decoding (exact) ------------------------------------------ */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* zero or subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);   /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xFF;
    int f = b & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);              /* f * 2^-126 * 2^-7 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);   /* (1 + f/2^7) * 2^(e-127) */
    return sign ? -v : v;
}

/* FP8 E4M3 (the OCP 8-bit "E4M3" format with no infinities, as the FP8 MFMA
 * of "Porting High-Performance HIP Kernels to FlyDSL", section "MFMA in
 * FlyDSL", takes it): 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits;
 * exponent field 15 with fraction 7 is NaN, every other pattern is finite
 * (largest 448). */
double oracle_fp8e4m3_to_f64(uint8_t x)
{
    int sign = (x >> 7) & 1;
    int e = (x >> 3) & 0xF;
    int f = x & 0x7;
    double v;
    if (e == 0)
        v = ldexp((double)f, -9);                /* f/8 * 2^(1-7) */
    else if (e == 15 && f == 7)
        v = NAN;
    else
        v = ldexp((double)(8 + f), e - 10);      /* (1 + f/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* Element idx of an operand array of type elem (0 FP16, 1 BF16, 2 FP8 E4M3). */
static double load(int elem, const void *p, int64_t idx)
{
    if (elem == 2)
        return oracle_fp8e4m3_to_f64(((const uint8_t *)p)[idx]);
    uint16_t h = ((const uint16_t *)p)[idx];
    return elem == 0 ? oracle_f16_to_f64(h) : oracle_bf16_to_f64(h);
}

/* ---- output rounding (round to nearest, ties to even) ------------------- */

/* Round |x| (finite, >= 0) to a multiple of 2^q, ties to even multiple. */
static double rne_to_quantum(double ax, int q)
{
    double s = ldexp(ax, -q);            /* exact: scaling by a power of two */
    double fl = floor(s);
    double rem = s - fl;                 /* exact */
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0))
        fl += 1.0;
    return ldexp(fl, q);
}

uint16_t oracle_f64_to_f16_rne(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return 0x7E00;
    double ax = fabs(x);
    if (isinf(ax))
        return sign | 0x7C00;
    /* quantum: 2^-24 for subnormals, else 2^(E-10) where 2^E <= |x| < 2^(E+1) */
    int E;
    if (ax < ldexp(1.0, -14))
        E = -14;
    else {
        frexp(ax, &E);                    /* ax = m * 2^E, m in [0.5, 1) */
        E -= 1;
    }
    double r = rne_to_quantum(ax, E - 10);
    if (r > 65504.0)                      /* past the largest finite binary16 */
        return sign | 0x7C00;
    if (r < ldexp(1.0, -14))              /* subnormal (or zero) */
        return sign | (uint16_t)ldexp(r, 24);
    int re;
    double m = frexp(r, &re);             /* r = m * 2^re, m in [0.5,1) */
    int exp16 = re - 1 + 15;
    uint16_t frac = (uint16_t)(ldexp(m, 11) - 1024.0);
    return sign | (uint16_t)(exp16 << 10) | frac;
}

uint16_t oracle_f64_to_bf16_rne(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return 0x7FC0;
    double ax = fabs(x);
    if (isinf(ax))
        return sign | 0x7F80;
    int E;
    if (ax < ldexp(1.0, -126))
        E = -126;
    else {
        frexp(ax, &E);
        E -= 1;
    }
    double r = rne_to_quantum(ax, E - 7);
    if (r >= ldexp(1.0, 128))              /* past the largest finite bfloat16 */
        return sign | 0x7F80;
    if (r < ldexp(1.0, -126))
        return sign | (uint16_t)ldexp(r, 133);
    int re;
    double m = frexp(r, &re);
    int exp8 = re - 1 + 127;
    uint16_t frac = (uint16_t)(ldexp(m, 8) - 128.0);
    return sign | (uint16_t)(exp8 << 7) | frac;
}

/* ---- the product -------------------------------------------------------- */

struct job {
    int elem;
    int64_t K, N;
    const void *A;
    int64_t lda;
    const double *bt;      /* b(k,j) widened, stored at bt[j*K + k] */
    int64_t row0, row1;    /* rows of C computed by the whole call */
    double *C, *S;         /* (row1-row0) x N, row-major */
    int tid, nthreads;
};

static void *rows_worker(void *p)
{
    struct job *jb = (struct job *)p;
    double *arow = (double *)malloc(sizeof(double) * (size_t)(jb->K > 0 ? jb->K : 1));
    for (int64_t i = jb->row0 + jb->tid; i < jb->row1; i += jb->nthreads) {
        for (int64_t k = 0; k < jb->K; ++k)
            arow[k] = load(jb->elem, jb->A, i * jb->lda + k);
        for (int64_t j = 0; j < jb->N; ++j) {
            const double *bcol = jb->bt + j * jb->K;
            double s = 0.0, sa = 0.0;
            for (int64_t k = 0; k < jb->K; ++k) {
                double p = arow[k] * bcol[k];
                s += p;
                sa += fabs(p);
            }
            jb->C[(i - jb->row0) * jb->N + j] = s;
            if (jb->S)
                jb->S[(i - jb->row0) * jb->N + j] = sa;
        }
    }
    free(arow);
    return NULL;
}

/*
 * Rows row0..row1-1 of Cref (and Sabs if S != NULL), each (row1-row0) x N
 * row-major.  elem: 0 = FP16 operands, 1 = BF16, 2 = FP8 E4M3 (one byte per
 * element; leading dimensions are in elements).
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_gemm_rows(int elem, int64_t M, int64_t N, int64_t K,
                     const void *A, int64_t lda,
                     const void *B, int64_t ldb, int trans_b,
                     int64_t row0, int64_t row1,
                     double *C, double *S, int nthreads)
{
    if (elem < 0 || elem > 2)
        return -1;
    if (M < 0 || N < 0 || K < 0 || row0 < 0 || row1 > M || row0 > row1)
        return -1;
    if (trans_b != 0 && trans_b != 1)
        return -1;
    if (nthreads < 1)
        nthreads = 1;

    double *bt = (double *)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
    if (!bt)
        return -1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j)
            bt[j * K + k] = load(elem, B, trans_b ? j * ldb + k : k * ldb + j);

    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    struct job *jobs = (struct job *)malloc(sizeof(struct job) * (size_t)nthreads);
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (struct job){elem, K, N, A, lda, bt, row0, row1, C, S, t, nthreads};
        if (nthreads == 1)
            rows_worker(&jobs[t]);
        else
            pthread_create(&th[t], NULL, rows_worker, &jobs[t]);
    }
    if (nthreads > 1)
        for (int t = 0; t < nthreads; ++t)
            pthread_join(th[t], NULL);
    free(jobs);
    free(th);
    free(bt);
    return 0;
}

/*
 * Cref and Sabs at n chosen points (ii[p], jj[p]); same definition as above,
 * each point one plain k-loop.  Used for sampled checks of large products.
 */
int oracle_gemm_points(int elem, int64_t M, int64_t N, int64_t K,
                       const void *A, int64_t lda,
                       const void *B, int64_t ldb, int trans_b,
                       int64_t n, const int64_t *ii, const int64_t *jj,
                       double *C, double *S)
{
    if (elem < 0 || elem > 2)
        return -1;
    if (trans_b != 0 && trans_b != 1)
        return -1;
    for (int64_t p = 0; p < n; ++p) {
        int64_t i = ii[p], j = jj[p];
        if (i < 0 || i >= M || j < 0 || j >= N)
            return -1;
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = load(elem, A, i * lda + k);
            double b = load(elem, B, trans_b ? j * ldb + k : k * ldb + j);
            s += a * b;
            sa += fabs(a * b);
        }
        C[p] = s;
        if (S)
            S[p] = sa;
    }
    return 0;
}

/* Vectorised conveniences over n values (bit patterns in / out). */
void oracle_decode(int elem, int64_t n, const void *in, double *out)
{
    for (int64_t p = 0; p < n; ++p)
        out[p] = load(elem, in, p);
}

void oracle_round(int elem, int64_t n, const double *in, uint16_t *out)
{
    for (int64_t p = 0; p < n; ++p)
        out[p] = elem == 0 ? oracle_f64_to_f16_rne(in[p]) : oracle_f64_to_bf16_rne(in[p]);
}
