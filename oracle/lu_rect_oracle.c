/*
 * lu_rect_oracle.c -- plain, slow CPU oracle for batched LU with partial
 * pivoting of m x n matrices (getrf on a rectangular A).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header or constant with the HIP path.
 *
 * What it follows: BatchLAS performance notes, "LU" page, the family table
 * (getrf on a non-square A, and batches whose matrices differ in size, are
 * routed to the vendor library there: LAPACK's getrf meaning), with the
 * same step readings as the square oracle in lu_oracle.c:
 *   R1  pivot metric |x| (complex |re| + |im|); a NaN ranks above every
 *       number and the first NaN wins; ties go to the lowest row;
 *   R2  a zero pivot skips scaling and the rank-1 update; info keeps the
 *       first such step (1-based); ipiv is still recorded;
 *   R3  l = a * r with r = 1/pivot rounded once (complex: Smith's
 *       reciprocal), a / pivot when the pivot metric is below the smallest
 *       normal;
 *   R4  a_ik = fma(-l_ij, u_jk, a_ik) for i > j, k > j, column k outer;
 *       complex z -= x*y as re: -xr*yr then +xi*yi, im: -xr*yi then -xi*yr;
 *       complex l = a*r as re = fma(ar, rr, -(ai*ri)), im = fma(ar, ri, ai*rr).
 * For an m x n matrix there are min(m, n) steps: step j searches rows j ..
 * m-1 of column j, swaps whole rows (all n columns), scales rows j+1 .. m-1
 * and updates columns j+1 .. n-1 (LAPACK getf2 on a rectangular matrix).
 * ipiv holds min(m, n) entries.
 *
 * Arithmetic is in the working precision of the data type; margins are
 * reported in double.  Build with -ffp-contract=off.
 */
#include <math.h>
#include <float.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { RT_R32 = 0, RT_R64 = 1, RT_C64 = 2, RT_C128 = 3 };

/* R1: x ranks above best */
static int rt_above(double x, double best)
{
    if (isnan(best)) return 0;
    if (isnan(x)) return 1;
    return x > best;
}

static double rt_margin(double winner, double runner, int have_runner)
{
    if (!have_runner) return 0.0;
    if (isnan(winner)) return isnan(runner) ? 1.0 : 0.0;
    if (winner == 0.0) return 1.0;
    return runner / winner;
}

#define RT_IDX(i, k) ((size_t)(i) + (size_t)(k) * (size_t)lda)

#define DEFINE_RECT_REAL(NAME, T, FMA, FABS, SFMIN)                            \
static void NAME(int m, int n, T* A, int lda, int* ipiv, int* info,            \
                 double* margin)                                               \
{                                                                              \
    const int steps = m < n ? m : n;                                           \
    *info = 0;                                                                 \
    for (int j = 0; j < steps; ++j) {                                          \
        int p = j;                                                             \
        T best = FABS(A[RT_IDX(j, j)]);                                        \
        double runner = 0.0; int have = 0;                                     \
        for (int i = j + 1; i < m; ++i) {                                      \
            T v = FABS(A[RT_IDX(i, j)]);                                       \
            if (rt_above((double)v, (double)best)) {                           \
                runner = (double)best; have = 1; best = v; p = i;              \
            } else if (!have || rt_above((double)v, runner)) {                 \
                runner = (double)v; have = 1;                                  \
            }                                                                  \
        }                                                                      \
        if (margin) margin[j] = rt_margin((double)best, runner, have);         \
        ipiv[j] = p + 1;                                                       \
        if (p != j)                                                            \
            for (int k = 0; k < n; ++k) {                                      \
                T t = A[RT_IDX(j, k)];                                         \
                A[RT_IDX(j, k)] = A[RT_IDX(p, k)];                             \
                A[RT_IDX(p, k)] = t;                                           \
            }                                                                  \
        const T piv = A[RT_IDX(j, j)];                                         \
        if (FABS(piv) == (T)0) {                                /* R2 */       \
            if (*info == 0) *info = j + 1;                                     \
            continue;                                                          \
        }                                                                      \
        if (FABS(piv) >= SFMIN) {                               /* R3 */       \
            const T r = (T)1 / piv;                                            \
            for (int i = j + 1; i < m; ++i) A[RT_IDX(i, j)] = A[RT_IDX(i, j)] * r; \
        } else {                                                               \
            for (int i = j + 1; i < m; ++i) A[RT_IDX(i, j)] = A[RT_IDX(i, j)] / piv; \
        }                                                                      \
        for (int k = j + 1; k < n; ++k) {                       /* R4 */       \
            const T u = A[RT_IDX(j, k)];                                       \
            for (int i = j + 1; i < m; ++i)                                    \
                A[RT_IDX(i, k)] = FMA(-A[RT_IDX(i, j)], u, A[RT_IDX(i, k)]);   \
        }                                                                      \
    }                                                                          \
}

DEFINE_RECT_REAL(rect_sgetrf, float, fmaf, fabsf, FLT_MIN)
DEFINE_RECT_REAL(rect_dgetrf, double, fma, fabs, DBL_MIN)

/* complex: element (i, k) is A[2 * RT_IDX(i, k)] (re) and the next (im) */
#define DEFINE_RECT_COMPLEX(PFX, T, FMA, FABS, SFMIN)                          \
static T PFX##_metric(const T* z) { return FABS(z[0]) + FABS(z[1]); }          \
static void PFX##_smith_recip(T c, T d, T* out)                                \
{                                                                              \
    if (FABS(c) >= FABS(d)) {                                                  \
        T e = d / c; T f = c + d * e;                                          \
        out[0] = (T)1 / f; out[1] = -e / f;                                    \
    } else {                                                                   \
        T e = c / d; T f = d + c * e;                                          \
        out[0] = e / f; out[1] = -(T)1 / f;                                    \
    }                                                                          \
}                                                                              \
static void PFX##_smith_div(T a, T b, T c, T d, T* out)                        \
{                                                                              \
    if (FABS(c) >= FABS(d)) {                                                  \
        T e = d / c; T f = c + d * e;                                          \
        out[0] = (a + b * e) / f; out[1] = (b - a * e) / f;                    \
    } else {                                                                   \
        T e = c / d; T f = d + c * e;                                          \
        out[0] = (a * e + b) / f; out[1] = (b * e - a) / f;                    \
    }                                                                          \
}                                                                              \
static void PFX##_scale(T* a, const T* r)                                      \
{                                                                              \
    T t = a[1] * r[1];                                                         \
    T re = FMA(a[0], r[0], -t);                                                \
    T t2 = a[1] * r[0];                                                        \
    T im = FMA(a[0], r[1], t2);                                                \
    a[0] = re; a[1] = im;                                                      \
}                                                                              \
static void PFX##_update(T* z, const T* x, const T* y)                         \
{                                                                              \
    T re = FMA(-x[0], y[0], z[0]);                                             \
    re = FMA(x[1], y[1], re);                                                  \
    T im = FMA(-x[0], y[1], z[1]);                                             \
    im = FMA(-x[1], y[0], im);                                                 \
    z[0] = re; z[1] = im;                                                      \
}                                                                              \
static void rect_##PFX##getrf(int m, int n, T* A, int lda, int* ipiv,          \
                              int* info, double* margin)                       \
{                                                                              \
    const int steps = m < n ? m : n;                                           \
    *info = 0;                                                                 \
    for (int j = 0; j < steps; ++j) {                                          \
        int p = j;                                                             \
        T best = PFX##_metric(A + 2 * RT_IDX(j, j));                           \
        double runner = 0.0; int have = 0;                                     \
        for (int i = j + 1; i < m; ++i) {                                      \
            T v = PFX##_metric(A + 2 * RT_IDX(i, j));                          \
            if (rt_above((double)v, (double)best)) {                           \
                runner = (double)best; have = 1; best = v; p = i;              \
            } else if (!have || rt_above((double)v, runner)) {                 \
                runner = (double)v; have = 1;                                  \
            }                                                                  \
        }                                                                      \
        if (margin) margin[j] = rt_margin((double)best, runner, have);         \
        ipiv[j] = p + 1;                                                       \
        if (p != j)                                                            \
            for (int k = 0; k < n; ++k)                                        \
                for (int h = 0; h < 2; ++h) {                                  \
                    T t = A[2 * RT_IDX(j, k) + h];                             \
                    A[2 * RT_IDX(j, k) + h] = A[2 * RT_IDX(p, k) + h];         \
                    A[2 * RT_IDX(p, k) + h] = t;                               \
                }                                                              \
        const T* piv = A + 2 * RT_IDX(j, j);                                   \
        const T pm = PFX##_metric(piv);                                        \
        if (pm == (T)0) {                                       /* R2 */       \
            if (*info == 0) *info = j + 1;                                     \
            continue;                                                          \
        }                                                                      \
        if (pm >= SFMIN) {                                      /* R3 */       \
            T r[2]; PFX##_smith_recip(piv[0], piv[1], r);                      \
            for (int i = j + 1; i < m; ++i) PFX##_scale(A + 2 * RT_IDX(i, j), r); \
        } else {                                                               \
            for (int i = j + 1; i < m; ++i) {                                  \
                T* a = A + 2 * RT_IDX(i, j);                                   \
                PFX##_smith_div(a[0], a[1], piv[0], piv[1], a);                \
            }                                                                  \
        }                                                                      \
        for (int k = j + 1; k < n; ++k) {                       /* R4 */       \
            const T* u = A + 2 * RT_IDX(j, k);                                 \
            for (int i = j + 1; i < m; ++i)                                    \
                PFX##_update(A + 2 * RT_IDX(i, k), A + 2 * RT_IDX(i, j), u);   \
        }                                                                      \
    }                                                                          \
}

DEFINE_RECT_COMPLEX(c, float, fmaf, fabsf, FLT_MIN)
DEFINE_RECT_COMPLEX(z, double, fma, fabs, DBL_MIN)

typedef struct {
    int t, m, n;
    char* A; int lda; long long sA;
    int* ipiv; long long sP;
    int* info;
    double* margin;     /* min(m, n) per matrix, may be NULL */
    int begin, end;
} rt_job_t;

static size_t rt_elem(int t) { return t == RT_R32 ? 4 : (t == RT_C128 ? 16 : 8); }

static void* rt_worker(void* arg)
{
    rt_job_t* J = (rt_job_t*)arg;
    const int steps = J->m < J->n ? J->m : J->n;
    for (int b = J->begin; b < J->end; ++b) {
        void* A = J->A + (size_t)b * J->sA * rt_elem(J->t);
        int* ip = J->ipiv + (size_t)b * J->sP;
        double* mg = J->margin ? J->margin + (size_t)b * steps : NULL;
        switch (J->t) {
        case RT_R32: rect_sgetrf(J->m, J->n, (float*)A, J->lda, ip, J->info + b, mg); break;
        case RT_R64: rect_dgetrf(J->m, J->n, (double*)A, J->lda, ip, J->info + b, mg); break;
        case RT_C64: rect_cgetrf(J->m, J->n, (float*)A, J->lda, ip, J->info + b, mg); break;
        case RT_C128: rect_zgetrf(J->m, J->n, (double*)A, J->lda, ip, J->info + b, mg); break;
        }
    }
    return NULL;
}

/* Factor `batch` m x n matrices (element (i, k) of matrix b at
   A + b*strideA + i + k*lda) in place.  Returns the host threads used. */
int oracle_getrf_rect_batch(int t, int m, int n, void* A, int lda, long long strideA,
                            int* ipiv, long long strideP, int* info, double* margin,
                            int batch, int nthreads)
{
    if (batch <= 0) return 0;
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > batch) nthreads = batch;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    rt_job_t jobs[256];
    for (int k = 0; k < nthreads; ++k) {
        rt_job_t J = {t, m, n, (char*)A, lda, strideA, ipiv, strideP, info, margin, 0, 0};
        J.begin = (int)((long long)batch * k / nthreads);
        J.end = (int)((long long)batch * (k + 1) / nthreads);
        jobs[k] = J;
    }
    int started = 0;
    for (int k = 1; k < nthreads; ++k)
        if (pthread_create(&th[k], NULL, rt_worker, &jobs[k]) == 0) started = k;
        else break;
    rt_worker(&jobs[0]);
    for (int k = 1; k <= started; ++k) pthread_join(th[k], NULL);
    for (int k = started + 1; k < nthreads; ++k) rt_worker(&jobs[k]);
    return nthreads;
}
