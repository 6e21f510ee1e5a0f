/*
 * lu_oracle.c -- plain, slow CPU oracle for batched LU with partial pivoting
 * (getrf), the LU solve (getrs) and their composition (gesv).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or constant with the
 * HIP path.
 *
 * What it follows (BatchLAS performance notes, "LU" page):
 *   - the host oracle paragraph: a BLAS-free triple-loop getf2 that records,
 *     at every elimination step, margin = metric(runner-up) / metric(winner);
 *   - the tiny-tier paragraph: pivot metric cabs1 (|re| + |im|) for complex,
 *     ties resolved to the lowest row, a NaN must be mapped, ipiv is 1-based,
 *     elimination continues past a zero pivot, info names the first failure;
 *   - the getrs paragraphs: permutation, forward substitution against the
 *     unit-lower L, back substitution against U.
 * and, for the reciprocal-then-multiply scaling, the Blackwell page's getrs
 * tiny paragraph (one reciprocal per row instead of a divide per element).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   R1  NaN ranks above every number, Inf included; among NaNs the first wins.
 *   R2  A zero pivot (metric == 0) skips scaling and the rank-1 update; info
 *       keeps the first such step (1-based); ipiv is still recorded.
 *   R3  Multipliers are l = a * r with r = 1/pivot rounded once; when the
 *       pivot metric is below the smallest normal the multiplier is a / pivot.
 *       Complex 1/p and a/p use Smith's algorithm, every operation rounded.
 *   R4  The rank-1 update is one fused multiply-add per element and step,
 *       a_ik = fma(-l_ij, u_jk, a_ik), steps in ascending j.  Complex
 *       z -= x*y is four real fmas in the order re: -xr*yr, +xi*yi;
 *       im: -xr*yi, -xi*yr.  Complex l = a*r is re = fma(ar, rr, -(ai*ri)),
 *       im = fma(ar, ri, ai*rr).
 *   R5  getrs: x_k = y_k / u_kk (true division), then y_i -= u_ik * x_k.
 *   R6  gesv leaves B untouched for a matrix whose info > 0.
 *   R7  getrs with op(A) = A^T or A^H (the pages name a Trans solve kernel
 *       and test every transpose without spelling it out): LAPACK's meaning,
 *       A^T = U^T L^T P, solved as U^T w = b with true division by u_kk,
 *       then L^T z = w, then x = P^T z (transpositions in reverse order);
 *       A^H uses the conjugates of the factors.  Forward sums run in
 *       ascending k, backward sums in descending k, as in R5.
 *   R8  getri (inverse from the factors; the LU page's getri row describes
 *       only how the pivoting is undone without a separate pass, not the
 *       arithmetic): C = A^{-1} as the solution of A C = I with the
 *       NoTrans solve of R5, out of place.
 *
 * Arithmetic is in the working precision of the data type (the pivot choice
 * must be reproduced exactly); margins are reported in double.  Build with
 * -ffp-contract=off so that no multiply-add is fused behind our back.
 */
#include <math.h>
#include <float.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { OR_R32 = 0, OR_R64 = 1, OR_C64 = 2, OR_C128 = 3 };

/* ------------------------------------------------------------------ */
/* pivot comparison with the NaN reading R1                            */
/* ------------------------------------------------------------------ */
static int better_d(double x, double best)
{
    if (isnan(best)) return 0;      /* an earlier NaN is never displaced */
    if (isnan(x)) return 1;         /* a NaN beats every number          */
    return x > best;                /* strict: ties keep the lower row   */
}

static double step_margin(double winner, double runner, int have_runner)
{
    if (!have_runner) return 0.0;
    if (isnan(winner)) return isnan(runner) ? 1.0 : 0.0;
    if (winner == 0.0) return 1.0;
    return runner / winner;
}

/* ------------------------------------------------------------------ */
/* real getf2: one template body for float and double                  */
/* ------------------------------------------------------------------ */
#define DEFINE_REAL_GETRF(NAME, T, FMA, FABS, SFMIN)                           \
void NAME(int n, T* A, int lda, int* ipiv, int* info, double* margin)          \
{                                                                              \
    *info = 0;                                                                 \
    for (int j = 0; j < n; ++j) {                                              \
        /* a1: first argmax of |a_ij| over i >= j, with runner-up */          \
        int p = j;                                                             \
        T best = FABS(A[j + (size_t)j * lda]);                                 \
        double runner = 0.0; int have_runner = 0;                              \
        for (int i = j + 1; i < n; ++i) {                                      \
            T m = FABS(A[i + (size_t)j * lda]);                                \
            if (better_d((double)m, (double)best)) {                           \
                runner = (double)best; have_runner = 1;                        \
                best = m; p = i;                                               \
            } else if (!have_runner || better_d((double)m, runner)) {          \
                runner = (double)m; have_runner = 1;                           \
            }                                                                  \
        }                                                                      \
        if (margin) margin[j] = step_margin((double)best, runner, have_runner);\
        ipiv[j] = p + 1;                                                       \
        /* a2: swap whole rows j and p */                                      \
        if (p != j)                                                            \
            for (int k = 0; k < n; ++k) {                                      \
                T t = A[j + (size_t)k * lda];                                  \
                A[j + (size_t)k * lda] = A[p + (size_t)k * lda];               \
                A[p + (size_t)k * lda] = t;                                    \
            }                                                                  \
        T piv = A[j + (size_t)j * lda];                                        \
        if (FABS(piv) == (T)0) {            /* R2 */                           \
            if (*info == 0) *info = j + 1;                                     \
            continue;                                                          \
        }                                                                      \
        /* a3: multipliers (R3) */                                             \
        if (FABS(piv) >= SFMIN) {                                              \
            T r = (T)1 / piv;                                                  \
            for (int i = j + 1; i < n; ++i) A[i + (size_t)j * lda] *= r;       \
        } else {                                                               \
            for (int i = j + 1; i < n; ++i) A[i + (size_t)j * lda] /= piv;     \
        }                                                                      \
        /* a4: rank-1 update, column k outer, row i inner (R4) */              \
        for (int k = j + 1; k < n; ++k) {                                      \
            T u = A[j + (size_t)k * lda];                                      \
            for (int i = j + 1; i < n; ++i)                                    \
                A[i + (size_t)k * lda] =                                       \
                    FMA(-A[i + (size_t)j * lda], u, A[i + (size_t)k * lda]);   \
        }                                                                      \
    }                                                                          \
}

DEFINE_REAL_GETRF(oracle_sgetrf, float, fmaf, fabsf, FLT_MIN)
DEFINE_REAL_GETRF(oracle_dgetrf, double, fma, fabs, DBL_MIN)

/* ------------------------------------------------------------------ */
/* real getrs (NoTrans): permute, forward (unit L), back (U)           */
/* ------------------------------------------------------------------ */
#define DEFINE_REAL_GETRS(NAME, T, FMA)                                        \
void NAME(int n, int nrhs, const T* A, int lda, const int* ipiv,               \
          T* B, int ldb)                                                       \
{                                                                              \
    for (int c = 0; c < nrhs; ++c) {                                           \
        T* b = B + (size_t)c * ldb;                                            \
        for (int k = 0; k < n; ++k) {       /* a8: transpositions in order */  \
            int p = ipiv[k] - 1;                                               \
            if (p != k) { T t = b[k]; b[k] = b[p]; b[p] = t; }                 \
        }                                                                      \
        for (int k = 0; k < n; ++k)         /* a9: L y = P b */                \
            for (int i = k + 1; i < n; ++i)                                    \
                b[i] = FMA(-A[i + (size_t)k * lda], b[k], b[i]);               \
        for (int k = n - 1; k >= 0; --k) {  /* a10: U x = y (R5) */            \
            b[k] = b[k] / A[k + (size_t)k * lda];                              \
            for (int i = 0; i < k; ++i)                                        \
                b[i] = FMA(-A[i + (size_t)k * lda], b[k], b[i]);               \
        }                                                                      \
    }                                                                          \
}

DEFINE_REAL_GETRS(oracle_sgetrs, float, fmaf)
DEFINE_REAL_GETRS(oracle_dgetrs, double, fma)

/* ------------------------------------------------------------------ */
/* real getrs (Trans): A = P^T L U, so A^T = U^T L^T P and the solve   */
/* is U^T w = b (forward, dividing by u_kk), L^T z = w (backward, unit */
/* diagonal), then x = P^T z: the transpositions in reverse order.     */
/* Both substitutions accumulate in substitution order, as for NoTrans. */
/* ------------------------------------------------------------------ */
#define DEFINE_REAL_GETRS_T(NAME, T, FMA)                                      \
void NAME(int n, int nrhs, const T* A, int lda, const int* ipiv,               \
          T* B, int ldb)                                                       \
{                                                                              \
    for (int c = 0; c < nrhs; ++c) {                                           \
        T* b = B + (size_t)c * ldb;                                            \
        for (int k = 0; k < n; ++k) {       /* U^T w = b: (U^T)_ik = u_ki */   \
            b[k] = b[k] / A[k + (size_t)k * lda];                              \
            for (int i = k + 1; i < n; ++i)                                    \
                b[i] = FMA(-A[k + (size_t)i * lda], b[k], b[i]);               \
        }                                                                      \
        for (int k = n - 1; k >= 0; --k)    /* L^T z = w: (L^T)_ik = l_ki */   \
            for (int i = 0; i < k; ++i)                                        \
                b[i] = FMA(-A[k + (size_t)i * lda], b[k], b[i]);               \
        for (int k = n - 1; k >= 0; --k) {  /* x = P^T z */                    \
            int p = ipiv[k] - 1;                                               \
            if (p != k) { T t = b[k]; b[k] = b[p]; b[p] = t; }                 \
        }                                                                      \
    }                                                                          \
}

DEFINE_REAL_GETRS_T(oracle_sgetrs_t, float, fmaf)
DEFINE_REAL_GETRS_T(oracle_dgetrs_t, double, fma)

/* ------------------------------------------------------------------ */
/* complex helpers (interleaved re, im), every operation rounded once  */
/* ------------------------------------------------------------------ */
#define DEFINE_COMPLEX_GETRF_GETRS(PFX, T, FMA, FABS, SFMIN)                   \
static T PFX##_cabs1(const T* z) { return FABS(z[0]) + FABS(z[1]); }           \
/* Smith: out = 1 / (c + d i) */                                               \
static void PFX##_recip(T c, T d, T* out)                                      \
{                                                                              \
    if (FABS(c) >= FABS(d)) {                                                  \
        T e = d / c; T f = c + d * e;                                          \
        out[0] = (T)1 / f; out[1] = -e / f;                                    \
    } else {                                                                   \
        T e = c / d; T f = d + c * e;                                          \
        out[0] = e / f; out[1] = -(T)1 / f;                                    \
    }                                                                          \
}                                                                              \
/* Smith: out = (a + b i) / (c + d i) */                                       \
static void PFX##_div(T a, T b, T c, T d, T* out)                              \
{                                                                              \
    if (FABS(c) >= FABS(d)) {                                                  \
        T e = d / c; T f = c + d * e;                                          \
        out[0] = (a + b * e) / f; out[1] = (b - a * e) / f;                    \
    } else {                                                                   \
        T e = c / d; T f = d + c * e;                                          \
        out[0] = (a * e + b) / f; out[1] = (b * e - a) / f;                    \
    }                                                                          \
}                                                                              \
/* l = a * r (R4) */                                                           \
static void PFX##_mul(const T* a, const T* r, T* out)                          \
{                                                                              \
    T t = a[1] * r[1];                                                         \
    T re = FMA(a[0], r[0], -t);                                                \
    T t2 = a[1] * r[0];                                                        \
    T im = FMA(a[0], r[1], t2);                                                \
    out[0] = re; out[1] = im;                                                  \
}                                                                              \
/* z -= x * y (R4) */                                                          \
static void PFX##_fms(T* z, const T* x, const T* y)                            \
{                                                                              \
    T re = FMA(-x[0], y[0], z[0]);                                             \
    re = FMA(x[1], y[1], re);                                                  \
    T im = FMA(-x[0], y[1], z[1]);                                             \
    im = FMA(-x[1], y[0], im);                                                 \
    z[0] = re; z[1] = im;                                                      \
}                                                                              \
void oracle_##PFX##getrf(int n, T* A, int lda, int* ipiv, int* info,           \
                         double* margin)                                       \
{                                                                              \
    /* element (i, k) lives at A + 2 * (i + k * lda) */                        \
    *info = 0;                                                                 \
    for (int j = 0; j < n; ++j) {                                              \
        int p = j;                                                             \
        T best = PFX##_cabs1(A + 2 * (j + (size_t)j * lda));                   \
        double runner = 0.0; int have_runner = 0;                              \
        for (int i = j + 1; i < n; ++i) {                                      \
            T m = PFX##_cabs1(A + 2 * (i + (size_t)j * lda));                  \
            if (better_d((double)m, (double)best)) {                           \
                runner = (double)best; have_runner = 1;                        \
                best = m; p = i;                                               \
            } else if (!have_runner || better_d((double)m, runner)) {          \
                runner = (double)m; have_runner = 1;                           \
            }                                                                  \
        }                                                                      \
        if (margin) margin[j] = step_margin((double)best, runner, have_runner);\
        ipiv[j] = p + 1;                                                       \
        if (p != j)                                                            \
            for (int k = 0; k < n; ++k)                                        \
                for (int h = 0; h < 2; ++h) {                                  \
                    T t = A[2 * (j + (size_t)k * lda) + h];                    \
                    A[2 * (j + (size_t)k * lda) + h] =                         \
                        A[2 * (p + (size_t)k * lda) + h];                      \
                    A[2 * (p + (size_t)k * lda) + h] = t;                      \
                }                                                              \
        T* piv = A + 2 * (j + (size_t)j * lda);                                \
        T pm = PFX##_cabs1(piv);                                               \
        if (pm == (T)0) {                                                      \
            if (*info == 0) *info = j + 1;                                     \
            continue;                                                          \
        }                                                                      \
        if (pm >= SFMIN) {                                                     \
            T r[2]; PFX##_recip(piv[0], piv[1], r);                            \
            for (int i = j + 1; i < n; ++i) {                                  \
                T* a = A + 2 * (i + (size_t)j * lda);                          \
                PFX##_mul(a, r, a);                                            \
            }                                                                  \
        } else {                                                               \
            for (int i = j + 1; i < n; ++i) {                                  \
                T* a = A + 2 * (i + (size_t)j * lda);                          \
                PFX##_div(a[0], a[1], piv[0], piv[1], a);                      \
            }                                                                  \
        }                                                                      \
        for (int k = j + 1; k < n; ++k) {                                      \
            const T* u = A + 2 * (j + (size_t)k * lda);                        \
            for (int i = j + 1; i < n; ++i)                                    \
                PFX##_fms(A + 2 * (i + (size_t)k * lda),                       \
                          A + 2 * (i + (size_t)j * lda), u);                   \
        }                                                                      \
    }                                                                          \
}                                                                              \
void oracle_##PFX##getrs(int n, int nrhs, const T* A, int lda,                 \
                         const int* ipiv, T* B, int ldb)                       \
{                                                                              \
    for (int c = 0; c < nrhs; ++c) {                                           \
        T* b = B + 2 * (size_t)c * ldb;                                        \
        for (int k = 0; k < n; ++k) {                                          \
            int p = ipiv[k] - 1;                                               \
            if (p != k)                                                        \
                for (int h = 0; h < 2; ++h) {                                  \
                    T t = b[2 * k + h]; b[2 * k + h] = b[2 * p + h];           \
                    b[2 * p + h] = t;                                          \
                }                                                              \
        }                                                                      \
        for (int k = 0; k < n; ++k)                                            \
            for (int i = k + 1; i < n; ++i)                                    \
                PFX##_fms(b + 2 * i, A + 2 * (i + (size_t)k * lda), b + 2 * k);\
        for (int k = n - 1; k >= 0; --k) {                                     \
            const T* u = A + 2 * (k + (size_t)k * lda);                        \
            PFX##_div(b[2 * k], b[2 * k + 1], u[0], u[1], b + 2 * k);          \
            for (int i = 0; i < k; ++i)                                        \
                PFX##_fms(b + 2 * i, A + 2 * (i + (size_t)k * lda), b + 2 * k);\
        }                                                                      \
    }                                                                          \
}                                                                              \
void oracle_##PFX##getrs_t(int n, int nrhs, const T* A, int lda,               \
                           const int* ipiv, T* B, int ldb, int conj)           \
{                                                                              \
    const T sg = conj ? (T)-1 : (T)1;   /* 'C' uses conj(u_ki), conj(l_ki) */  \
    for (int c = 0; c < nrhs; ++c) {                                           \
        T* b = B + 2 * (size_t)c * ldb;                                        \
        for (int k = 0; k < n; ++k) {                                          \
            const T* u = A + 2 * (k + (size_t)k * lda);                        \
            PFX##_div(b[2 * k], b[2 * k + 1], u[0], sg * u[1], b + 2 * k);     \
            for (int i = k + 1; i < n; ++i) {                                  \
                const T* e = A + 2 * (k + (size_t)i * lda);                    \
                T x[2] = {e[0], sg * e[1]};                                    \
                PFX##_fms(b + 2 * i, x, b + 2 * k);                            \
            }                                                                  \
        }                                                                      \
        for (int k = n - 1; k >= 0; --k)                                       \
            for (int i = 0; i < k; ++i) {                                      \
                const T* e = A + 2 * (k + (size_t)i * lda);                    \
                T x[2] = {e[0], sg * e[1]};                                    \
                PFX##_fms(b + 2 * i, x, b + 2 * k);                            \
            }                                                                  \
        for (int k = n - 1; k >= 0; --k) {                                     \
            int p = ipiv[k] - 1;                                               \
            if (p != k)                                                        \
                for (int h = 0; h < 2; ++h) {                                  \
                    T t = b[2 * k + h]; b[2 * k + h] = b[2 * p + h];           \
                    b[2 * p + h] = t;                                          \
                }                                                              \
        }                                                                      \
    }                                                                          \
}

DEFINE_COMPLEX_GETRF_GETRS(c, float, fmaf, fabsf, FLT_MIN)
DEFINE_COMPLEX_GETRF_GETRS(z, double, fma, fabs, DBL_MIN)

/* ------------------------------------------------------------------ */
/* batch drivers: one matrix per task, tasks spread over host threads  */
/* ------------------------------------------------------------------ */
static size_t elem_size(int t)
{
    switch (t) {
    case OR_R32: return 4;
    case OR_R64: return 8;
    case OR_C64: return 8;
    case OR_C128: return 16;
    default: return 0;
    }
}

typedef struct {
    int op;            /* 0 getrf, 1 getrs, 2 gesv */
    int trans;         /* getrs only: 0 A, 1 A^T, 2 A^H */
    int t, n, nrhs;
    char* A; int lda; long long sA;
    int* ipiv; long long sP;
    int* info;
    double* margin;    /* n per matrix, may be NULL */
    char* B; int ldb; long long sB;
    int begin, end;
} job_t;

static void one_getrf(const job_t* J, int b)
{
    size_t es = elem_size(J->t);
    void* A = J->A + (size_t)b * J->sA * es;
    int* ip = J->ipiv + (size_t)b * J->sP;
    double* mg = J->margin ? J->margin + (size_t)b * J->n : NULL;
    int* inf = J->info + b;
    switch (J->t) {
    case OR_R32: oracle_sgetrf(J->n, (float*)A, J->lda, ip, inf, mg); break;
    case OR_R64: oracle_dgetrf(J->n, (double*)A, J->lda, ip, inf, mg); break;
    case OR_C64: oracle_cgetrf(J->n, (float*)A, J->lda, ip, inf, mg); break;
    case OR_C128: oracle_zgetrf(J->n, (double*)A, J->lda, ip, inf, mg); break;
    }
}

static void one_getrs(const job_t* J, int b)
{
    size_t es = elem_size(J->t);
    const void* A = J->A + (size_t)b * J->sA * es;
    const int* ip = J->ipiv + (size_t)b * J->sP;
    void* B = J->B + (size_t)b * J->sB * es;
    if (J->trans) {
        switch (J->t) {
        case OR_R32: oracle_sgetrs_t(J->n, J->nrhs, (const float*)A, J->lda, ip, (float*)B, J->ldb); break;
        case OR_R64: oracle_dgetrs_t(J->n, J->nrhs, (const double*)A, J->lda, ip, (double*)B, J->ldb); break;
        case OR_C64: oracle_cgetrs_t(J->n, J->nrhs, (const float*)A, J->lda, ip, (float*)B, J->ldb,
                                     J->trans == 2); break;
        case OR_C128: oracle_zgetrs_t(J->n, J->nrhs, (const double*)A, J->lda, ip, (double*)B, J->ldb,
                                      J->trans == 2); break;
        }
        return;
    }
    switch (J->t) {
    case OR_R32: oracle_sgetrs(J->n, J->nrhs, (const float*)A, J->lda, ip, (float*)B, J->ldb); break;
    case OR_R64: oracle_dgetrs(J->n, J->nrhs, (const double*)A, J->lda, ip, (double*)B, J->ldb); break;
    case OR_C64: oracle_cgetrs(J->n, J->nrhs, (const float*)A, J->lda, ip, (float*)B, J->ldb); break;
    case OR_C128: oracle_zgetrs(J->n, J->nrhs, (const double*)A, J->lda, ip, (double*)B, J->ldb); break;
    }
}

static void* worker(void* arg)
{
    job_t* J = (job_t*)arg;
    for (int b = J->begin; b < J->end; ++b) {
        if (J->op == 0 || J->op == 2) one_getrf(J, b);
        if (J->op == 1 || (J->op == 2 && J->info[b] == 0)) one_getrs(J, b);  /* R6 */
    }
    return NULL;
}

static int run_batch(job_t proto, int batch, int nthreads)
{
    if (batch <= 0) return 0;
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > batch) nthreads = batch;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    job_t jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].begin = (int)((long long)batch * t / nthreads);
        jobs[t].end = (int)((long long)batch * (t + 1) / nthreads);
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[t], NULL, worker, &jobs[t]) == 0) started = t;
        else break;
    worker(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    for (int t = started + 1; t < nthreads; ++t) worker(&jobs[t]);  /* if a create failed */
    return nthreads;
}

/* Returns the number of host threads used. */
int oracle_getrf_batch(int t, int n, void* A, int lda, long long strideA,
                       int* ipiv, long long strideP, int* info, double* margin,
                       int batch, int nthreads)
{
    job_t J; memset(&J, 0, sizeof J);
    J.op = 0; J.t = t; J.n = n; J.A = (char*)A; J.lda = lda; J.sA = strideA;
    J.ipiv = ipiv; J.sP = strideP; J.info = info; J.margin = margin;
    return run_batch(J, batch, nthreads);
}

int oracle_getrs_batch(int t, int n, int nrhs, const void* A, int lda,
                       long long strideA, const int* ipiv, long long strideP,
                       void* B, int ldb, long long strideB, int batch, int nthreads)
{
    job_t J; memset(&J, 0, sizeof J);
    J.op = 1; J.t = t; J.n = n; J.nrhs = nrhs; J.A = (char*)A; J.lda = lda;
    J.sA = strideA; J.ipiv = (int*)ipiv; J.sP = strideP; J.B = (char*)B;
    J.ldb = ldb; J.sB = strideB;
    return run_batch(J, batch, nthreads);
}

/* getri, out of place: C = A^{-1} from the factors and ipiv, as the
   solution of A C = I (C set to the identity, then the NoTrans solve,
   column by column).  R8 of the header. */
int oracle_getri_batch(int t, int n, const void* A, int lda, long long strideA,
                       const int* ipiv, long long strideP, void* C, int ldc,
                       long long strideC, int batch, int nthreads)
{
    size_t es = elem_size(t);
    for (int b = 0; b < batch; ++b) {
        char* c = (char*)C + (size_t)b * strideC * es;
        for (int j = 0; j < n; ++j) {
            memset(c + (size_t)j * ldc * es, 0, (size_t)n * es);
            if (t == OR_R32) ((float*)c)[j + (size_t)j * ldc] = 1.0f;
            else if (t == OR_R64) ((double*)c)[j + (size_t)j * ldc] = 1.0;
            else if (t == OR_C64) ((float*)c)[2 * (j + (size_t)j * ldc)] = 1.0f;
            else ((double*)c)[2 * (j + (size_t)j * ldc)] = 1.0;
        }
    }
    return oracle_getrs_batch(t, n, n, A, lda, strideA, ipiv, strideP, C, ldc, strideC,
                              batch, nthreads);
}

/* trans: 0 solves A X = B, 1 solves A^T X = B, 2 solves A^H X = B */
int oracle_getrs_trans_batch(int t, int trans, int n, int nrhs, const void* A, int lda,
                             long long strideA, const int* ipiv, long long strideP,
                             void* B, int ldb, long long strideB, int batch, int nthreads)
{
    job_t J; memset(&J, 0, sizeof J);
    J.op = 1; J.trans = trans; J.t = t; J.n = n; J.nrhs = nrhs; J.A = (char*)A; J.lda = lda;
    J.sA = strideA; J.ipiv = (int*)ipiv; J.sP = strideP; J.B = (char*)B;
    J.ldb = ldb; J.sB = strideB;
    return run_batch(J, batch, nthreads);
}

int oracle_gesv_batch(int t, int n, int nrhs, void* A, int lda, long long strideA,
                      int* ipiv, long long strideP, void* B, int ldb,
                      long long strideB, int* info, double* margin, int batch,
                      int nthreads)
{
    job_t J; memset(&J, 0, sizeof J);
    J.op = 2; J.t = t; J.n = n; J.nrhs = nrhs; J.A = (char*)A; J.lda = lda;
    J.sA = strideA; J.ipiv = ipiv; J.sP = strideP; J.info = info;
    J.margin = margin; J.B = (char*)B; J.ldb = ldb; J.sB = strideB;
    return run_batch(J, batch, nthreads);
}
