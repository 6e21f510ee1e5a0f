/*
 * chol_oracle.c -- plain, slow CPU oracle for batched Cholesky (potrf), the
 * Cholesky solve (potrs) and their composition (posv).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header or constant with the HIP path.
 *
 * What it follows (BatchLAS performance notes):
 *   - "Blackwell" page, LPanel paragraph: the left-looking panel update
 *     accumulates every entry over k in ascending order;
 *   - "Blackwell" page, POD complex / TRSM-division paragraph: a Cholesky
 *     diagonal is real and handled with real-component helpers, reference
 *     potf2 multiplies by a reciprocal of the diagonal while reference trsm
 *     divides;
 *   - "trsm" page, posv passages: posv is potrf followed by two triangular
 *     solves (lower, then its conjugate transpose);
 *   - "Blackwell" page, posv note on the fused solve arm solving on both
 *     triangles: uplo 'L' (A = L L^H) and 'U' (A = U^H U) are both served.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   C1  Column j: d = re(a_jj) minus |l_jk|^2 for k = 0 .. j-1 in ascending
 *       k, each term as fused multiply-adds (complex: -re*re then -im*im);
 *       the imaginary part of a diagonal entry is never read.
 *   C2  d > 0 (not NaN): l_jj = sqrt(d) correctly rounded, r = 1/l_jj
 *       rounded once, and for i > j: s = a_ij minus l_ik conj(l_jk) over k
 *       ascending, one fused multiply-add per real term, then l_ij = s * r
 *       (complex: each part times r).  Complex s -= x conj(y) is re:
 *       fma(-xr, yr), then fma(-xi, yi); im: fma(xr, yi), then fma(-xi, yr).
 *   C3  d <= 0 or NaN (LAPACK potf2's test): a_jj = d (imaginary part 0),
 *       info = j + 1, and the factorisation stops.  Only columns 0 .. j-1
 *       and the entry a_jj are defined afterwards.
 *   C4  Only the named triangle is read or written.  'U' computes exactly
 *       the conjugate transpose of the 'L' computation (conjugation is
 *       exact, so u_ji = conj(l_ij) bit for bit); a stored diagonal entry
 *       of either triangle is (l_jj, +0).
 *   C5  potrs: L y = b with y_k = b_k / l_kk (true division, complex by
 *       parts) then b_i -= l_ik y_k for i > k, k ascending; then L^H x = y
 *       with x_k = y_k / l_kk then y_i -= conj(l_ki) x_k for i < k, k
 *       descending.  Complex z -= x*y: re fma(-xr, yr), fma(xi, yi);
 *       im fma(-xr, yi), fma(-xi, yr); z -= conj(x)*y: re fma(-xr, yr),
 *       fma(-xi, yi); im fma(-xr, yi), fma(xi, yr).
 *   C6  posv leaves B untouched for a matrix whose info > 0.
 *
 * Arithmetic is in the working precision of the data type.  Build with
 * -ffp-contract=off so that no multiply-add is fused behind our back.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { CH_R32 = 0, CH_R64 = 1, CH_C64 = 2, CH_C128 = 3 };

/* ------------------------------------------------------------------ */
/* real potrf / potrs                                                  */
/* element (i, k) of the working lower factor: for uplo 'L' it is      */
/* A[i + k*lda]; for 'U' it is A[k + i*lda] (real: no conjugation)     */
/* ------------------------------------------------------------------ */
#define DEFINE_REAL_CHOL(PFX, T, FMA, SQRT)                                    \
static T* PFX##_at(T* A, int lda, int up, int i, int k)                        \
{                                                                              \
    return up ? &A[k + (size_t)i * lda] : &A[i + (size_t)k * lda];             \
}                                                                              \
void oracle_##PFX##potrf(int up, int n, T* A, int lda, int* info)              \
{                                                                              \
    *info = 0;                                                                 \
    for (int j = 0; j < n; ++j) {                                              \
        T d = *PFX##_at(A, lda, up, j, j);                   /* C1 */          \
        for (int k = 0; k < j; ++k) {                                          \
            T l = *PFX##_at(A, lda, up, j, k);                                 \
            d = FMA(-l, l, d);                                                 \
        }                                                                      \
        if (!(d > (T)0)) {                                   /* C3 */          \
            *PFX##_at(A, lda, up, j, j) = d;                                   \
            *info = j + 1;                                                     \
            return;                                                            \
        }                                                                      \
        T ljj = SQRT(d);                                     /* C2 */          \
        *PFX##_at(A, lda, up, j, j) = ljj;                                     \
        T r = (T)1 / ljj;                                                      \
        for (int i = j + 1; i < n; ++i) {                                      \
            T s = *PFX##_at(A, lda, up, i, j);                                 \
            for (int k = 0; k < j; ++k)                                        \
                s = FMA(-*PFX##_at(A, lda, up, i, k),                          \
                        *PFX##_at(A, lda, up, j, k), s);                       \
            *PFX##_at(A, lda, up, i, j) = s * r;                               \
        }                                                                      \
    }                                                                          \
}                                                                              \
void oracle_##PFX##potrs(int up, int n, int nrhs, T* A, int lda,              \
                         T* B, int ldb)                                        \
{                                                                              \
    for (int c = 0; c < nrhs; ++c) {                                           \
        T* b = B + (size_t)c * ldb;                                            \
        for (int k = 0; k < n; ++k) {                        /* C5 forward */  \
            b[k] = b[k] / *PFX##_at(A, lda, up, k, k);                         \
            for (int i = k + 1; i < n; ++i)                                    \
                b[i] = FMA(-*PFX##_at(A, lda, up, i, k), b[k], b[i]);          \
        }                                                                      \
        for (int k = n - 1; k >= 0; --k) {                   /* C5 back */     \
            b[k] = b[k] / *PFX##_at(A, lda, up, k, k);                         \
            for (int i = 0; i < k; ++i)                                        \
                b[i] = FMA(-*PFX##_at(A, lda, up, k, i), b[k], b[i]);          \
        }                                                                      \
    }                                                                          \
}

DEFINE_REAL_CHOL(s, float, fmaf, sqrtf)
DEFINE_REAL_CHOL(d, double, fma, sqrt)

/* ------------------------------------------------------------------ */
/* complex potrf / potrs: T is the real part type, an element is T[2]  */
/* for 'U' the working element (i, k) is conj(A[k + i*lda])            */
/* ------------------------------------------------------------------ */
#define DEFINE_COMPLEX_CHOL(PFX, T, FMA, SQRT)                                 \
static void PFX##_get(const T* A, int lda, int up, int i, int k, T* out)       \
{                                                                              \
    const T* p = up ? &A[2 * (k + (size_t)i * lda)] : &A[2 * (i + (size_t)k * lda)]; \
    out[0] = p[0];                                                             \
    out[1] = up ? -p[1] : p[1];                                                \
}                                                                              \
static void PFX##_put(T* A, int lda, int up, int i, int k, const T* v)         \
{                                                                              \
    T* p = up ? &A[2 * (k + (size_t)i * lda)] : &A[2 * (i + (size_t)k * lda)]; \
    p[0] = v[0];                                                               \
    p[1] = (up && i != k) ? -v[1] : v[1];   /* a diagonal keeps +0 (C4) */     \
}                                                                              \
/* z -= x * conj(y) (C2) */                                                    \
static void PFX##_fms_conj(T* z, const T* x, const T* y)                       \
{                                                                              \
    T re = FMA(-x[0], y[0], z[0]);                                             \
    re = FMA(-x[1], y[1], re);                                                 \
    T im = FMA(x[0], y[1], z[1]);                                              \
    im = FMA(-x[1], y[0], im);                                                 \
    z[0] = re; z[1] = im;                                                      \
}                                                                              \
/* z -= x * y (C5) */                                                          \
static void PFX##_fms(T* z, const T* x, const T* y)                            \
{                                                                              \
    T re = FMA(-x[0], y[0], z[0]);                                             \
    re = FMA(x[1], y[1], re);                                                  \
    T im = FMA(-x[0], y[1], z[1]);                                             \
    im = FMA(-x[1], y[0], im);                                                 \
    z[0] = re; z[1] = im;                                                      \
}                                                                              \
/* z -= conj(x) * y (C5) */                                                    \
static void PFX##_fms_cx(T* z, const T* x, const T* y)                         \
{                                                                              \
    T re = FMA(-x[0], y[0], z[0]);                                             \
    re = FMA(-x[1], y[1], re);                                                 \
    T im = FMA(-x[0], y[1], z[1]);                                             \
    im = FMA(x[1], y[0], im);                                                  \
    z[0] = re; z[1] = im;                                                      \
}                                                                              \
void oracle_##PFX##potrf(int up, int n, T* A, int lda, int* info)              \
{                                                                              \
    *info = 0;                                                                 \
    for (int j = 0; j < n; ++j) {                                              \
        T djj[2], l[2];                                                        \
        PFX##_get(A, lda, up, j, j, djj);                                      \
        T d = djj[0];                                        /* C1 */          \
        for (int k = 0; k < j; ++k) {                                          \
            PFX##_get(A, lda, up, j, k, l);                                    \
            d = FMA(-l[0], l[0], d);                                           \
            d = FMA(-l[1], l[1], d);                                           \
        }                                                                      \
        if (!(d > (T)0)) {                                   /* C3 */          \
            T v[2] = {d, (T)0};                                                \
            PFX##_put(A, lda, up, j, j, v);                                    \
            *info = j + 1;                                                     \
            return;                                                            \
        }                                                                      \
        T ljj = SQRT(d);                                     /* C2 */          \
        T v[2] = {ljj, (T)0};                                                  \
        PFX##_put(A, lda, up, j, j, v);                                        \
        T r = (T)1 / ljj;                                                      \
        for (int i = j + 1; i < n; ++i) {                                      \
            T s[2], x[2], y[2];                                                \
            PFX##_get(A, lda, up, i, j, s);                                    \
            for (int k = 0; k < j; ++k) {                                      \
                PFX##_get(A, lda, up, i, k, x);                                \
                PFX##_get(A, lda, up, j, k, y);                                \
                PFX##_fms_conj(s, x, y);                                       \
            }                                                                  \
            s[0] = s[0] * r;                                                   \
            s[1] = s[1] * r;                                                   \
            PFX##_put(A, lda, up, i, j, s);                                    \
        }                                                                      \
    }                                                                          \
}                                                                              \
void oracle_##PFX##potrs(int up, int n, int nrhs, T* A, int lda,              \
                         T* B, int ldb)                                        \
{                                                                              \
    for (int c = 0; c < nrhs; ++c) {                                           \
        T* b = B + 2 * (size_t)c * ldb;                                        \
        T l[2], dk[2];                                                         \
        for (int k = 0; k < n; ++k) {                        /* C5 forward */  \
            PFX##_get(A, lda, up, k, k, dk);                                   \
            b[2 * k] = b[2 * k] / dk[0];                                       \
            b[2 * k + 1] = b[2 * k + 1] / dk[0];                               \
            for (int i = k + 1; i < n; ++i) {                                  \
                PFX##_get(A, lda, up, i, k, l);                                \
                PFX##_fms(&b[2 * i], l, &b[2 * k]);                            \
            }                                                                  \
        }                                                                      \
        for (int k = n - 1; k >= 0; --k) {                   /* C5 back */     \
            PFX##_get(A, lda, up, k, k, dk);                                   \
            b[2 * k] = b[2 * k] / dk[0];                                       \
            b[2 * k + 1] = b[2 * k + 1] / dk[0];                               \
            for (int i = 0; i < k; ++i) {                                      \
                PFX##_get(A, lda, up, k, i, l);                                \
                PFX##_fms_cx(&b[2 * i], l, &b[2 * k]);                         \
            }                                                                  \
        }                                                                      \
    }                                                                          \
}

DEFINE_COMPLEX_CHOL(c, float, fmaf, sqrtf)
DEFINE_COMPLEX_CHOL(z, double, fma, sqrt)

/* ------------------------------------------------------------------ */
/* batch drivers: one matrix per task, tasks spread over host threads  */
/* ------------------------------------------------------------------ */
typedef struct {
    int op;                 /* 0 potrf, 1 potrs, 2 posv */
    int t, up, n, nrhs;
    char* A; int lda; long long sA;
    int* info;
    char* B; int ldb; long long sB;
    int begin, end;
} chol_job_t;

static size_t ch_elem_size(int t)
{
    return t == CH_R32 ? 4 : (t == CH_R64 || t == CH_C64) ? 8 : 16;
}

static void ch_one(const chol_job_t* J, int b)
{
    size_t es = ch_elem_size(J->t);
    void* A = J->A + (size_t)b * J->sA * es;
    if (J->op == 0 || J->op == 2) {
        int* inf = J->info + b;
        switch (J->t) {
        case CH_R32: oracle_spotrf(J->up, J->n, (float*)A, J->lda, inf); break;
        case CH_R64: oracle_dpotrf(J->up, J->n, (double*)A, J->lda, inf); break;
        case CH_C64: oracle_cpotrf(J->up, J->n, (float*)A, J->lda, inf); break;
        case CH_C128: oracle_zpotrf(J->up, J->n, (double*)A, J->lda, inf); break;
        }
        if (J->op == 2 && *inf != 0) return;                 /* C6 */
    }
    if (J->op == 1 || J->op == 2) {
        void* B = J->B + (size_t)b * J->sB * es;
        switch (J->t) {
        case CH_R32: oracle_spotrs(J->up, J->n, J->nrhs, (float*)A, J->lda, (float*)B, J->ldb); break;
        case CH_R64: oracle_dpotrs(J->up, J->n, J->nrhs, (double*)A, J->lda, (double*)B, J->ldb); break;
        case CH_C64: oracle_cpotrs(J->up, J->n, J->nrhs, (float*)A, J->lda, (float*)B, J->ldb); break;
        case CH_C128: oracle_zpotrs(J->up, J->n, J->nrhs, (double*)A, J->lda, (double*)B, J->ldb); break;
        }
    }
}

static void* ch_worker(void* arg)
{
    chol_job_t* J = (chol_job_t*)arg;
    for (int b = J->begin; b < J->end; ++b) ch_one(J, b);
    return NULL;
}

static int ch_run(chol_job_t proto, int batch, int nthreads)
{
    if (batch <= 0) return 0;
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > batch) nthreads = batch;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    chol_job_t jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].begin = (int)((long long)batch * t / nthreads);
        jobs[t].end = (int)((long long)batch * (t + 1) / nthreads);
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[t], NULL, ch_worker, &jobs[t]) == 0) started = t;
        else break;
    ch_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    for (int t = started + 1; t < nthreads; ++t) ch_worker(&jobs[t]);  /* if a create failed */
    return nthreads;
}

/* op: 0 potrf, 1 potrs, 2 posv; up: 0 lower ('L'), 1 upper ('U').
   Returns the number of host threads used. */
int oracle_chol_batch(int op, int t, int up, int n, int nrhs, void* A, int lda,
                      long long strideA, int* info, void* B, int ldb, long long strideB,
                      int batch, int nthreads)
{
    chol_job_t J;
    memset(&J, 0, sizeof J);
    J.op = op; J.t = t; J.up = up; J.n = n; J.nrhs = nrhs;
    J.A = (char*)A; J.lda = lda; J.sA = strideA; J.info = info;
    J.B = (char*)B; J.ldb = ldb; J.sB = strideB;
    return ch_run(J, batch, nthreads);
}
