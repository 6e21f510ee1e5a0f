/*
 * batchlu.h -- C ABI of the batched LU library for AMD Instinct MI355X (gfx950).
 *
 * Operations (BatchLAS performance notes, "LU" page, family table at the top
 * of the page): getrf factors each matrix of a homogeneous batch with partial
 * pivoting, P*A = L*U; getrs solves A*X = B from those factors; gesv is the
 * composition of the two.
 *
 * Common conventions (same page: the tiny-tier and register-panel paragraphs
 * fix ipiv and info; the common can_run term fixes square A and B.rows == n;
 * the Blackwell page's trsm paragraph requires padded leading dimensions and
 * batch strides to work):
 *   - Every matrix is column-major.  Element (i, j) of matrix b of A is at
 *     A + b*strideA + i + j*lda, counted in elements of the data type.
 *     Complex types are interleaved (re, im) pairs, like std::complex.
 *   - All pointers are DEVICE pointers and stay owned by the caller.  The
 *     library allocates nothing per call and frees nothing.
 *   - Every call is asynchronous on `stream` (0 = the null stream).  ipiv,
 *     info, the factors and X are valid once the stream has reached the
 *     point after the call.
 *   - ipiv is int32, 1-based and global: ipiv[b*strideP + j] = p + 1 means
 *     rows j and p were exchanged at step j (in that order, j = 0 .. n-1).
 *   - info[b] = 0 on success, or j + 1 for the first step j whose pivot is
 *     exactly zero.  The factorisation still completes (the zero column is
 *     left unscaled).  A numerically singular matrix is not an error.
 *   - Pivot choice: the largest |a| (real) or |re| + |im| (complex) in the
 *     column; ties go to the lowest row; a NaN ranks above every number and
 *     the first NaN wins.
 *   - Arguments are checked on the host before anything is launched.  A bad
 *     argument returns -k, where k is its 1-based position in the signature.
 *     n == 0, nrhs == 0 or batch == 0 succeed without launching anything.
 *   - A shape no tier can run is refused with BATCHLU_ERR_CAPACITY, never
 *     truncated (BatchLAS "trsm" page: the over-capacity defect).
 */
#ifndef BATCHLU_H
#define BATCHLU_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BATCHLU_R32 = 0,   /* float                    */
    BATCHLU_R64 = 1,   /* double                   */
    BATCHLU_C64 = 2,   /* complex float  (re, im)  */
    BATCHLU_C128 = 3   /* complex double (re, im)  */
} batchlu_dtype;

/* status codes (negative values -1 .. -20 name an invalid argument) */
#define BATCHLU_OK 0
#define BATCHLU_ERR_UNSUPPORTED (-100) /* e.g. getrs or getri with n > 4096    */
#define BATCHLU_ERR_CAPACITY (-101)    /* no tier can run this shape           */
#define BATCHLU_ERR_LAUNCH (-102)      /* a kernel launch failed (HIP error)   */

/* tiers (see batchlu_select_tier) */
#define BATCHLU_TIER_AUTO 0
#define BATCHLU_TIER_TINY 1    /* several matrices per wavefront, rows in VGPRs */
#define BATCHLU_TIER_CTA 2     /* one work-group per matrix, rows in VGPRs       */
#define BATCHLU_TIER_BLOCKED 3 /* nb = 32 right-looking: panel, laswp, trsm, gemm */
#define BATCHLU_TIER_CTA_LDS 4 /* one work-group per matrix, [A | B] staged in LDS */

/*
 * batchlu_getrf -- LU with partial pivoting of `batch` n x n matrices, in place.
 *   1 t        data type
 *   2 n        order, 0 <= n <= 4096 (larger n returns BATCHLU_ERR_CAPACITY)
 *   3 A        device, in: the matrices; out: L (unit diagonal not stored)
 *              below the diagonal and U on and above it, rows in pivoted order
 *   4 lda      >= max(1, n)
 *   5 strideA  elements between matrices, >= lda*n when batch > 1
 *   6 ipiv     device int32, out: strideP entries per matrix, first n written
 *   7 strideP  >= n when batch > 1
 *   8 info     device int32[batch], out
 *   9 batch    >= 0
 *  10 stream
 * Follows: BatchLAS "LU" page, getrf rows of the family table and the tiny,
 * cta and blocked paragraphs.
 */
int batchlu_getrf(batchlu_dtype t, int n, void* A, int lda, long long strideA,
                  int* ipiv, long long strideP, int* info, int batch,
                  hipStream_t stream);

/*
 * batchlu_getrs -- solve op(A) X = B with the factors and ipiv of batchlu_getrf.
 *   1 t, 2 trans: 'N' solves A X = B, 'T' A^T X = B, 'C' A^H X = B (A^T
 *     for real types),
 *   3 n (<= 4096, else BATCHLU_ERR_UNSUPPORTED: one launch solves n <= 1024,
 *     larger n runs block row by block row), 4 nrhs >= 0, 5 A (device, read only), 6 lda, 7 strideA,
 *   8 ipiv (device, read only; an entry outside 1..n is read as "no
 *     interchange" so that a corrupt list cannot address rows outside B),
 *   9 strideP,
 *  10 B (device, in: right-hand sides, out: X), 11 ldb >= max(1, n),
 *  12 strideB >= ldb*nrhs when batch > 1, 13 batch, 14 stream.
 * The factors of a matrix whose info was > 0 give inf/NaN, as in LAPACK.
 * Follows: BatchLAS "LU" page, getrs paragraphs (permutation, then forward
 * substitution with unit-lower L, then back substitution with U; the fused
 * kernels exist for NoTrans and Trans).  For op(A) = A^T = U^T L^T P the
 * order is forward with U^T (division by u_kk), back with unit L^T, then
 * the interchanges undone in reverse; A^H uses the conjugated factors.
 */
int batchlu_getrs(batchlu_dtype t, char trans, int n, int nrhs, const void* A,
                  int lda, long long strideA, const int* ipiv,
                  long long strideP, void* B, int ldb, long long strideB,
                  int batch, hipStream_t stream);

/*
 * batchlu_gesv -- factor and solve: getrf on A, then getrs on B.
 *   1 t, 2 n (<= 4096, else BATCHLU_ERR_CAPACITY), 3 nrhs, 4 A, 5 lda, 6 strideA, 7 ipiv, 8 strideP,
 *   9 B, 10 ldb, 11 strideB, 12 info, 13 batch, 14 stream.
 * A matrix with info[b] > 0 keeps its B unchanged (LAPACK gesv behaviour).
 * Follows: BatchLAS "LU" page, gesv rows of the family table (a fused
 * factor-and-solve for small n; getrf then getrs otherwise).
 */
int batchlu_gesv(batchlu_dtype t, int n, int nrhs, void* A, int lda,
                 long long strideA, int* ipiv, long long strideP, void* B,
                 int ldb, long long strideB, int* info, int batch,
                 hipStream_t stream);

/*
 * batchlu_getri -- C = A^{-1} from the factors and ipiv of batchlu_getrf,
 * out of place.
 *   1 t, 2 n (0 <= n <= 4096; larger n returns BATCHLU_ERR_UNSUPPORTED),
 *   3 A (device, read only: the factors), 4 lda >= max(1, n),
 *   5 strideA >= lda*n when batch > 1,
 *   6 ipiv (device, read only; an entry outside 1..n is read as "no
 *     interchange"), 7 strideP >= n when batch > 1,
 *   8 C (device, out: the n x n inverses; its bytes must not overlap A's,
 *     else -8), 9 ldc >= max(1, n), 10 strideC >= ldc*n when batch > 1,
 *  11 batch, 12 stream.
 * Rows n..ldc-1 of C are not written.  A matrix whose info was > 0 gets
 * inf/NaN entries (LAPACK returns info there and leaves the inverse
 * undefined).  Follows: BatchLAS "LU" page, getri row of the family table
 * and the section on the shared interchange kernels (the pivoting is undone
 * inside the solve, with no separate permutation pass): computed as the
 * NoTrans solve of A C = I, whose right-hand sides are formed in registers
 * and never stored (n <= 1024), or, for larger n, C set to the identity and
 * then solved in place block row by block row.
 */
int batchlu_getri(batchlu_dtype t, int n, const void* A, int lda,
                  long long strideA, const int* ipiv, long long strideP,
                  void* C, int ldc, long long strideC, int batch,
                  hipStream_t stream);

/*
 * batchlu_getrf_rect -- LU with partial pivoting of `batch` m x n matrices
 * (LAPACK getrf on a rectangular A), in place: min(m, n) steps, each
 * searching all m rows of its column, swapping whole rows and updating every
 * column to its right.
 *   1 t, 2 m >= 0, 3 n >= 0, 4 A (device), 5 lda >= max(1, m),
 *   6 strideA >= lda*n when batch > 1, 7 ipiv (device int32, min(m, n)
 *   1-based entries per matrix), 8 strideP >= min(m, n) when batch > 1,
 *   9 info (device int32[batch]: 0, or the first step whose pivot is exactly
 *   zero, 1-based), 10 batch, 11 stream.
 * m == n runs batchlu_getrf.  Otherwise m <= 1024 for float (512 for double
 * and complex float, 256 for complex double) and n <= 1024, else
 * BATCHLU_ERR_CAPACITY.  Pivot, tie, NaN, zero-pivot and
 * rounding conventions are those of batchlu_getrf.  m == 0, n == 0 or
 * batch == 0 launch nothing.  Follows: BatchLAS "LU" page, family table (a
 * non-square A is served there only by the vendor's LAPACK-style getrf).
 */
int batchlu_getrf_rect(batchlu_dtype t, int m, int n, void* A, int lda,
                       long long strideA, int* ipiv, long long strideP,
                       int* info, int batch, hipStream_t stream);

/*
 * batchlu_getrf_vbatched -- LU with partial pivoting of a batch whose
 * matrices differ in size: matrix b is m[b] x n[b] at A[b] with leading
 * dimension lda[b] and pivots ipiv[b] (min(m[b], n[b]) entries).
 *   1 t, 2 m, 3 n, 5 lda (device int32[batch] each), 4 A (device array of
 *   batch device pointers), 6 ipiv (device array of batch device int32
 *   pointers), 7 info (device int32[batch], out), 8 max_m, 9 max_n (upper
 *   bounds of m[b] and n[b]: max_m within the rows batchlu_getrf_rect
 *   takes for the type, max_n <= 1024, else BATCHLU_ERR_CAPACITY), 10 batch, 11 stream.
 * A matrix whose sizes are negative, above max_m / max_n, or whose
 * lda[b] < max(1, m[b]), is not touched and gets info[b] = -1.  One launch
 * for the whole batch (one work-group per matrix).  Follows: BatchLAS "LU"
 * page, family table (a heterogeneous A has no route there).
 */
int batchlu_getrf_vbatched(batchlu_dtype t, const int* m, const int* n,
                           void* const* A, const int* lda, int* const* ipiv,
                           int* info, int max_m, int max_n, int batch,
                           hipStream_t stream);

/*
 * batchlu_getrs_vbatched -- solve A_b X_b = B_b (NoTrans) for a square
 * variable-size batch with the factors and pivots of batchlu_getrf_vbatched.
 *   1 t, 2 n, 3 nrhs, 5 lda, 8 ldb (device int32[batch] each), 4 A, 7 B
 *   (device arrays of batch device pointers; B[b] is n[b] x nrhs[b], in:
 *   right-hand sides, out: X), 6 ipiv (device array of pointers),
 *   9 max_n (upper bound of n[b], <= 1024), 10 batch, 11 stream.
 * Matrices with n[b] <= 0, nrhs[b] <= 0, n[b] above max_n rounded up to 64,
 * or lda[b] / ldb[b] < n[b] are skipped.  Order of operations as
 * batchlu_getrs.
 */
int batchlu_getrs_vbatched(batchlu_dtype t, const int* n, const int* nrhs,
                           void* const* A, const int* lda, int* const* ipiv,
                           void* const* B, const int* ldb, int max_n,
                           int batch, hipStream_t stream);

/*
 * batchlu_gesv_vbatched -- batchlu_getrf_vbatched (square, m = n), then
 * batchlu_getrs_vbatched on the matrices whose info is 0 (the others keep
 * their B).  Arguments as those two; 9 info (device int32[batch], out),
 * 10 max_n, 11 batch, 12 stream.
 */
int batchlu_gesv_vbatched(batchlu_dtype t, const int* n, const int* nrhs,
                          void* const* A, const int* lda, int* const* ipiv,
                          void* const* B, const int* ldb, int* info,
                          int max_n, int batch, hipStream_t stream);

/*
 * batchlu_potrf -- Cholesky factorisation of `batch` Hermitian (real:
 * symmetric) positive definite n x n matrices, in place.
 *   1 t, 2 uplo: 'L' computes A = L L^H and overwrites the lower triangle
 *     with L; 'U' computes A = U^H U and overwrites the upper triangle with
 *     U.  The other triangle is neither read nor written, and the imaginary
 *     part of a diagonal entry is never read (a stored diagonal entry of the
 *     factor has imaginary part +0),
 *   3 n >= 0, 4 A (device), 5 lda >= max(1, n), 6 strideA >= lda*n when
 *     batch > 1, 7 info (device int32[batch], out), 8 batch >= 0, 9 stream.
 * info[b] = 0 on success, or j + 1 when column j is the first whose diagonal
 * value (a_jj minus the squares of the row's earlier entries) is not
 * positive or is NaN: then a_jj holds that value, the factorisation stops,
 * and only columns 0 .. j-1 and a_jj of the factor are defined.  Orders up
 * to 1024 (complex double 512); larger ones return BATCHLU_ERR_CAPACITY.
 * Follows: BatchLAS "Blackwell" page, potrf rows of the status table and
 * the LPanel paragraph (entries accumulate over k in ascending order), and
 * the note that reference potf2 multiplies by a reciprocal of the diagonal.
 */
int batchlu_potrf(batchlu_dtype t, char uplo, int n, void* A, int lda,
                  long long strideA, int* info, int batch, hipStream_t stream);

/*
 * batchlu_potrs -- solve A X = B with the factor of batchlu_potrf.
 *   1 t, 2 uplo (the triangle holding the factor), 3 n, 4 nrhs >= 0,
 *   5 A (device, read only), 6 lda, 7 strideA, 8 B (device, in: right-hand
 *   sides, out: X), 9 ldb >= max(1, n), 10 strideB >= ldb*nrhs when
 *   batch > 1, 11 batch, 12 stream.
 * Forward with L (y_k = b_k / l_kk), then back with L^H, each a true
 * division by the real diagonal as reference trsm does.  n <= 1024, else
 * BATCHLU_ERR_CAPACITY.  Follows: BatchLAS "trsm" page, posv passages (posv
 * is potrf followed by the two triangular solves).
 */
int batchlu_potrs(batchlu_dtype t, char uplo, int n, int nrhs, const void* A,
                  int lda, long long strideA, void* B, int ldb,
                  long long strideB, int batch, hipStream_t stream);

/*
 * batchlu_posv -- potrf on A, then potrs on B.
 *   1 t, 2 uplo, 3 n, 4 nrhs, 5 A, 6 lda, 7 strideA, 8 B, 9 ldb,
 *  10 strideB, 11 info, 12 batch, 13 stream.
 * A matrix with info[b] > 0 keeps its B unchanged (LAPACK posv behaviour).
 * For n <= 64 (complex double 32) and nrhs <= 16 the solve is fused into
 * the factorisation kernel.  Follows: BatchLAS "Blackwell" page, posv
 * passages (fused solve arm on both triangles) and "trsm" page, posv
 * passages.
 */
int batchlu_posv(batchlu_dtype t, char uplo, int n, int nrhs, void* A,
                 int lda, long long strideA, void* B, int ldb,
                 long long strideB, int* info, int batch, hipStream_t stream);

/*
 * batchlu_select_tier -- the tier an AUTO call would use for this shape
 * (op: 0 getrf, 1 getrs, 2 gesv, 3 potrf, 4 posv; the Cholesky register
 * kernel reports as BATCHLU_TIER_CTA), or BATCHLU_ERR_CAPACITY / -k on bad
 * arguments.  Host only, launches nothing.  Follows: BatchLAS "LU" page,
 * routing tables (a rank of tiers per shape).
 */
int batchlu_select_tier(batchlu_dtype t, int op, int n, int nrhs, int batch);

/*
 * batchlu_set_tier -- pin every later call in this process to one tier
 * (BATCHLU_TIER_*; AUTO restores the selector).  For tests and A/B timing.
 * A pinned tier that cannot run a shape makes the call return
 * BATCHLU_ERR_CAPACITY.  Returns the previous setting.
 */
int batchlu_set_tier(int tier);

/*
 * batchlu_check_reciprocal -- device self-check of the fast float reciprocal
 * the register tiers use for pivots (BatchLAS "Blackwell" page, getrs tiny
 * paragraph: one reciprocal per pivot instead of a division per element;
 * the library forms it as v_rcp_f32 plus one Newton step wherever
 * 2^-125 <= |x| <= 2^125 and divides elsewhere, and relies on the result
 * being the correctly rounded 1/x there).
 *   1 lo_bits, 2 hi_bits  the inclusive range of float bit patterns to test
 *                         (hi_bits >= lo_bits, else -2)
 *   3 mismatches          device uint64, in: 0; out: += number of inputs in
 *                         the range whose fast reciprocal differs from the
 *                         IEEE quotient 1/x (inputs outside the fast range
 *                         are not counted: the library divides there)
 *   4 first_bad           device uint32, in: 0xffffffff; out: the lowest
 *                         such bit pattern (atomic minimum)
 *   5 stream
 * Diagnostic only; the factorisations never call it.
 */
int batchlu_check_reciprocal(unsigned int lo_bits, unsigned int hi_bits,
                             unsigned long long* mismatches,
                             unsigned int* first_bad, hipStream_t stream);

/* Human-readable name of a status code. */
const char* batchlu_status_string(int status);

/* Library version string. */
const char* batchlu_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BATCHLU_H */
