// internal.h -- host-side interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace batchlu {

enum Dtype { R32 = 0, R64 = 1, C64 = 2, C128 = 3 };

inline int elem_bytes(int t) { return t == R32 ? 4 : (t == C128 ? 16 : 8); }

// One batched problem on strided, column-major storage.  Offsets are in
// elements of the data type.  `mode` selects what a fused kernel does.
struct Problem {
    int n = 0, nrhs = 0, batch = 0;
    void* A = nullptr;  int lda = 0;  long long sA = 0;
    int* ipiv = nullptr;  long long sP = 0;
    int* info = nullptr;
    void* B = nullptr;  int ldb = 0;  long long sB = 0;
    int trans = 0;      // getrs: 0 solves A X = B, 1 A^T X = B, 2 A^H X = B
    bool inverse = false;   // getri: B is the output C; the solve runs on the identity
    bool upper = false;     // Cholesky: the factor lives in the upper triangle (A = U^H U)
};

enum Mode { MODE_GETRF = 0, MODE_GESV = 1 };

// Register tiers.  Return hipSuccess, or the launch error.  `supported`
// answers whether the kernel set holds an instantiation for the shape.
bool register_supported(int dtype, int n, int nrhs, int mode, bool one_wave_per_matrix);
hipError_t register_launch(int dtype, const Problem& p, int mode, bool one_wave_per_matrix,
                           hipStream_t s);

// Solve with given factors in one launch (one work-group per matrix and RHS
// tile, one row per thread), n <= 1024, for every p.trans.  With p.info
// set, matrices whose info is non-zero are skipped (composed gesv, NoTrans).
bool getrs_rows_supported(int dtype, int n);
hipError_t getrs_rows_launch(int dtype, const Problem& p, hipStream_t s);

// LDS-staged work-group tier: one work-group per matrix, [A | B] in LDS
// (n <= 128, complex double 64; gesv fused for nrhs <= 16).
bool cta_lds_supported(int dtype, int n, int nrhs, int mode);
hipError_t cta_lds_launch(int dtype, const Problem& p, int mode, hipStream_t s);

// Blocked tier in one work-group per matrix (real types, n <= 256).
bool blocked_fused_supported(int dtype, int n, int lda);
hipError_t blocked_fused_getrf(int dtype, const Problem& p, hipStream_t s);

// A second stream on the current device for running a panel beside the
// previous panel's trailing update, with the two events of the fork and the
// join.  Created once per device; lookahead_begin also takes a lock held
// until lookahead_end, so that concurrent callers do not interleave their
// event records.  lookahead_begin returns false (and the caller runs without
// look-ahead) if the stream or events cannot be created.
struct LookAhead {
    hipStream_t side = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    bool held = false;
};
bool lookahead_begin(LookAhead& la);
hipError_t lookahead_fork(LookAhead& la, hipStream_t s);       // side waits for s's work so far
hipError_t lookahead_join_record(LookAhead& la);               // marks the side's work so far
hipError_t lookahead_join_wait(LookAhead& la, hipStream_t s);  // s waits for that mark
hipError_t lookahead_end(LookAhead& la, hipError_t status);    // releases the lock, returns status

// Blocked right-looking tier (panel, laswp, trsm, gemm) and blocked getrs.
// blocked_getrs serves every p.trans and, with p.inverse, getri (B is the
// output C, set to the identity first); n <= 4096.
bool blocked_supported(int dtype, int n);
bool blocked_getrs_supported(int dtype, int n);
hipError_t blocked_getrf(int dtype, const Problem& p, hipStream_t s);
hipError_t blocked_getrs(int dtype, const Problem& p, hipStream_t s);

// Cholesky (potrf / potrs / posv), both triangles.  Register tier: n <= 64
// (complex double 32), posv fused for nrhs <= 16.  Blocked tier: n <= 1024
// (complex double 512).  Solve: n <= 1024.
// LU of m x n matrices and of variable-size batches (one work-group per
// matrix, m <= general_max_rows, n <= 1024); the solve for square
// variable-size batches (n <= 1024).  Matrices whose sizes fall outside
// what the launch covers get info = -1 and are not touched.
int general_max_rows(int dtype);
hipError_t general_getrf_strided(int dtype, void* A, int m, int n, int lda, long long sA, int* ipiv, long long sP,
                                 int* info, int batch, hipStream_t s);
hipError_t general_getrf_vbatched(int dtype, void* const* A, const int* m, const int* n, const int* lda,
                                  int* const* ipiv, int* info, int max_m, int batch, hipStream_t s);
hipError_t general_getrs_vbatched(int dtype, void* const* A, const int* n, const int* lda, int* const* ipiv,
                                  const int* nrhs, void* const* B, const int* ldb, int* info, int max_n, int batch,
                                  hipStream_t s);

bool chol_register_supported(int dtype, int n);
bool chol_blocked_supported(int dtype, int n);
bool chol_solve_supported(int dtype, int n);
hipError_t chol_register_launch(int dtype, const Problem& p, bool solve, hipStream_t s);
hipError_t chol_blocked_launch(int dtype, const Problem& p, hipStream_t s);
hipError_t chol_solve_launch(int dtype, const Problem& p, hipStream_t s);

}  // namespace batchlu
