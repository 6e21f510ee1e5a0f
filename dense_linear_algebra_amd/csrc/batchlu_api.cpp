// batchlu_api.cpp -- the C ABI: argument checks, tier selection, dispatch.
//
// Tier selection (BatchLAS "LU" page, family table and routing tables): the
// pages rank register-resident kernels first for small n, a one-work-group
// kernel for mid n and the blocked right-looking driver above, keyed on the
// shape and the batch.  On gfx950 the register tiers hold a matrix in VGPRs:
//   tiny    n <= 32: several matrices per wavefront;
//   cta     32 < n <= 64 (complex double: none): one wavefront per matrix;
//   blocked larger n, nb = 32;
//   cta_lds one work-group per matrix with the matrix in LDS (n <= 128):
//           the fastest gesv for small batches in the cells listed below,
//           slower than the others at batch >= 1024 and at n >= 96.
// gesv runs fused (factor + forward + back in one kernel) in the register
// tiers while nrhs <= 16, except where the measured crossovers below pick
// the composed factor-then-solve; otherwise it is getrf followed by getrs.
#include <atomic>
#include <climits>
#include <cstdlib>
#include <cstring>

#include "../../include/batchlu.h"
#include "internal.h"

using namespace batchlu;

namespace {

std::atomic<int> g_tier_pin{-1};   // -1: not read from the environment yet

int tier_pin() {
    int v = g_tier_pin.load(std::memory_order_relaxed);
    if (v >= 0) return v;
    int from_env = BATCHLU_TIER_AUTO;
    if (const char* e = std::getenv("BATCHLU_TIER")) {
        if (!std::strcmp(e, "tiny")) from_env = BATCHLU_TIER_TINY;
        else if (!std::strcmp(e, "cta")) from_env = BATCHLU_TIER_CTA;
        else if (!std::strcmp(e, "blocked")) from_env = BATCHLU_TIER_BLOCKED;
    }
    int expected = -1;
    g_tier_pin.compare_exchange_strong(expected, from_env);
    return g_tier_pin.load();
}

bool valid_dtype(int t) { return t >= BATCHLU_R32 && t <= BATCHLU_C128; }

enum Op { OP_GETRF = 0, OP_GETRS = 1, OP_GESV = 2 };

bool tier_can_run(int tier, int t, int op, int n, int nrhs) {
    switch (tier) {
    case BATCHLU_TIER_TINY:
    case BATCHLU_TIER_CTA: {
        const bool one_wave = tier == BATCHLU_TIER_CTA;
        if (op == OP_GETRS) return getrs_rows_supported(t, n) && n <= 64;
        if (op == OP_GESV) return register_supported(t, n, nrhs, MODE_GESV, one_wave) ||
                                  (register_supported(t, n, 0, MODE_GETRF, one_wave) &&
                                   getrs_rows_supported(t, n));
        return register_supported(t, n, 0, MODE_GETRF, one_wave);
    }
    case BATCHLU_TIER_BLOCKED:
        if (op == OP_GETRS) return blocked_getrs_supported(t, n) || getrs_rows_supported(t, n);
        return blocked_supported(t, n);
    case BATCHLU_TIER_CTA_LDS:
        if (op == OP_GETRS) return getrs_rows_supported(t, n) && cta_lds_supported(t, n, 0, MODE_GETRF);
        if (op == OP_GESV) return cta_lds_supported(t, n, nrhs, MODE_GESV) ||
                                  (cta_lds_supported(t, n, 0, MODE_GETRF) && getrs_rows_supported(t, n));
        return cta_lds_supported(t, n, 0, MODE_GETRF);
    default:
        return false;
    }
}

// Measured crossovers (MI355X, every tier timed on a grid of type x n in
// {8..256} x batch in {1..8192} x nrhs in {1, 16}; `bench.py --tier-sweep`,
// summary in profiles/selector_sweep.md).  The register tiers win getrf
// everywhere they run, and gesv everywhere at batch >= 1024; at batch <= 256
// with more than 8 right-hand sides the fused kernel's one wavefront per
// matrix carries the whole solve serially, and factoring in the register or
// blocked tier then solving with one work-group per (matrix, RHS tile) is
// faster for these orders (ratios 0.6 - 0.95 of the fused time).
constexpr int kSmallBatch = 256;

bool lu_composed_wins(int t, int n) {
    switch (t) {
    case BATCHLU_R32: return n <= 8;
    case BATCHLU_R64: return n >= 16;
    // complex float: the register tiers' back substitution with one x_k
    // entry per lane made them the fastest at n = 32 too (0.89 - 0.93 of
    // the composition's time)
    case BATCHLU_C64: return false;
    default: return n >= 16;
    }
}

// gesv at batch <= 256 (same sweep): the LDS-staged work-group tier is the
// fastest for complex double at 33 <= n <= 64 (no register tier there;
// 0.54 - 0.94 of the blocked time) and, with more than 8 right-hand sides,
// for these small orders (0.6 - 0.9 of the next best).
bool lds_wins(int t, int n, int nrhs) {
    switch (t) {
    case BATCHLU_R32: return nrhs > 8 && n <= 8;
    case BATCHLU_R64: return nrhs > 8 && (n <= 16 || (n >= 33 && n <= 40));
    case BATCHLU_C64: return nrhs > 8 && (n <= 16 || (n >= 33 && n <= 48));
    default: return (n >= 33 && n <= 64) || (nrhs > 8 && n <= 16);
    }
}

int auto_tier(int t, int op, int n, int nrhs, int batch) {
    // float n <= 8 with many right-hand sides: the LDS tier still wins at
    // batch 1024 (0.67 of the next best), not at 8192
    if (op == OP_GESV && t == BATCHLU_R32 && n <= 8 && nrhs > 8 && batch <= 4 * kSmallBatch &&
        tier_can_run(BATCHLU_TIER_CTA_LDS, t, op, n, nrhs))
        return BATCHLU_TIER_CTA_LDS;
    if (op == OP_GESV && batch <= kSmallBatch && nrhs > 0) {
        if (lds_wins(t, n, nrhs) && tier_can_run(BATCHLU_TIER_CTA_LDS, t, op, n, nrhs))
            return BATCHLU_TIER_CTA_LDS;
        if (nrhs > 8 && lu_composed_wins(t, n) && tier_can_run(BATCHLU_TIER_BLOCKED, t, op, n, nrhs))
            return BATCHLU_TIER_BLOCKED;
    }
    const int order[3] = {BATCHLU_TIER_TINY, BATCHLU_TIER_CTA, BATCHLU_TIER_BLOCKED};
    for (int tier : order)
        if (tier_can_run(tier, t, op, n, nrhs)) return tier;
    return BATCHLU_ERR_CAPACITY;
}

int choose(int t, int op, int n, int nrhs, int batch) {
    const int pin = tier_pin();
    if (pin != BATCHLU_TIER_AUTO) return tier_can_run(pin, t, op, n, nrhs) ? pin : BATCHLU_ERR_CAPACITY;
    return auto_tier(t, op, n, nrhs, batch);
}

int status_of(hipError_t e) { return e == hipSuccess ? BATCHLU_OK : BATCHLU_ERR_LAUNCH; }

int run_getrf(int tier, int t, const Problem& p, hipStream_t s) {
    switch (tier) {
    case BATCHLU_TIER_TINY: return status_of(register_launch(t, p, MODE_GETRF, false, s));
    case BATCHLU_TIER_CTA: return status_of(register_launch(t, p, MODE_GETRF, true, s));
    case BATCHLU_TIER_BLOCKED: return status_of(blocked_getrf(t, p, s));
    case BATCHLU_TIER_CTA_LDS: return status_of(cta_lds_launch(t, p, MODE_GETRF, s));
    default: return BATCHLU_ERR_CAPACITY;
    }
}

// The one-launch solve covers n <= 1024; larger orders use the blocked
// sequence of triangular-block solves and GEMM updates.
int run_getrs(int tier, int t, const Problem& p, hipStream_t s) {
    (void)tier;
    if (getrs_rows_supported(t, p.n)) return status_of(getrs_rows_launch(t, p, s));
    return status_of(blocked_getrs(t, p, s));
}

}  // namespace

extern "C" {

int batchlu_getrf(batchlu_dtype t, int n, void* A, int lda, long long strideA, int* ipiv,
                  long long strideP, int* info, int batch, hipStream_t stream) {
    if (!valid_dtype(t)) return -1;
    if (n < 0) return -2;
    if (lda < (n > 1 ? n : 1)) return -4;
    if (batch < 0) return -9;
    if (batch > 1 && strideA < (long long)lda * n) return -5;
    if (batch > 1 && strideP < n) return -7;
    if (n == 0 || batch == 0) return BATCHLU_OK;
    if (!A) return -3;
    if (!ipiv) return -6;
    if (!info) return -8;
    const int tier = choose(t, OP_GETRF, n, 0, batch);
    if (tier < 0) return tier;
    Problem p;
    p.n = n; p.batch = batch; p.A = A; p.lda = lda; p.sA = strideA;
    p.ipiv = ipiv; p.sP = strideP; p.info = info;
    return run_getrf(tier, t, p, stream);
}

int batchlu_getrs(batchlu_dtype t, char trans, int n, int nrhs, const void* A, int lda,
                  long long strideA, const int* ipiv, long long strideP, void* B, int ldb,
                  long long strideB, int batch, hipStream_t stream) {
    if (!valid_dtype(t)) return -1;
    if (trans != 'N' && trans != 'n' && trans != 'T' && trans != 't' && trans != 'C' && trans != 'c')
        return -2;
    if (n < 0) return -3;
    if (nrhs < 0) return -4;
    if (lda < (n > 1 ? n : 1)) return -6;
    if (ldb < (n > 1 ? n : 1)) return -11;
    if (batch < 0) return -13;
    if (batch > 1 && strideA < (long long)lda * n) return -7;
    if (batch > 1 && strideP < n) return -9;
    if (batch > 1 && strideB < (long long)ldb * nrhs) return -12;
    const int op = (trans == 'N' || trans == 'n') ? 0 : (trans == 'T' || trans == 't') ? 1 : 2;
    if (n == 0 || nrhs == 0 || batch == 0) return BATCHLU_OK;
    if (!A) return -5;
    if (!ipiv) return -8;
    if (!B) return -10;
    if (!getrs_rows_supported(t, n) && !blocked_getrs_supported(t, n)) return BATCHLU_ERR_UNSUPPORTED;
    const int tier = choose(t, OP_GETRS, n, nrhs, batch);
    if (tier < 0) return tier;
    Problem p;
    p.n = n; p.nrhs = nrhs; p.batch = batch; p.A = const_cast<void*>(A); p.lda = lda; p.sA = strideA;
    p.ipiv = const_cast<int*>(ipiv); p.sP = strideP; p.B = B; p.ldb = ldb; p.sB = strideB;
    p.trans = op;
    return run_getrs(tier, t, p, stream);
}

int batchlu_getri(batchlu_dtype t, int n, const void* A, int lda, long long strideA, const int* ipiv,
                  long long strideP, void* C, int ldc, long long strideC, int batch, hipStream_t stream) {
    if (!valid_dtype(t)) return -1;
    if (n < 0) return -2;
    if (lda < (n > 1 ? n : 1)) return -4;
    if (ldc < (n > 1 ? n : 1)) return -9;
    if (batch < 0) return -11;
    if (batch > 1 && strideA < (long long)lda * n) return -5;
    if (batch > 1 && strideP < n) return -7;
    if (batch > 1 && strideC < (long long)ldc * n) return -10;
    if (n == 0 || batch == 0) return BATCHLU_OK;
    if (!A) return -3;
    if (!ipiv) return -6;
    if (!C) return -8;
    {   // out of place: the byte ranges of A and C must not meet
        const long long es = (t == BATCHLU_C128) ? 16 : (t == BATCHLU_R32) ? 4 : 8;
        const long long ea = es * ((long long)(batch - 1) * strideA + (long long)(n - 1) * lda + n);
        const long long ec = es * ((long long)(batch - 1) * strideC + (long long)(n - 1) * ldc + n);
        const char* a0 = (const char*)A;
        const char* c0 = (const char*)C;
        if (c0 < a0 + ea && a0 < c0 + ec) return -8;
    }
    if (!getrs_rows_supported(t, n) && !blocked_getrs_supported(t, n)) return BATCHLU_ERR_UNSUPPORTED;
    Problem p;
    p.n = n; p.nrhs = n; p.batch = batch; p.A = const_cast<void*>(A); p.lda = lda; p.sA = strideA;
    p.ipiv = const_cast<int*>(ipiv); p.sP = strideP; p.B = C; p.ldb = ldc; p.sB = strideC;
    p.inverse = true;
    if (getrs_rows_supported(t, n)) return status_of(getrs_rows_launch(t, p, stream));
    return status_of(blocked_getrs(t, p, stream));
}

int batchlu_gesv(batchlu_dtype t, int n, int nrhs, void* A, int lda, long long strideA, int* ipiv,
                 long long strideP, void* B, int ldb, long long strideB, int* info, int batch,
                 hipStream_t stream) {
    if (!valid_dtype(t)) return -1;
    if (n < 0) return -2;
    if (nrhs < 0) return -3;
    if (lda < (n > 1 ? n : 1)) return -5;
    if (ldb < (n > 1 ? n : 1)) return -10;
    if (batch < 0) return -13;
    if (batch > 1 && strideA < (long long)lda * n) return -6;
    if (batch > 1 && strideP < n) return -8;
    if (batch > 1 && strideB < (long long)ldb * nrhs) return -11;
    if (n == 0 || batch == 0) return BATCHLU_OK;
    if (!A) return -4;
    if (!ipiv) return -7;
    if (nrhs > 0 && !B) return -9;
    if (!info) return -12;
    const int tier = choose(t, OP_GESV, n, nrhs, batch);
    if (tier < 0) return tier;
    Problem p;
    p.n = n; p.nrhs = nrhs; p.batch = batch; p.A = A; p.lda = lda; p.sA = strideA;
    p.ipiv = ipiv; p.sP = strideP; p.info = info; p.B = B; p.ldb = ldb; p.sB = strideB;
    if (tier == BATCHLU_TIER_CTA_LDS && nrhs > 0 && cta_lds_supported(t, n, nrhs, MODE_GESV))
        return status_of(cta_lds_launch(t, p, MODE_GESV, stream));
    if ((tier == BATCHLU_TIER_TINY || tier == BATCHLU_TIER_CTA) && nrhs > 0 &&
        register_supported(t, n, nrhs, MODE_GESV, tier == BATCHLU_TIER_CTA))
        return status_of(register_launch(t, p, MODE_GESV, tier == BATCHLU_TIER_CTA, stream));
    int st = run_getrf(tier, t, p, stream);
    if (st != BATCHLU_OK || nrhs == 0) return st;
    // getrs on matrices with info > 0 would overwrite B; LAPACK gesv leaves B
    // alone there.  The composed path therefore solves into B only where the
    // factorisation succeeded: the solve kernels read info when it is given.
    return run_getrs(tier, t, p, stream);
}

// ---------------------------------------------------------------------------
// Cholesky.  Tiers: the register kernel (TINY and CTA pins both name it),
// else the blocked driver; posv fuses the solve in the register kernel for
// nrhs <= 16 and otherwise composes potrf with the one-launch solve.
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

bool valid_uplo(char u) { return u == 'L' || u == 'l' || u == 'U' || u == 'u'; }
bool is_upper(char u) { return u == 'U' || u == 'u'; }

// posv at batch <= 256 (same sweep): the blocked potrf plus the one-launch
// solve beats the fused register kernel for these orders with more than 8
// right-hand sides, and for double at n >= 64 with any number.
bool chol_composed_wins(int t, int n, int nrhs) {
    if (t == BATCHLU_R64 && n >= 64) return true;
    if (nrhs <= 8) return false;
    switch (t) {
    case BATCHLU_R32: return n >= 48;
    case BATCHLU_R64: return n >= 32;
    case BATCHLU_C64: return n >= 32;
    default: return n >= 16;
    }
}

int chol_tier(int t, int op, int n, int nrhs, int batch) {
    const int pin = tier_pin();
    const bool reg = chol_register_supported(t, n), blk = chol_blocked_supported(t, n);
    if (pin == BATCHLU_TIER_TINY || pin == BATCHLU_TIER_CTA) return reg ? pin : BATCHLU_ERR_CAPACITY;
    if (pin == BATCHLU_TIER_BLOCKED) return blk ? pin : BATCHLU_ERR_CAPACITY;
    if (pin == BATCHLU_TIER_CTA_LDS) return BATCHLU_ERR_CAPACITY;   // no LDS-staged Cholesky
    if (reg && blk && op == 4 && batch <= kSmallBatch && nrhs > 0 && chol_composed_wins(t, n, nrhs))
        return BATCHLU_TIER_BLOCKED;
    return reg ? BATCHLU_TIER_CTA : blk ? BATCHLU_TIER_BLOCKED : BATCHLU_ERR_CAPACITY;
}

int run_potrf(int tier, int t, const Problem& p, hipStream_t s) {
    if (tier == BATCHLU_TIER_BLOCKED) return status_of(chol_blocked_launch(t, p, s));
    return status_of(chol_register_launch(t, p, false, s));
}

}  // namespace

extern "C" {

int batchlu_potrf(batchlu_dtype t, char uplo, int n, void* A, int lda, long long strideA, int* info, int batch,
                  hipStream_t stream) {
    if (!valid_dtype(t)) return -1;
    if (!valid_uplo(uplo)) return -2;
    if (n < 0) return -3;
    if (lda < (n > 1 ? n : 1)) return -5;
    if (batch < 0) return -8;
    if (batch > 1 && strideA < (long long)lda * n) return -6;
    if (n == 0 || batch == 0) return BATCHLU_OK;
    if (!A) return -4;
    if (!info) return -7;
    const int tier = chol_tier(t, 3, n, 0, batch);
    if (tier < 0) return tier;
    Problem p;
    p.n = n; p.batch = batch; p.A = A; p.lda = lda; p.sA = strideA; p.info = info; p.upper = is_upper(uplo);
    return run_potrf(tier, t, p, stream);
}

int batchlu_potrs(batchlu_dtype t, char uplo, int n, int nrhs, const void* A, int lda, long long strideA, void* B,
                  int ldb, long long strideB, int batch, hipStream_t stream) {
    if (!valid_dtype(t)) return -1;
    if (!valid_uplo(uplo)) return -2;
    if (n < 0) return -3;
    if (nrhs < 0) return -4;
    if (lda < (n > 1 ? n : 1)) return -6;
    if (ldb < (n > 1 ? n : 1)) return -9;
    if (batch < 0) return -11;
    if (batch > 1 && strideA < (long long)lda * n) return -7;
    if (batch > 1 && strideB < (long long)ldb * nrhs) return -10;
    if (n == 0 || nrhs == 0 || batch == 0) return BATCHLU_OK;
    if (!A) return -5;
    if (!B) return -8;
    if (!chol_solve_supported(t, n)) return BATCHLU_ERR_CAPACITY;
    Problem p;
    p.n = n; p.nrhs = nrhs; p.batch = batch; p.A = const_cast<void*>(A); p.lda = lda; p.sA = strideA;
    p.B = B; p.ldb = ldb; p.sB = strideB; p.upper = is_upper(uplo);
    return status_of(chol_solve_launch(t, p, stream));
}

int batchlu_posv(batchlu_dtype t, char uplo, int n, int nrhs, void* A, int lda, long long strideA, void* B, int ldb,
                 long long strideB, int* info, int batch, hipStream_t stream) {
    if (!valid_dtype(t)) return -1;
    if (!valid_uplo(uplo)) return -2;
    if (n < 0) return -3;
    if (nrhs < 0) return -4;
    if (lda < (n > 1 ? n : 1)) return -6;
    if (ldb < (n > 1 ? n : 1)) return -9;
    if (batch < 0) return -12;
    if (batch > 1 && strideA < (long long)lda * n) return -7;
    if (batch > 1 && strideB < (long long)ldb * nrhs) return -10;
    if (n == 0 || batch == 0) return BATCHLU_OK;
    if (!A) return -5;
    if (nrhs > 0 && !B) return -8;
    if (!info) return -11;
    const int tier = chol_tier(t, 4, n, nrhs, batch);
    if (tier < 0) return tier;
    if (nrhs > 0 && !chol_solve_supported(t, n)) return BATCHLU_ERR_CAPACITY;
    Problem p;
    p.n = n; p.nrhs = nrhs; p.batch = batch; p.A = A; p.lda = lda; p.sA = strideA; p.info = info;
    p.B = B; p.ldb = ldb; p.sB = strideB; p.upper = is_upper(uplo);
    if (tier != BATCHLU_TIER_BLOCKED && nrhs > 0 && nrhs <= 16)
        return status_of(chol_register_launch(t, p, true, stream));
    const int st = run_potrf(tier, t, p, stream);
    if (st != BATCHLU_OK || nrhs == 0) return st;
    return status_of(chol_solve_launch(t, p, stream));   // skips matrices whose info > 0
}

// ---------------------------------------------------------------------------
// Rectangular and variable-size LU (one work-group per matrix).
// ---------------------------------------------------------------------------
int batchlu_getrf_rect(batchlu_dtype t, int m, int n, void* A, int lda, long long strideA, int* ipiv,
                       long long strideP, int* info, int batch, hipStream_t stream) {
    if (!valid_dtype(t)) return -1;
    if (m < 0) return -2;
    if (n < 0) return -3;
    if (lda < (m > 1 ? m : 1)) return -5;
    if (batch < 0) return -10;
    const int k = m < n ? m : n;
    if (batch > 1 && strideA < (long long)lda * n) return -6;
    if (batch > 1 && strideP < k) return -8;
    if (m == 0 || n == 0 || batch == 0) return BATCHLU_OK;   // no work: nothing is launched
    if (!info) return -9;
    if (!A) return -4;
    if (!ipiv) return -7;
    if (m == n) return batchlu_getrf(t, n, A, lda, strideA, ipiv, strideP, info, batch, stream);
    if (m > general_max_rows(t) || n > 1024) return BATCHLU_ERR_CAPACITY;
    return status_of(general_getrf_strided(t, A, m, n, lda, strideA, ipiv, strideP, info, batch, stream));
}

int batchlu_getrf_vbatched(batchlu_dtype t, const int* m, const int* n, void* const* A, const int* lda,
                           int* const* ipiv, int* info, int max_m, int max_n, int batch, hipStream_t stream) {
    if (!valid_dtype(t)) return -1;
    if (batch < 0) return -10;
    if (max_m < 0) return -8;
    if (max_n < 0) return -9;
    if (batch == 0) return BATCHLU_OK;
    if (!m) return -2;
    if (!n) return -3;
    if (!A) return -4;
    if (!lda) return -5;
    if (!ipiv) return -6;
    if (!info) return -7;
    if (max_m > general_max_rows(t) || max_n > 1024) return BATCHLU_ERR_CAPACITY;
    return status_of(general_getrf_vbatched(t, A, m, n, lda, ipiv, info, max_m > 0 ? max_m : 1, batch, stream));
}

int batchlu_getrs_vbatched(batchlu_dtype t, const int* n, const int* nrhs, void* const* A, const int* lda,
                           int* const* ipiv, void* const* B, const int* ldb, int max_n, int batch,
                           hipStream_t stream) {
    if (!valid_dtype(t)) return -1;
    if (max_n < 0) return -9;
    if (batch < 0) return -10;
    if (batch == 0 || max_n == 0) return BATCHLU_OK;
    if (!n) return -2;
    if (!nrhs) return -3;
    if (!A) return -4;
    if (!lda) return -5;
    if (!ipiv) return -6;
    if (!B) return -7;
    if (!ldb) return -8;
    if (max_n > 1024) return BATCHLU_ERR_CAPACITY;
    return status_of(general_getrs_vbatched(t, A, n, lda, ipiv, nrhs, B, ldb, nullptr, max_n, batch, stream));
}

int batchlu_gesv_vbatched(batchlu_dtype t, const int* n, const int* nrhs, void* const* A, const int* lda,
                          int* const* ipiv, void* const* B, const int* ldb, int* info, int max_n, int batch,
                          hipStream_t stream) {
    if (!valid_dtype(t)) return -1;
    if (max_n < 0) return -10;
    if (batch < 0) return -11;
    if (batch == 0) return BATCHLU_OK;
    if (!n) return -2;
    if (!nrhs) return -3;
    if (!A) return -4;
    if (!lda) return -5;
    if (!ipiv) return -6;
    if (!B) return -7;
    if (!ldb) return -8;
    if (!info) return -9;
    if (max_n > general_max_rows(t) || max_n > 1024) return BATCHLU_ERR_CAPACITY;
    const int mm = max_n > 0 ? max_n : 1;
    int st = status_of(general_getrf_vbatched(t, A, n, n, lda, ipiv, info, mm, batch, stream));
    if (st != BATCHLU_OK) return st;
    return status_of(general_getrs_vbatched(t, A, n, lda, ipiv, nrhs, B, ldb, info, mm, batch, stream));
}

int batchlu_select_tier(batchlu_dtype t, int op, int n, int nrhs, int batch) {
    if (!valid_dtype(t)) return -1;
    if (op < OP_GETRF || op > 4) return -2;
    if (n < 0) return -3;
    if (nrhs < 0) return -4;
    if (batch < 0) return -5;
    if (op >= 3) return chol_tier(t, op, n, nrhs, batch);   // 3 potrf, 4 posv
    return choose(t, op, n, nrhs, batch);
}

int batchlu_set_tier(int tier) {
    const int prev = tier_pin();
    if (tier < BATCHLU_TIER_AUTO || tier > BATCHLU_TIER_CTA_LDS) return -1;
    g_tier_pin.store(tier);
    return prev;
}

const char* batchlu_status_string(int status) {
    switch (status) {
    case BATCHLU_OK: return "ok";
    case BATCHLU_ERR_UNSUPPORTED: return "unsupported option";
    case BATCHLU_ERR_CAPACITY: return "shape exceeds every tier's capacity";
    case BATCHLU_ERR_LAUNCH: return "kernel launch failed";
    default: return status < 0 && status > -20 ? "invalid argument" : "unknown status";
    }
}

const char* batchlu_version(void) { return "batchlu 0.1.0 (gfx950)"; }

}  // extern "C"
