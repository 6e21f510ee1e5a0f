// chol_dispatch.cpp -- host dispatch of the Cholesky kernels by data type.
#include "internal.h"

namespace batchlu {

hipError_t chol_register_r32(const Problem& p, bool solve, hipStream_t s);
hipError_t chol_register_r64(const Problem& p, bool solve, hipStream_t s);
hipError_t chol_register_c64(const Problem& p, bool solve, hipStream_t s);
hipError_t chol_register_c128(const Problem& p, bool solve, hipStream_t s);
hipError_t chol_blocked_r32(const Problem& p, hipStream_t s);
hipError_t chol_blocked_r64(const Problem& p, hipStream_t s);
hipError_t chol_blocked_c64(const Problem& p, hipStream_t s);
hipError_t chol_blocked_c128(const Problem& p, hipStream_t s);
hipError_t chol_solve_r32(const Problem& p, hipStream_t s);
hipError_t chol_solve_r64(const Problem& p, hipStream_t s);
hipError_t chol_solve_c64(const Problem& p, hipStream_t s);
hipError_t chol_solve_c128(const Problem& p, hipStream_t s);

bool chol_register_supported(int dtype, int n) { return n >= 1 && n <= (dtype == C128 ? 32 : 64); }
bool chol_blocked_supported(int dtype, int n) { return n >= 1 && n <= (dtype == C128 ? 512 : 1024); }
bool chol_solve_supported(int dtype, int n) {
    (void)dtype;
    return n >= 1 && n <= 1024;
}

hipError_t chol_register_launch(int dtype, const Problem& p, bool solve, hipStream_t s) {
    if (!chol_register_supported(dtype, p.n) || (solve && p.nrhs > 16)) return hipErrorInvalidValue;
    switch (dtype) {
    case R32: return chol_register_r32(p, solve, s);
    case R64: return chol_register_r64(p, solve, s);
    case C64: return chol_register_c64(p, solve, s);
    case C128: return chol_register_c128(p, solve, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t chol_blocked_launch(int dtype, const Problem& p, hipStream_t s) {
    if (!chol_blocked_supported(dtype, p.n)) return hipErrorInvalidValue;
    switch (dtype) {
    case R32: return chol_blocked_r32(p, s);
    case R64: return chol_blocked_r64(p, s);
    case C64: return chol_blocked_c64(p, s);
    case C128: return chol_blocked_c128(p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t chol_solve_launch(int dtype, const Problem& p, hipStream_t s) {
    if (!chol_solve_supported(dtype, p.n)) return hipErrorInvalidValue;
    switch (dtype) {
    case R32: return chol_solve_r32(p, s);
    case R64: return chol_solve_r64(p, s);
    case C64: return chol_solve_c64(p, s);
    case C128: return chol_solve_c128(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace batchlu
