// chol_r64.hip -- Cholesky kernels for one data type (split per type so
// the unrolled register kernels compile in parallel).
#include "chol_kernels.h"

namespace batchlu {

hipError_t chol_register_r64(const Problem& p, bool solve, hipStream_t s) {
    return chol::launch_reg<double>(p, solve, s);
}
hipError_t chol_blocked_r64(const Problem& p, hipStream_t s) { return chol::launch_potrf_blocked<double>(p, s); }
hipError_t chol_solve_r64(const Problem& p, hipStream_t s) { return chol::launch_solve<double>(p, s); }

}  // namespace batchlu
