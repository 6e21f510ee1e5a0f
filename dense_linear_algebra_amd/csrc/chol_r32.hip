// chol_r32.hip -- Cholesky kernels for one data type (split per type so
// the unrolled register kernels compile in parallel).
#include "chol_kernels.h"

namespace batchlu {

hipError_t chol_register_r32(const Problem& p, bool solve, hipStream_t s) {
    return chol::launch_reg<float>(p, solve, s);
}
hipError_t chol_blocked_r32(const Problem& p, hipStream_t s) { return chol::launch_potrf_blocked<float>(p, s); }
hipError_t chol_solve_r32(const Problem& p, hipStream_t s) { return chol::launch_solve<float>(p, s); }

}  // namespace batchlu
