// chol_c64.hip -- Cholesky kernels for one data type (split per type so
// the unrolled register kernels compile in parallel).
#include "chol_kernels.h"

namespace batchlu {

hipError_t chol_register_c64(const Problem& p, bool solve, hipStream_t s) {
    return chol::launch_reg<cplx<float>>(p, solve, s);
}
hipError_t chol_blocked_c64(const Problem& p, hipStream_t s) { return chol::launch_potrf_blocked<cplx<float>>(p, s); }
hipError_t chol_solve_c64(const Problem& p, hipStream_t s) { return chol::launch_solve<cplx<float>>(p, s); }

}  // namespace batchlu
