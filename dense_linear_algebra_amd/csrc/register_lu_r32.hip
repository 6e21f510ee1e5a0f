// register_lu_r32.hip -- register-tier instantiations for one data type
// (split per type so the large unrolled kernels compile in parallel).
#include "register_lu_kernel.h"
#include "register_lu_row16.h"

namespace batchlu {

// Orders 9..32 use one matrix per 16-lane DPP row (pivot row and x_k moved
// by DPP); the other orders use the generic lane-group kernel.
hipError_t register_launch_r32(const Problem& p, int mode, hipStream_t s) {
    if (p.n >= 9 && p.n <= 32) {
        const int nr = reg_detail::pick_nr(p.nrhs, mode);
        if (nr >= 0) return row16_detail::launch_row16(p, mode, nr, s);
    }
    return reg_detail::launch_type<float>(p, mode, s);
}

}  // namespace batchlu
