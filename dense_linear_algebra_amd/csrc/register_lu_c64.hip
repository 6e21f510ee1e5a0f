// register_lu_c64.hip -- register-tier instantiations for one data type
// (split per type so the large unrolled kernels compile in parallel).
#include "register_lu_kernel.h"

namespace batchlu {

hipError_t register_launch_c64(const Problem& p, int mode, hipStream_t s) {
    return reg_detail::launch_type<cplx<float>>(p, mode, s);
}

}  // namespace batchlu
