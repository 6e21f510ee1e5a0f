// register_lu_c128.hip -- register-tier instantiations for one data type
// (split per type so the large unrolled kernels compile in parallel).
#include "register_lu_kernel.h"

namespace batchlu {

hipError_t register_launch_c128(const Problem& p, int mode, hipStream_t s) {
    return reg_detail::launch_type<cplx<double>>(p, mode, s);
}

}  // namespace batchlu
