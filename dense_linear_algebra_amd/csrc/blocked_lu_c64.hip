// blocked_lu_c64.hip -- blocked-tier instantiations for one data type
// (split per type so the large unrolled panels compile in parallel).
#include "blocked_lu_impl.h"

namespace batchlu {

hipError_t blocked_getrf_c64(const Problem& p, hipStream_t s) { return getrf_t<cplx<float>>(p, s); }
hipError_t blocked_getrs_c64(const Problem& p, hipStream_t s) { return getrs_t<cplx<float>>(p, s); }
hipError_t blocked_getri_c64(const Problem& p, hipStream_t s) { return getri_t<cplx<float>>(p, s); }

}  // namespace batchlu
