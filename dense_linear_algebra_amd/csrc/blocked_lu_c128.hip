// blocked_lu_c128.hip -- blocked-tier instantiations for one data type
// (split per type so the large unrolled panels compile in parallel).
#include "blocked_lu_impl.h"

namespace batchlu {

hipError_t blocked_getrf_c128(const Problem& p, hipStream_t s) { return getrf_t<cplx<double>>(p, s); }
hipError_t blocked_getrs_c128(const Problem& p, hipStream_t s) { return getrs_t<cplx<double>>(p, s); }
hipError_t blocked_getri_c128(const Problem& p, hipStream_t s) { return getri_t<cplx<double>>(p, s); }

}  // namespace batchlu
