// blocked_lu_r32.hip -- blocked-tier instantiations for one data type
// (split per type so the large unrolled panels compile in parallel).
#include "blocked_lu_impl.h"

namespace batchlu {

hipError_t blocked_getrf_r32(const Problem& p, hipStream_t s) { return getrf_t<float>(p, s); }
hipError_t blocked_getrs_r32(const Problem& p, hipStream_t s) { return getrs_t<float>(p, s); }
hipError_t blocked_getri_r32(const Problem& p, hipStream_t s) { return getri_t<float>(p, s); }

}  // namespace batchlu
