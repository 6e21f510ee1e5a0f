// blocked_lu.cpp -- host dispatch of the blocked tier (the kernels and the
// per-panel launch sequence are in blocked_lu_impl.h, instantiated once per
// data type in blocked_lu_{r32,r64,c64,c128}.hip).
#include "internal.h"

namespace batchlu {

hipError_t blocked_getrf_r32(const Problem& p, hipStream_t s);
hipError_t blocked_getrf_r64(const Problem& p, hipStream_t s);
hipError_t blocked_getrf_c64(const Problem& p, hipStream_t s);
hipError_t blocked_getrf_c128(const Problem& p, hipStream_t s);
hipError_t blocked_getrs_r32(const Problem& p, hipStream_t s);
hipError_t blocked_getrs_r64(const Problem& p, hipStream_t s);
hipError_t blocked_getrs_c64(const Problem& p, hipStream_t s);
hipError_t blocked_getrs_c128(const Problem& p, hipStream_t s);

bool blocked_supported(int dtype, int n) {
    // the largest orders the parity tests run: float and double 2048, the
    // complex types 1024 (double panels above 1024 rows and complex double
    // panels above 512 rows hold four rows per thread and spill registers:
    // correct, slower)
    const int cap = (dtype == R32 || dtype == R64) ? 2048 : 1024;
    return n >= 1 && n <= cap;
}

hipError_t blocked_getrf(int dtype, const Problem& p, hipStream_t s) {
    if (!blocked_supported(dtype, p.n)) return hipErrorInvalidValue;
    // real orders up to 256: the whole blocked sequence in one work-group
    if (blocked_fused_supported(dtype, p.n, p.lda)) return blocked_fused_getrf(dtype, p, s);
    switch (dtype) {
    case R32: return blocked_getrf_r32(p, s);
    case R64: return blocked_getrf_r64(p, s);
    case C64: return blocked_getrf_c64(p, s);
    case C128: return blocked_getrf_c128(p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t blocked_getrs(int dtype, const Problem& p, hipStream_t s) {
    if (!blocked_supported(dtype, p.n)) return hipErrorInvalidValue;
    switch (dtype) {
    case R32: return blocked_getrs_r32(p, s);
    case R64: return blocked_getrs_r64(p, s);
    case C64: return blocked_getrs_c64(p, s);
    case C128: return blocked_getrs_c128(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace batchlu
