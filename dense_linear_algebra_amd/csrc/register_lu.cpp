// register_lu.cpp -- host dispatch for the register tiers.
#include "internal.h"

namespace batchlu {

hipError_t register_launch_r32(const Problem& p, int mode, hipStream_t s);
hipError_t register_launch_r64(const Problem& p, int mode, hipStream_t s);
hipError_t register_launch_c64(const Problem& p, int mode, hipStream_t s);
hipError_t register_launch_c128(const Problem& p, int mode, hipStream_t s);

bool register_supported(int dtype, int n, int nrhs, int mode, bool one_wave_per_matrix) {
    if (n < 1) return false;
    const int cap = dtype == C128 ? 32 : 64;
    if (n > cap) return false;
    if (one_wave_per_matrix != (n > 32)) return false;
    if (mode != MODE_GESV) return true;
    return nrhs >= 0 && nrhs <= 16;
}

hipError_t register_launch(int dtype, const Problem& p, int mode, bool one_wave_per_matrix,
                           hipStream_t s) {
    if (!register_supported(dtype, p.n, p.nrhs, mode, one_wave_per_matrix)) return hipErrorInvalidValue;
    switch (dtype) {
    case R32: return register_launch_r32(p, mode, s);
    case R64: return register_launch_r64(p, mode, s);
    case C64: return register_launch_c64(p, mode, s);
    case C128: return register_launch_c128(p, mode, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace batchlu
