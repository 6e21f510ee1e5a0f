// blocked_lu.hip -- blocked right-looking LU (nb = 32) for larger n.
#include "device_ops.h"
#include "internal.h"

namespace batchlu {

bool blocked_supported(int dtype, int n) {
    (void)dtype;
    (void)n;
    return false;
}

hipError_t blocked_getrf(int dtype, const Problem& p, hipStream_t s) {
    (void)dtype; (void)p; (void)s;
    return hipErrorInvalidValue;
}

hipError_t blocked_getrs(int dtype, const Problem& p, hipStream_t s) {
    (void)dtype; (void)p; (void)s;
    return hipErrorInvalidValue;
}

}  // namespace batchlu
