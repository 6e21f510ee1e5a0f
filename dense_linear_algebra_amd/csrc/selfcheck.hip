// selfcheck.hip -- device self-check of the fast float reciprocal that the
// register tiers use for pivots (one v_rcp_f32 and one Newton step in place
// of a division, after the Blackwell page's getrs tiny paragraph: one
// reciprocal per pivot instead of a divide per element).  The tiers rely on
// it returning exactly the correctly rounded 1/x inside the range where
// recip_fast_ok() holds; this kernel compares the two for every float bit
// pattern of a given range and counts the differences.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/batchlu.h"
#include "device_ops.h"

namespace batchlu {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 64;   // consecutive bit patterns per thread

__global__ void __launch_bounds__(kThreads) reciprocal_check_kernel(uint32_t lo, uint64_t count,
                                                                    unsigned long long* mismatches,
                                                                    uint32_t* first_bad)
{
    const uint64_t start = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) * kPerThread;
    unsigned bad = 0;
    uint32_t first = 0xffffffffu;
    for (int k = 0; k < kPerThread; ++k) {
        const uint64_t idx = start + (uint64_t)k;
        if (idx >= count) break;
        const uint32_t bits = lo + (uint32_t)idx;
        const float x = __builtin_bit_cast(float, bits);
        const float want = 1.0f / x;   // IEEE division (no fast-math in this library)
        const float ax = __builtin_fabsf(x);
        // inside the fast range the fast form must give the same bits; outside
        // it the callers divide, so only the range test is checked there
        const bool ok = recip_fast_ok(ax);
        const bool differs = ok && __builtin_bit_cast(uint32_t, recip_fast(x)) != __builtin_bit_cast(uint32_t, want);
        if (differs) {
            ++bad;
            if (bits < first) first = bits;
        }
    }
    // one vector atomic per wavefront (lane 0 after a wavefront sum)
    unsigned long long wsum = bad;
    for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);
    uint32_t wfirst = first;
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t o = __shfl_xor(wfirst, off);
        wfirst = o < wfirst ? o : wfirst;
    }
    if ((threadIdx.x & 63) == 0 && wsum != 0) {
        atomicAdd(mismatches, wsum);
        atomicMin(first_bad, wfirst);
    }
}

}  // namespace
}  // namespace batchlu

extern "C" int batchlu_check_reciprocal(unsigned int lo_bits, unsigned int hi_bits,
                                        unsigned long long* mismatches, unsigned int* first_bad,
                                        hipStream_t stream)
{
    if (hi_bits < lo_bits) return -2;
    if (!mismatches) return -3;
    if (!first_bad) return -4;
    const uint64_t count = (uint64_t)hi_bits - lo_bits + 1;
    const uint64_t per_block = (uint64_t)batchlu::kThreads * batchlu::kPerThread;
    const uint64_t blocks = (count + per_block - 1) / per_block;
    hipLaunchKernelGGL(batchlu::reciprocal_check_kernel, dim3((unsigned)blocks), dim3(batchlu::kThreads), 0, stream,
                       (uint32_t)lo_bits, count, mismatches, (uint32_t*)first_bad);
    return hipGetLastError() == hipSuccess ? BATCHLU_OK : BATCHLU_ERR_LAUNCH;
}
