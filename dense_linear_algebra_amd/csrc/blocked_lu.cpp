// blocked_lu.cpp -- host dispatch of the blocked tier (the kernels and the
// per-panel launch sequence are in blocked_lu_impl.h, instantiated once per
// data type in blocked_lu_{r32,r64,c64,c128}.hip).
#include <mutex>

#include "internal.h"

namespace batchlu {

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_la_mutex;
struct LaSlot {
    bool tried = false, ok = false;
    hipStream_t side = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
LaSlot g_la[kMaxDevices];

}  // namespace

bool lookahead_begin(LookAhead& la) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
    g_la_mutex.lock();
    LaSlot& sl = g_la[dev];
    if (!sl.tried) {
        sl.tried = true;
        // default priority; events without timing
        sl.ok = hipStreamCreateWithFlags(&sl.side, hipStreamNonBlocking) == hipSuccess &&
                hipEventCreateWithFlags(&sl.fork, hipEventDisableTiming) == hipSuccess &&
                hipEventCreateWithFlags(&sl.join, hipEventDisableTiming) == hipSuccess;
    }
    if (!sl.ok) {
        g_la_mutex.unlock();
        return false;
    }
    la.side = sl.side;
    la.fork = sl.fork;
    la.join = sl.join;
    la.held = true;
    return true;
}

hipError_t lookahead_fork(LookAhead& la, hipStream_t s) {
    hipError_t e = hipEventRecord(la.fork, s);
    if (e != hipSuccess) return e;
    return hipStreamWaitEvent(la.side, la.fork, 0);
}

hipError_t lookahead_join_record(LookAhead& la) { return hipEventRecord(la.join, la.side); }

hipError_t lookahead_join_wait(LookAhead& la, hipStream_t s) { return hipStreamWaitEvent(s, la.join, 0); }

hipError_t lookahead_end(LookAhead& la, hipError_t status) {
    if (la.held) {
        la.held = false;
        g_la_mutex.unlock();
    }
    return status;
}

hipError_t blocked_getrf_r32(const Problem& p, hipStream_t s);
hipError_t blocked_getrf_r64(const Problem& p, hipStream_t s);
hipError_t blocked_getrf_c64(const Problem& p, hipStream_t s);
hipError_t blocked_getrf_c128(const Problem& p, hipStream_t s);
hipError_t blocked_getrs_r32(const Problem& p, hipStream_t s);
hipError_t blocked_getrs_r64(const Problem& p, hipStream_t s);
hipError_t blocked_getrs_c64(const Problem& p, hipStream_t s);
hipError_t blocked_getrs_c128(const Problem& p, hipStream_t s);
hipError_t blocked_getri_r32(const Problem& p, hipStream_t s);
hipError_t blocked_getri_r64(const Problem& p, hipStream_t s);
hipError_t blocked_getri_c64(const Problem& p, hipStream_t s);
hipError_t blocked_getri_c128(const Problem& p, hipStream_t s);

// Every type to n = 4096: panels taller than the register-resident kernels
// reach stay in memory (the deferred left interchanges hold four rows per
// thread of 1024).
bool blocked_supported(int dtype, int n) {
    (void)dtype;
    return n >= 1 && n <= 4096;
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

// The blocked solve has no register-resident panel; its one bound is the
// row permutation's LDS stage (two int and one element per row).
bool blocked_getrs_supported(int dtype, int n) {
    (void)dtype;
    return n >= 1 && n <= 4096;
}

hipError_t blocked_getrs(int dtype, const Problem& p, hipStream_t s) {
    if (!blocked_getrs_supported(dtype, p.n) || p.trans < 0 || p.trans > 2) return hipErrorInvalidValue;
    if (p.inverse) {
        switch (dtype) {
        case R32: return blocked_getri_r32(p, s);
        case R64: return blocked_getri_r64(p, s);
        case C64: return blocked_getri_c64(p, s);
        case C128: return blocked_getri_c128(p, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (dtype) {
    case R32: return blocked_getrs_r32(p, s);
    case R64: return blocked_getrs_r64(p, s);
    case C64: return blocked_getrs_c64(p, s);
    case C128: return blocked_getrs_c128(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace batchlu
