// device_ops.h -- element arithmetic and wavefront exchanges shared by the
// LU kernels (gfx950, wave64).
//
// Element arithmetic (BatchLAS "LU" page, tiny-tier and register-panel
// paragraphs; "GEMM" page, POD complex scalar paragraph):
//   - pivot metric |x| for real, cabs1 = |re| + |im| for complex;
//   - multipliers l = a * r with r = 1/pivot rounded once, or a / pivot when
//     the pivot metric is below the smallest normal;
//   - complex 1/p and a/p by Smith's algorithm, each operation rounded;
//   - a rank-1 update is one fused multiply-add per element and step; for
//     complex z -= x*y it is four real fmas in a fixed order.
// The whole library is built with -ffp-contract=off, so no other product is
// fused behind these spellings.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace batchlu {

template <typename R>
struct cplx {
    R re, im;
};

template <typename T>
struct ops;

template <>
struct ops<float> {
    using R = float;
    using K = uint32_t;
    static constexpr bool is_complex = false;
    __device__ static constexpr R sfmin() { return 1.17549435082228750797e-38f; }
    __device__ static float zero() { return 0.0f; }
    __device__ static float one() { return 1.0f; }
    __device__ static R metric(float x) { return __builtin_fabsf(x); }
    __device__ static float recip(float p) { return 1.0f / p; }
    __device__ static float div(float a, float p) { return a / p; }
    __device__ static float mul(float a, float r) { return a * r; }
    __device__ static void fms(float& z, float x, float y) { z = __builtin_fmaf(-x, y, z); }
};

template <>
struct ops<double> {
    using R = double;
    using K = uint64_t;
    static constexpr bool is_complex = false;
    __device__ static constexpr R sfmin() { return 2.22507385850720138309e-308; }
    __device__ static double zero() { return 0.0; }
    __device__ static double one() { return 1.0; }
    __device__ static R metric(double x) { return __builtin_fabs(x); }
    __device__ static double recip(double p) { return 1.0 / p; }
    __device__ static double div(double a, double p) { return a / p; }
    __device__ static double mul(double a, double r) { return a * r; }
    __device__ static void fms(double& z, double x, double y) { z = __builtin_fma(-x, y, z); }
};

template <typename R, typename KK>
struct complex_ops {
    using T = cplx<R>;
    using K = KK;
    static constexpr bool is_complex = true;
    __device__ static R fabsr(R x) {
        if constexpr (sizeof(R) == 4) return __builtin_fabsf(x);
        else return __builtin_fabs(x);
    }
    __device__ static R fmar(R a, R b, R c) {
        if constexpr (sizeof(R) == 4) return __builtin_fmaf(a, b, c);
        else return __builtin_fma(a, b, c);
    }
    __device__ static T zero() { return T{R(0), R(0)}; }
    __device__ static T one() { return T{R(1), R(0)}; }
    __device__ static R metric(T z) { return fabsr(z.re) + fabsr(z.im); }
    // Smith: 1 / (c + d i)
    __device__ static T recip(T p) {
        R c = p.re, d = p.im;
        if (fabsr(c) >= fabsr(d)) {
            R e = d / c;
            R f = c + d * e;
            return T{R(1) / f, -e / f};
        }
        R e = c / d;
        R f = d + c * e;
        return T{e / f, -R(1) / f};
    }
    // Smith: (a + b i) / (c + d i)
    __device__ static T div(T x, T p) {
        R a = x.re, b = x.im, c = p.re, d = p.im;
        if (fabsr(c) >= fabsr(d)) {
            R e = d / c;
            R f = c + d * e;
            return T{(a + b * e) / f, (b - a * e) / f};
        }
        R e = c / d;
        R f = d + c * e;
        return T{(a * e + b) / f, (b * e - a) / f};
    }
    // l = a * r: re = fma(ar, rr, -(ai*ri)), im = fma(ar, ri, ai*rr)
    __device__ static T mul(T a, T r) {
        R t = a.im * r.im;
        R re = fmar(a.re, r.re, -t);
        R t2 = a.im * r.re;
        R im = fmar(a.re, r.im, t2);
        return T{re, im};
    }
    // z -= x * y: re: -xr*yr then +xi*yi; im: -xr*yi then -xi*yr
    __device__ static void fms(T& z, T x, T y) {
        R re = fmar(-x.re, y.re, z.re);
        re = fmar(x.im, y.im, re);
        R im = fmar(-x.re, y.im, z.im);
        im = fmar(-x.im, y.re, im);
        z.re = re;
        z.im = im;
    }
};

template <>
struct ops<cplx<float>> : complex_ops<float, uint32_t> {
    using R = float;
    __device__ static constexpr R sfmin() { return 1.17549435082228750797e-38f; }
};

template <>
struct ops<cplx<double>> : complex_ops<double, uint64_t> {
    using R = double;
    __device__ static constexpr R sfmin() { return 2.22507385850720138309e-308; }
};

// ---------------------------------------------------------------------------
// 1/x rounded once, fast: v_rcp_f32 and one Newton step.  For every |x| in
// [2^-125, 2^125] this equals the correctly rounded quotient 1/x; the
// library's self-check (batchlu_check_reciprocal) compares the two over every
// float of that range on the device.  Outside the range, callers divide.
// ---------------------------------------------------------------------------
__device__ inline float recip_fast(float x) {
    const float r0 = __builtin_amdgcn_rcpf(x);
    const float e = __builtin_fmaf(-x, r0, 1.0f);
    return __builtin_fmaf(e, r0, r0);
}
__device__ inline bool recip_fast_ok(float ax) { return ax >= 0x1p-125f && ax <= 0x1p125f; }

// ---------------------------------------------------------------------------
// pivot keys: a candidate's key is (bits of its metric) + 1, every NaN
// clamped to the bit pattern just above +inf (so all NaNs tie, above every
// number, and the lowest position among them wins); non-candidates get 0.
// Metrics are >= 0, so unsigned order of the bits is numeric order.
// ---------------------------------------------------------------------------
__device__ inline uint32_t pivot_key(float m) {
    uint32_t b = __builtin_bit_cast(uint32_t, m);
    return (b < 0x7f800001u ? b : 0x7f800001u) + 1u;
}
__device__ inline uint64_t pivot_key(double m) {
    uint64_t b = __builtin_bit_cast(uint64_t, m);
    return (b < 0x7ff0000000000001ull ? b : 0x7ff0000000000001ull) + 1ull;
}

// ---------------------------------------------------------------------------
// v_readlane for every element type (the lane index must be wavefront-uniform)
// ---------------------------------------------------------------------------
__device__ inline float readlane_t(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ inline double readlane_t(double v, int l) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
template <typename R>
__device__ inline cplx<R> readlane_t(cplx<R> v, int l) {
    return cplx<R>{readlane_t(v.re, l), readlane_t(v.im, l)};
}

// ---------------------------------------------------------------------------
// all-reduce over aligned groups of G lanes inside a wave64.  Stage order
// matters: quad_perm swaps (xor 1, xor 2), then row_half_mirror and
// row_mirror (valid once each quad / half row already agrees), then
// ds_swizzle xor 16 inside 32 lanes, then a cross-half bpermute.  The DPP
// stages pass the operation's identity as the "old" value so that the
// compiler folds the move into the max / min (one VALU op per stage).
// ---------------------------------------------------------------------------
template <int STAGE>
__device__ inline uint32_t exchange32(uint32_t v, uint32_t identity) {
    if constexpr (STAGE == 1)
        return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, 0xB1, 0xF, 0xF, false);
    else if constexpr (STAGE == 2)
        return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, 0x4E, 0xF, 0xF, false);
    else if constexpr (STAGE == 4)
        return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, 0x141, 0xF, 0xF, false);
    else if constexpr (STAGE == 8)
        return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, 0x140, 0xF, 0xF, false);
    else if constexpr (STAGE == 16)
        return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);               // xor 16 in 32
    else
        return (uint32_t)__builtin_amdgcn_ds_bpermute((int)((__lane_id() ^ 32) << 2), (int)v);
}

template <int STAGE, typename K>
__device__ inline K exchange_max_operand(K v) {
    if constexpr (sizeof(K) == 8) {
        uint32_t lo = exchange32<STAGE>((uint32_t)v, 0u);
        uint32_t hi = exchange32<STAGE>((uint32_t)((uint64_t)v >> 32), 0u);
        return (K)(((uint64_t)hi << 32) | lo);
    } else {
        return (K)exchange32<STAGE>((uint32_t)v, 0u);
    }
}

template <int G, typename K>
__device__ inline K group_max(K v) {
    if constexpr (G >= 2) { K o = exchange_max_operand<1>(v); v = o > v ? o : v; }
    if constexpr (G >= 4) { K o = exchange_max_operand<2>(v); v = o > v ? o : v; }
    if constexpr (G >= 8) { K o = exchange_max_operand<4>(v); v = o > v ? o : v; }
    if constexpr (G >= 16) { K o = exchange_max_operand<8>(v); v = o > v ? o : v; }
    if constexpr (G >= 32) { K o = exchange_max_operand<16>(v); v = o > v ? o : v; }
    if constexpr (G >= 64) { K o = exchange_max_operand<32>(v); v = o > v ? o : v; }
    return v;
}

template <int G>
__device__ inline int group_min(int v) {
    constexpr uint32_t id = 0x7fffffffu;
    if constexpr (G >= 2) { int o = (int)exchange32<1>((uint32_t)v, id); v = o < v ? o : v; }
    if constexpr (G >= 4) { int o = (int)exchange32<2>((uint32_t)v, id); v = o < v ? o : v; }
    if constexpr (G >= 8) { int o = (int)exchange32<4>((uint32_t)v, id); v = o < v ? o : v; }
    if constexpr (G >= 16) { int o = (int)exchange32<8>((uint32_t)v, id); v = o < v ? o : v; }
    if constexpr (G >= 32) { int o = (int)exchange32<16>((uint32_t)v, id); v = o < v ? o : v; }
    if constexpr (G >= 64) { int o = (int)exchange32<32>((uint32_t)v, id); v = o < v ? o : v; }
    return v;
}

// ---------------------------------------------------------------------------
// wavefront argmax and an LDS-only work-group barrier (blocked-tier panels)
// ---------------------------------------------------------------------------
// maximum over the wavefront, returned wave-uniform: DPP inside each row of
// 16 lanes, then across the rows
__device__ inline uint32_t wave_max(uint32_t v) {
    v = group_max<16>(v);
    // row_bcast:15 hands each even row's maximum to the next row (rows 1 and
    // 3), row_bcast:31 row 1's to rows 2 and 3; lane 63 then holds the
    // wavefront's maximum (disabled rows keep the identity 0 as the operand)
    uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);
    v = o > v ? o : v;
    o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);
    v = o > v ? o : v;
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// 64-bit keys: the high words first, then the low words among the lanes
// that hold the maximal high word
__device__ inline uint64_t wave_max(uint64_t v) {
    const uint32_t hi = (uint32_t)(v >> 32);
    const uint32_t mh = wave_max(hi);
    const uint32_t ml = wave_max(hi == mh ? (uint32_t)v : 0u);
    return ((uint64_t)mh << 32) | ml;
}

// argmax over the wavefront: the maximal key (wave-uniform) and the lane that
// holds it, the lowest position winning among equal keys; win = -1 when no
// lane holds a candidate (every key 0)
__device__ inline void tie_break(bool at_max, int pos, int& win) {
    const int q = group_min<64>(at_max ? pos : 0x7fffffff);
    win = __builtin_ctzll(__builtin_amdgcn_ballot_w64(pos == q));
}
__device__ inline void wave_argmax(uint32_t key, int pos, uint32_t& kmax, int& win) {
    kmax = wave_max(key);
    win = -1;
    if (kmax == 0) return;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(key == kmax);
    win = __builtin_ctzll(hit);
    if (__builtin_expect(__builtin_popcountll(hit) != 1, 0)) tie_break(key == kmax, pos, win);
}
// 64-bit keys: the high words decide unless several lanes share the maximal
// high word; only then are the low words reduced
__device__ inline void wave_argmax(uint64_t key, int pos, uint64_t& kmax, int& win) {
    const uint32_t hi = (uint32_t)(key >> 32);
    const uint32_t mh = wave_max(hi);
    uint64_t hit = __builtin_amdgcn_ballot_w64(hi == mh);
    win = -1;
    if (__builtin_expect(mh != 0 && __builtin_popcountll(hit) == 1, 1)) {
        win = __builtin_ctzll(hit);
        kmax = ((uint64_t)mh << 32) | (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key, win);
        return;
    }
    const uint32_t ml = wave_max(hi == mh ? (uint32_t)key : 0u);
    kmax = ((uint64_t)mh << 32) | ml;
    if (kmax == 0) return;
    hit = __builtin_amdgcn_ballot_w64(key == kmax);
    win = __builtin_ctzll(hit);
    if (__builtin_expect(__builtin_popcountll(hit) != 1, 0)) tie_break(key == kmax, pos, win);
}


// work-group barrier that orders LDS only: global stores still in flight are
// not waited for (used where the next phase reads nothing those stores write)
__device__ inline void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace batchlu
