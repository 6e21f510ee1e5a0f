// chol_kernels.h -- batched Cholesky (potrf), its solve (potrs) and the
// fused factor-and-solve (posv) on gfx950, both triangles.
//
// BatchLAS performance notes, "Blackwell" page (potrf rows of the status
// table: a tiny register tier, a left-looking panel tier and a blocked
// nb / W tier; the LPanel paragraph; posv as potrf plus two triangular
// solves, fused for small orders) and "trsm" page (posv passages);
// redesigned for wave64:
//   register   n <= 64 (complex double: 32): NB lanes of a wavefront hold one
//              matrix, lane i its row i of the lower factor in VGPRs.  Step
//              j publishes column j in LDS; every lane forms the same
//              r = 1/sqrt(d), scales its own entry and publishes it.  posv
//              rides along: the forward solve is fused into the elimination
//              steps, the back solve publishes row k of L per step, and the
//              divisions by the diagonal are spread over the lanes.
//   blocked    n <= 1024, nb = 32, right-looking: one work-group per matrix
//              factors the (n - j0) x 32 panel with one row per thread and
//              one barrier per column (double-buffered column slot); the
//              trailing update A22 -= L21 L21^H runs on MFMA 16x16x4 for the
//              lower tiles only (complex via real MFMAs, each complex k split
//              into two real k' in the order of the four-fma product).
//   solve      n <= 1024: one work-group per matrix and right-hand-side tile,
//              one row per thread: forward with L (true division by l_kk),
//              then back with L^H, a 32-row block at a time.
// Arithmetic per element is the unblocked order: the diagonal and every
// entry accumulate over k in ascending order by fused multiply-adds, l_ij =
// s_ij * (1/l_jj), the solves divide; so the factor and X are bit-identical
// to the plain unblocked computation.  'U' storage is served by the same
// kernels through conjugate-transposed addressing (u_ji = conj(l_ij)); a
// stored diagonal entry is (l_jj, +0) in either triangle.
#pragma once

#include <type_traits>

#include "device_ops.h"
#include "internal.h"

namespace batchlu {

namespace chol {

// ---------------------------------------------------------------------------
// element arithmetic
// ---------------------------------------------------------------------------
template <typename T>
struct cops;

template <typename R>
struct cops_real {
    using T = R;
    static constexpr bool is_complex = false;
    __device__ static R fmar(R a, R b, R c) {
        if constexpr (sizeof(R) == 4) return __builtin_fmaf(a, b, c);
        else return __builtin_fma(a, b, c);
    }
    __device__ static R re(T x) { return x; }
    __device__ static T diag(R x) { return x; }
    __device__ static T scale(T x, R r) { return x * r; }
    __device__ static T divr(T x, R d) { return x / d; }
    __device__ static T cj(T x) { return x; }
    __device__ static T zero() { return R(0); }
    // z -= x * conj(y)
    __device__ static void fms_conj(T& z, T x, T y) { z = fmar(-x, y, z); }
    // z -= x * y
    __device__ static void fms(T& z, T x, T y) { z = fmar(-x, y, z); }
    // z -= conj(x) * y
    __device__ static void fms_cx(T& z, T x, T y) { z = fmar(-x, y, z); }
};

template <typename R>
struct cops_cplx {
    using T = cplx<R>;
    static constexpr bool is_complex = true;
    __device__ static R fmar(R a, R b, R c) {
        if constexpr (sizeof(R) == 4) return __builtin_fmaf(a, b, c);
        else return __builtin_fma(a, b, c);
    }
    __device__ static R re(T x) { return x.re; }
    __device__ static T diag(R x) { return T{x, R(0)}; }
    __device__ static T scale(T x, R r) { return T{x.re * r, x.im * r}; }
    __device__ static T divr(T x, R d) { return T{x.re / d, x.im / d}; }
    __device__ static T cj(T x) { return T{x.re, -x.im}; }
    __device__ static T zero() { return T{R(0), R(0)}; }
    // z -= x * conj(y): re -xr*yr then -xi*yi; im +xr*yi then -xi*yr
    __device__ static void fms_conj(T& z, T x, T y) {
        R r = fmar(-x.re, y.re, z.re);
        r = fmar(-x.im, y.im, r);
        R i = fmar(x.re, y.im, z.im);
        i = fmar(-x.im, y.re, i);
        z = T{r, i};
    }
    // z -= x * y: re -xr*yr then +xi*yi; im -xr*yi then -xi*yr
    __device__ static void fms(T& z, T x, T y) {
        R r = fmar(-x.re, y.re, z.re);
        r = fmar(x.im, y.im, r);
        R i = fmar(-x.re, y.im, z.im);
        i = fmar(-x.im, y.re, i);
        z = T{r, i};
    }
    // z -= conj(x) * y: re -xr*yr then -xi*yi; im -xr*yi then +xi*yr
    __device__ static void fms_cx(T& z, T x, T y) {
        R r = fmar(-x.re, y.re, z.re);
        r = fmar(-x.im, y.im, r);
        R i = fmar(-x.re, y.im, z.im);
        i = fmar(x.im, y.re, i);
        z = T{r, i};
    }
};

template <> struct cops<float> : cops_real<float> { using R = float; };
template <> struct cops<double> : cops_real<double> { using R = double; };
template <> struct cops<cplx<float>> : cops_cplx<float> { using R = float; };
template <> struct cops<cplx<double>> : cops_cplx<double> { using R = double; };

template <typename R>
__device__ inline R sqrt_r(R x) {
    if constexpr (sizeof(R) == 4) return __builtin_sqrtf(x);
    else return __builtin_sqrt(x);
}

// Element (i, k) of the working lower factor L of matrix base M: for 'L' it
// is M[i + k lda], for 'U' conj(M[k + i lda]).  Stores invert that; a
// diagonal entry is stored as is (its imaginary part is +0).
template <typename T>
__device__ inline T ld_elem(const T* M, long long lda, bool up, int i, int k) {
    if (!up) return M[i + k * lda];
    return cops<T>::cj(M[k + i * lda]);
}
template <typename T>
__device__ inline void st_elem(T* M, long long lda, bool up, int i, int k, T v) {
    if (!up) M[i + k * lda] = v;
    else M[k + i * lda] = (i == k) ? v : cops<T>::cj(v);
}

__device__ inline void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// register tier: potrf (NR = 0) or posv (NR right-hand sides, padded)
// ---------------------------------------------------------------------------
constexpr int kRegWaves = 4;

// Float at NB = 32 (two matrices per wavefront) is budgeted for five
// wavefronts per SIMD: left alone the compiler takes 98 VGPRs for the
// nrhs-8 kernel (four per SIMD); with the hint it needs 76 (six) with no
// spill, and posv n = 32, batch 32768 runs 3 - 16 % faster (nrhs 8: 0.220
// -> 0.203 ms).  Elsewhere the hint spilled (NB = 64) or was not needed.
template <typename T, int NB, int NR>
constexpr int chol_reg_waves() { return (sizeof(T) == 4 && NB == 32) ? 5 : 1; }

template <typename T, int NB, int NR>
__global__ void __launch_bounds__(64 * kRegWaves) __attribute__((amdgpu_waves_per_eu(chol_reg_waves<T, NB, NR>())))
chol_reg_kernel(Problem p)
{
    using O = cops<T>;
    using R = typename O::R;
    constexpr int GPW = 64 / NB;                   // matrices per wavefront
    constexpr int GPB = GPW * kRegWaves;           // matrices per block
    constexpr int NRP = NR > 0 ? NR : 1;
    constexpr int QPL = (NRP + NB - 1) / NB;       // right-hand sides divided per lane
    __shared__ T colbuf[GPB][NB];                  // column j (unscaled) / row k of L
    __shared__ T lbuf[GPB][NB];                    // column j scaled: l_kj
    __shared__ T ybuf[GPB][NRP];                   // b_j (or y_k) before its division
    __shared__ T xbuf[GPB][NRP];                   // y_j (or x_k) after it

    const int lane = threadIdx.x & 63;
    const int grp = (threadIdx.x >> 6) * GPW + lane / NB;
    const int li = lane % NB;                      // this lane's row
    const int n = p.n;
    const bool up = p.upper;

    long long m = (long long)blockIdx.x * GPB + grp;
    const bool live = m < p.batch;
    if (!live) m = p.batch - 1;   // idle groups factor a copy and store nothing

    T* A = (T*)p.A + m * p.sA;
    T* B = (T*)p.B + m * p.sB;
    const long long lda = p.lda, ldb = p.ldb;
    const bool have = li < n;

    // load row li of L (lower triangle only; identity past n)
    T a[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k)
        a[k] = (have && k <= li) ? ld_elem(A, lda, up, li, k) : (k == li ? O::diag(R(1)) : O::zero());
    T b[NRP];
#pragma unroll
    for (int r = 0; r < NRP; ++r) b[r] = (NR > 0 && have && r < p.nrhs) ? B[li + r * ldb] : O::zero();

    int info = 0;
    T* col = &colbuf[grp][0];
    T* lcol = &lbuf[grp][0];
    T* yb = &ybuf[grp][0];
    T* xb = &xbuf[grp][0];
    // Step j: lanes at or below the diagonal publish column j unscaled (and
    // lane j its right-hand-side row); every lane forms the same l_jj and
    // r = 1/l_jj; each lane scales its own entry and publishes it, and the
    // divisions y_j = b_j / l_jj are spread over the group's lanes; then the
    // rows below update with the scaled column and y_j.
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        if (j >= n) continue;   // uniform; a guard, not a break, keeps the loop unrolled
        if (li >= j) col[li] = a[j];
        if constexpr (NR > 0) {
            if (li == j)
#pragma unroll
                for (int q = 0; q < NR; ++q) yb[q] = b[q];
        }
        wave_sync();
        const R d = O::re(col[j]);
        const bool ok = d > R(0);
        if (!ok && info == 0) info = j + 1;
        const R ljj = sqrt_r(d);
        const R r = R(1) / ljj;
        if (li == j) a[j] = O::diag(ok ? ljj : d);
        else if (li > j) {
            a[j] = O::scale(a[j], r);
            lcol[li] = a[j];
        }
        if constexpr (NR > 0) {
#pragma unroll
            for (int t = 0; t < QPL; ++t) {
                const int q = li + NB * t;
                if (q < NR) xb[q] = O::divr(yb[q], ljj);
            }
        }
        wave_sync();
        if (li > j) {
#pragma unroll
            for (int k = j + 1; k < NB; ++k) O::fms_conj(a[k], a[j], lcol[k]);
            if constexpr (NR > 0) {
#pragma unroll
                for (int q = 0; q < NR; ++q) O::fms(b[q], a[j], xb[q]);
            }
        } else if constexpr (NR > 0) {
            if (li == j)
#pragma unroll
                for (int q = 0; q < NR; ++q) b[q] = xb[q];
        }
        wave_sync();
    }

    // back solve with L^H: x_k = y_k / l_kk (spread over the lanes), then
    // y_i -= conj(l_ki) x_k for the rows above
    if constexpr (NR > 0) {
#pragma unroll
        for (int k = NB - 1; k >= 0; --k) {
            if (k >= n) continue;
            if (li == k) {
#pragma unroll
                for (int q = 0; q < NR; ++q) yb[q] = b[q];
#pragma unroll
                for (int c = 0; c <= k; ++c) col[c] = a[c];
            }
            wave_sync();
            const R lkk = O::re(col[k]);
#pragma unroll
            for (int t = 0; t < QPL; ++t) {
                const int q = li + NB * t;
                if (q < NR) xb[q] = O::divr(yb[q], lkk);
            }
            wave_sync();
            if (li < k) {
                const T lki = col[li];
#pragma unroll
                for (int q = 0; q < NR; ++q) O::fms_cx(b[q], lki, xb[q]);
            } else if (li == k) {
#pragma unroll
                for (int q = 0; q < NR; ++q) b[q] = xb[q];
            }
            wave_sync();
        }
    }

    if (!live) return;
    if (have) {
#pragma unroll
        for (int k = 0; k < NB; ++k)
            if (k <= li) st_elem(A, lda, up, li, k, a[k]);
        if constexpr (NR > 0) {
            if (info == 0)
#pragma unroll
                for (int r = 0; r < NR; ++r)
                    if (r < p.nrhs) B[li + r * ldb] = b[r];
        }
    }
    if (li == 0) p.info[m] = info;
}

// ---------------------------------------------------------------------------
// blocked tier: panel
// ---------------------------------------------------------------------------
constexpr int NBP = 32;

// threads per panel work-group (one row each): the panel rows of complex
// double need 128 VGPRs, so that type stops at 512 rows
template <typename T>
constexpr int panel_max_rows() { return sizeof(T) == 16 ? 512 : 1024; }

template <typename T>
__global__ void __launch_bounds__(panel_max_rows<T>()) chol_panel_kernel(Problem p, int j0, int w)
{
    using O = cops<T>;
    using R = typename O::R;
    __shared__ T colbuf[2][NBP];
    const long long mat = blockIdx.x;
    if (j0 > 0 && p.info[mat] != 0) return;       // failed in an earlier panel
    const int t = threadIdx.x;
    const int m = p.n - j0;                        // panel height
    const bool up = p.upper;
    const long long lda = p.lda;
    T* D = (T*)p.A + mat * p.sA + j0 + j0 * lda;   // panel origin (same for both triangles)
    const bool have = t < m;

    T a[NBP];
#pragma unroll
    for (int c = 0; c < NBP; ++c)
        a[c] = (have && c < w && c <= t) ? ld_elem(D, lda, up, t, c) : O::zero();

    int fail = -1;
#pragma unroll
    for (int jj = 0; jj < NBP; ++jj) {
        if (jj >= w || fail >= 0) continue;       // uniform guards (no break: the loop stays unrolled)
        T* cb = colbuf[jj & 1];
        if (t < w && t >= jj) cb[t] = a[jj];
        lds_barrier();
        const R d = O::re(cb[jj]);
        if (!(d > R(0))) {                        // uniform: every thread read the same d
            if (t == jj) a[jj] = O::diag(d);
            fail = jj;
            continue;
        }
        const R ljj = sqrt_r(d);
        const R r = R(1) / ljj;
        if (t == jj) a[jj] = O::diag(ljj);
        else if (t > jj) {
            a[jj] = O::scale(a[jj], r);
#pragma unroll
            for (int c = jj + 1; c < NBP; ++c)
                if (c < w) O::fms_conj(a[c], a[jj], O::scale(cb[c], r));
        }
    }
    // the panel's columns (up to the failing one) back to memory
    const int wdone = fail < 0 ? w : fail + 1;
    if (have)
#pragma unroll
        for (int c = 0; c < NBP; ++c)
            if (c < wdone && c <= t && (c < wdone - 1 || fail < 0 || t == c)) st_elem(D, lda, up, t, c, a[c]);
    if (t == 0 && fail >= 0) p.info[mat] = j0 + fail + 1;
    if (t == 0 && fail < 0 && j0 == 0) p.info[mat] = 0;
}

// ---------------------------------------------------------------------------
// blocked tier: trailing update A22 -= L21 L21^H, lower tiles only
// (real types).  One work-group per 64-row strip of A22 walks the strip's
// column tiles left to right up to the diagonal tile; the strip's L21 rows
// stay in registers as MFMA operands, the next tile's L21 rows are staged in
// LDS and the next C tile loaded while the current one runs.  Computed as
// C^T += L21c^T (-L21s)^T so that a lane's accumulator holds consecutive
// columns of one row of C.  Elements above the diagonal of the diagonal tile
// are computed and dropped.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

// row inside a 16x16 MFMA output block held by (lane group lk, register r)
template <typename R>
__device__ inline int mfma_row(int lk, int r) {
    return sizeof(R) == 4 ? 4 * lk + r : lk + 4 * r;
}

// Work-group -> (matrix, part) for grids of `per` work-groups per matrix.
// Work-groups are dealt to the eight XCDs in turn; when the batch is a
// multiple of eight, the parts of one matrix go to one XCD, so the data they
// share (the panel, the factor) comes through one L2.
__device__ inline void chol_part_of(int per, long long& mat, int& part) {
    const unsigned b = blockIdx.x, batch = gridDim.x / (unsigned)per;
    if (per > 1 && (batch & 7) == 0) {
        const unsigned slot = b >> 3;
        mat = (long long)(slot / (unsigned)per) * 8 + (b & 7);
        part = (int)(slot % (unsigned)per);
    } else {
        mat = b / (unsigned)per;
        part = (int)(b % (unsigned)per);
    }
}

template <typename T>
__global__ void __launch_bounds__(256) chol_syrk_kernel(Problem p, int j0, int mstrips)
{
    using O = cops<T>;
    using V = typename std::conditional<sizeof(T) == 4, f32x4, f64x4>::type;
    constexpr int UPAD = 64 + (sizeof(T) == 4 ? 4 : 2);
    __shared__ __attribute__((aligned(16))) T Us[2][NBP][UPAD];
    const int tid = threadIdx.x;
    long long mat;
    int r0;
    chol_part_of(mstrips, mat, r0);
    r0 *= 64;
    if (p.info[mat] != 0) return;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave & 1, wc = wave >> 1;
    const int li = lane & 15, lk = lane >> 4;
    const bool up = p.upper;
    const long long lda = p.lda;
    T* base = (T*)p.A + mat * p.sA;
    const int M = p.n - j0 - NBP;                                    // order of A22
    T* Lp = base + (j0 + NBP) + (long long)j0 * lda;                 // L21 ('L' view origin)
    T* Lu = base + j0 + (long long)(j0 + NBP) * lda;                 // L21 ('U' storage origin)
    T* Cp = base + (j0 + NBP) + (long long)(j0 + NBP) * lda;         // A22
    const int nct = r0 / 64 + 1;
    auto l21 = [&](int i, int k) -> T { return up ? O::cj(Lu[k + (long long)i * lda]) : Lp[i + (long long)k * lda]; };
    // a tile of 64 L21 rows (c) x 32 columns (k) into the stage, as U[k][c]
    auto load_u = [&](int ct, T (&v)[8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = tid + 256 * u;
            const int k = up ? (e & (NBP - 1)) : (e >> 6), c = up ? (e >> 5) : (e & 63);
            const int cc = ct * 64 + c;
            v[u] = cc < M ? l21(cc, k) : O::zero();
        }
    };
    auto put_u = [&](int b, const T (&v)[8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = tid + 256 * u;
            const int k = up ? (e & (NBP - 1)) : (e >> 6), c = up ? (e >> 5) : (e & 63);
            Us[b][k][c] = v[u];
        }
    };
    {
        T v[8];
        load_u(0, v);
        put_u(0, v);
    }
    // this wavefront's L21 rows, negated
    T lv[2][NBP / 4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int i = r0 + wr * 32 + t * 16 + li;
#pragma unroll
        for (int s2 = 0; s2 < NBP / 4; ++s2) lv[t][s2] = i < M ? -l21(i, 4 * s2 + lk) : O::zero();
    }
    auto cat = [&](int i, int j) -> T* { return up ? &Cp[j + (long long)i * lda] : &Cp[i + (long long)j * lda]; };
    auto load_c = [&](int ct, V (&c)[2][2]) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = r0 + wr * 32 + t * 16 + li;
                    const int j = ct * 64 + wc * 32 + b * 16 + mfma_row<T>(lk, r);
                    c[t][b][r] = (i < M && j <= i) ? *cat(i, j) : O::zero();
                }
    };
    __syncthreads();
    V cc[2][2];
    load_c(0, cc);
#pragma unroll 1
    for (int ct = 0; ct < nct; ++ct) {
        const int buf = ct & 1;
        T un[8];
        V cn[2][2];
        const bool more = ct + 1 < nct;
        if (more) {
            load_u(ct + 1, un);
            load_c(ct + 1, cn);
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            T uv[NBP / 4];
#pragma unroll
            for (int s2 = 0; s2 < NBP / 4; ++s2) uv[s2] = Us[buf][4 * s2 + lk][wc * 32 + b * 16 + li];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                V acc = cc[t][b];
#pragma unroll
                for (int s2 = 0; s2 < NBP / 4; ++s2) {
                    if constexpr (sizeof(T) == 4)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(uv[s2], lv[t][s2], acc, 0, 0, 0);
                    else
                        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(uv[s2], lv[t][s2], acc, 0, 0, 0);
                }
                const int i = r0 + wr * 32 + t * 16 + li;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = ct * 64 + wc * 32 + b * 16 + mfma_row<T>(lk, r);
                    if (i < M && j <= i) *cat(i, j) = acc[r];
                }
            }
        }
        if (more) {
            put_u(buf ^ 1, un);
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int b = 0; b < 2; ++b) cc[t][b] = cn[t][b];
        }
        __syncthreads();
    }
}

// Complex trailing update A22 -= L21 L21^H on real MFMAs.  z -= x conj(y)
// is four real fmas (re: -xr*yr then -xi*yi; im: +xr*yi then -xi*yr); each
// complex k becomes two real k' = 2k + h, so that
//   re: sum over k' of Ur[c][k'] * Lr[k'][i], Ur = (y.re, y.im), Lr = (-x.re, -x.im)
//   im: sum over k' of Ui[c][k'] * Li[k'][i], Ui = (y.im, y.re), Li = (x.re, -x.im)
// and an MFMA chain in ascending k' accumulates like fused multiply-adds in
// k' order.  Strips of 32*TB rows, the same walk as the real kernel.
template <typename R>
struct HerkStrip {
    static constexpr int TB = sizeof(R) == 4 ? 2 : 1;   // 16-row blocks per wavefront
    static constexpr int SH = 32 * TB;                   // strip height
};

template <typename R>
__global__ void __launch_bounds__(256) chol_herk_kernel(Problem p, int j0, int mstrips)
{
    using T = cplx<R>;
    using O = cops<T>;
    using V = typename std::conditional<sizeof(R) == 4, f32x4, f64x4>::type;
    constexpr int TB = HerkStrip<R>::TB, SH = HerkStrip<R>::SH;
    constexpr int KP = 2 * NBP;
    constexpr int UPAD = 64 + (sizeof(R) == 4 ? 2 : 1);
    __shared__ __attribute__((aligned(16))) T Us[2][NBP][UPAD];
    const int tid = threadIdx.x;
    long long mat;
    int r0;
    chol_part_of(mstrips, mat, r0);
    r0 *= SH;
    if (p.info[mat] != 0) return;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave & 1, wc = wave >> 1;
    const int li = lane & 15, lk = lane >> 4;
    const bool hodd = (lk & 1) != 0;
    const bool up = p.upper;
    const long long lda = p.lda;
    T* base = (T*)p.A + mat * p.sA;
    const int M = p.n - j0 - NBP;
    T* Lp = base + (j0 + NBP) + (long long)j0 * lda;
    T* Lu = base + j0 + (long long)(j0 + NBP) * lda;
    T* Cp = base + (j0 + NBP) + (long long)(j0 + NBP) * lda;
    const int nct = (r0 + SH - 1) / 64 + 1;
    auto l21 = [&](int i, int k) -> T { return up ? O::cj(Lu[k + (long long)i * lda]) : Lp[i + (long long)k * lda]; };
    auto load_u = [&](int ct, T (&v)[8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = tid + 256 * u;
            const int k = up ? (e & (NBP - 1)) : (e >> 6), c = up ? (e >> 5) : (e & 63);
            const int cc = ct * 64 + c;
            v[u] = cc < M ? l21(cc, k) : O::zero();
        }
    };
    auto put_u = [&](int b, const T (&v)[8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = tid + 256 * u;
            const int k = up ? (e & (NBP - 1)) : (e >> 6), c = up ? (e >> 5) : (e & 63);
            Us[b][k][c] = v[u];
        }
    };
    {
        T v[8];
        load_u(0, v);
        put_u(0, v);
    }
    // lane (li, lk) holds row i at k' = 4 s2 + lk: complex k = 2 s2 + lk / 2
    R lre[TB][KP / 4], lim[TB][KP / 4];
#pragma unroll
    for (int t = 0; t < TB; ++t) {
        const int i = r0 + wr * 16 * TB + t * 16 + li;
#pragma unroll
        for (int s2 = 0; s2 < KP / 4; ++s2) {
            const int k = 2 * s2 + (lk >> 1);
            const T x = i < M ? l21(i, k) : O::zero();
            lre[t][s2] = hodd ? -x.im : -x.re;
            lim[t][s2] = hodd ? -x.im : x.re;
        }
    }
    auto cat = [&](int i, int j) -> T* { return up ? &Cp[j + (long long)i * lda] : &Cp[i + (long long)j * lda]; };
    auto load_c = [&](int ct, V (&cr)[TB][2], V (&ci)[TB][2]) {
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = r0 + wr * 16 * TB + t * 16 + li;
                    const int j = ct * 64 + wc * 32 + b * 16 + mfma_row<R>(lk, r);
                    T z = O::zero();
                    if (i < M && j <= i) {
                        z = *cat(i, j);
                        if (up) z = O::cj(z);
                    }
                    cr[t][b][r] = z.re;
                    ci[t][b][r] = z.im;
                }
    };
    __syncthreads();
    V cr[TB][2], ci[TB][2];
    load_c(0, cr, ci);
#pragma unroll 1
    for (int ct = 0; ct < nct; ++ct) {
        const int buf = ct & 1;
        T un[8];
        V nr[TB][2], ni[TB][2];
        const bool more = ct + 1 < nct;
        if (more) {
            load_u(ct + 1, un);
            load_c(ct + 1, nr, ni);
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int c = wc * 32 + b * 16 + li;
            R ur[KP / 4], ui[KP / 4];
#pragma unroll
            for (int s2 = 0; s2 < KP / 4; ++s2) {
                const T y = Us[buf][2 * s2 + (lk >> 1)][c];
                ur[s2] = hodd ? y.im : y.re;
                ui[s2] = hodd ? y.re : y.im;
            }
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                V accr = cr[t][b], acci = ci[t][b];
#pragma unroll
                for (int s2 = 0; s2 < KP / 4; ++s2) {
                    if constexpr (sizeof(R) == 4) {
                        accr = __builtin_amdgcn_mfma_f32_16x16x4f32(ur[s2], lre[t][s2], accr, 0, 0, 0);
                        acci = __builtin_amdgcn_mfma_f32_16x16x4f32(ui[s2], lim[t][s2], acci, 0, 0, 0);
                    } else {
                        accr = __builtin_amdgcn_mfma_f64_16x16x4f64(ur[s2], lre[t][s2], accr, 0, 0, 0);
                        acci = __builtin_amdgcn_mfma_f64_16x16x4f64(ui[s2], lim[t][s2], acci, 0, 0, 0);
                    }
                }
                const int i = r0 + wr * 16 * TB + t * 16 + li;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = ct * 64 + wc * 32 + b * 16 + mfma_row<R>(lk, r);
                    if (i < M && j <= i) {
                        const T z{accr[r], acci[r]};
                        *cat(i, j) = up ? O::cj(z) : z;
                    }
                }
            }
        }
        if (more) {
            put_u(buf ^ 1, un);
#pragma unroll
            for (int t = 0; t < TB; ++t)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    cr[t][b] = nr[t][b];
                    ci[t][b] = ni[t][b];
                }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// solve A X = B with the factor: one work-group per matrix and tile of NRT
// right-hand sides, one row per thread (n <= 1024).  Forward L y = b: the
// wavefront holding a 32-row block solves it (lane c divides by l_cc, the
// value is broadcast by readlane), publishes the block's y in LDS, and after
// one barrier every lower row subtracts l_ik y_k for the block's k in
// ascending order.  Back L^H x = y: blocks descending, the same with
// conj(l_ki) and k descending.  Skips matrices with info != 0 when p.info is
// set (posv keeps B there).
// ---------------------------------------------------------------------------
constexpr int BS = 32;

// x_k = y_k / l_kk for the NRT right-hand sides held by diagonal lane dl,
// broadcast in xc (lane dl keeps them in y): lane r divides right-hand side
// r by the broadcast real diagonal (the same operands, so the same bits), so
// the wavefront pays for one division per step rather than NRT.
template <typename O, typename T, int NRT>
__device__ inline void chol_diag_divide(T (&y)[NRT], T (&xc)[NRT], typename O::R diag, int dl, int lane) {
    T yc[NRT];
#pragma unroll
    for (int r = 0; r < NRT; ++r) yc[r] = readlane_t(y[r], dl);
    const typename O::R d = readlane_t(diag, dl);
    T v = yc[0];
#pragma unroll
    for (int r = 1; r < NRT; ++r)
        if (lane == r) v = yc[r];
    const T q = O::divr(v, d);
#pragma unroll
    for (int r = 0; r < NRT; ++r) xc[r] = readlane_t(q, r);
    if (lane == dl)
#pragma unroll
        for (int r = 0; r < NRT; ++r) y[r] = xc[r];
}

template <typename T, int NRT>
__global__ void __launch_bounds__(1024) chol_solve_kernel(Problem p, int rtiles)
{
    using O = cops<T>;
    __shared__ T ybuf[2][BS][NRT];
    const int n = p.n;
    long long m;
    int c0;
    chol_part_of(rtiles, m, c0);
    c0 *= NRT;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    if (p.info && p.info[m] != 0) return;
    const bool up = p.upper;
    const long long lda = p.lda;
    const T* F = (const T*)p.A + m * p.sA;
    T* B = (T*)p.B + m * p.sB;
    const int row = tid;
    const bool have = row < n;
    T y[NRT];
#pragma unroll
    for (int r = 0; r < NRT; ++r) y[r] = (have && c0 + r < p.nrhs) ? B[row + (long long)(c0 + r) * p.ldb] : O::zero();
    const int P = (n + BS - 1) / BS;
    // forward
    for (int kb = 0; kb < P; ++kb) {
        const int r0 = kb * BS;
        const int w = min(BS, n - r0);
        T(*yb)[NRT] = ybuf[kb & 1];
        if (wave == r0 / 64) {
            const int base = r0 % 64;
            const int mrow = lane - base;
            const bool inb = mrow >= 0 && mrow < w;
            T lrow[BS];
#pragma unroll
            for (int c = 0; c < BS; ++c)
                lrow[c] = (inb && c <= mrow) ? ld_elem(F, lda, up, row, r0 + c) : O::zero();
#pragma unroll
            for (int c = 0; c < BS; ++c) {
                if (c >= w) continue;
                T xc[NRT];
                if constexpr (NRT == 1) {
                    if (mrow == c) y[0] = O::divr(y[0], O::re(lrow[c]));
                    xc[0] = readlane_t(y[0], base + c);
                } else {
                    chol_diag_divide<O>(y, xc, O::re(lrow[c]), base + c, lane);
                }
                if (inb && mrow > c)
#pragma unroll
                    for (int r = 0; r < NRT; ++r) O::fms(y[r], lrow[c], xc[r]);
            }
            if (inb)
#pragma unroll
                for (int r = 0; r < NRT; ++r) yb[mrow][r] = y[r];
        }
        __syncthreads();
        if (have && row >= r0 + w) {
#pragma unroll 4
            for (int c = 0; c < w; ++c) {
                const T l = ld_elem(F, lda, up, row, r0 + c);
#pragma unroll
                for (int r = 0; r < NRT; ++r) O::fms(y[r], l, yb[c][r]);
            }
        }
    }
    __syncthreads();
    // back with L^H
    for (int kb = P - 1; kb >= 0; --kb) {
        const int r0 = kb * BS;
        const int w = min(BS, n - r0);
        T(*yb)[NRT] = ybuf[kb & 1];
        if (wave == r0 / 64) {
            const int base = r0 % 64;
            const int mrow = lane - base;
            const bool inb = mrow >= 0 && mrow < w;
            // lcol[c] = l_{r0+c, row}: column `row` of L inside the block
            T lcol[BS];
#pragma unroll
            for (int c = 0; c < BS; ++c)
                lcol[c] = (inb && c >= mrow && c < w) ? ld_elem(F, lda, up, r0 + c, row) : O::zero();
#pragma unroll
            for (int c = BS - 1; c >= 0; --c) {
                if (c >= w) continue;
                T xc[NRT];
                if constexpr (NRT == 1) {
                    if (mrow == c) y[0] = O::divr(y[0], O::re(lcol[c]));
                    xc[0] = readlane_t(y[0], base + c);
                } else {
                    chol_diag_divide<O>(y, xc, O::re(lcol[c]), base + c, lane);
                }
                if (inb && mrow < c)
#pragma unroll
                    for (int r = 0; r < NRT; ++r) O::fms_cx(y[r], lcol[c], xc[r]);
            }
            if (inb)
#pragma unroll
                for (int r = 0; r < NRT; ++r) yb[mrow][r] = y[r];
        }
        __syncthreads();
        if (have && row < r0) {
#pragma unroll 4
            for (int c = w - 1; c >= 0; --c) {
                const T l = ld_elem(F, lda, up, r0 + c, row);
#pragma unroll
                for (int r = 0; r < NRT; ++r) O::fms_cx(y[r], l, yb[c][r]);
            }
        }
    }
    if (have)
#pragma unroll
        for (int r = 0; r < NRT; ++r)
            if (c0 + r < p.nrhs) B[row + (long long)(c0 + r) * p.ldb] = y[r];
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <typename T>
constexpr int reg_max_n() { return sizeof(T) == 16 ? 32 : 64; }

template <typename T, int NB, int NR>
hipError_t launch_reg_nb(const Problem& p, hipStream_t s) {
    constexpr int GPB = (64 / NB) * kRegWaves;
    const dim3 grid((unsigned)((p.batch + GPB - 1) / GPB));
    hipLaunchKernelGGL((chol_reg_kernel<T, NB, NR>), grid, dim3(64 * kRegWaves), 0, s, p);
    return hipGetLastError();
}

template <typename T, int NR>
hipError_t launch_reg_nr(const Problem& p, hipStream_t s) {
    if (p.n <= 8) return launch_reg_nb<T, 8, NR>(p, s);
    if (p.n <= 16) return launch_reg_nb<T, 16, NR>(p, s);
    if (p.n <= 32) return launch_reg_nb<T, 32, NR>(p, s);
    if constexpr (reg_max_n<T>() >= 64) return launch_reg_nb<T, 64, NR>(p, s);
    return hipErrorInvalidValue;
}

// posv fused when nrhs <= 16; nrhs == 0 factors only
template <typename T>
hipError_t launch_reg(const Problem& p, bool solve, hipStream_t s) {
    if (p.n < 1 || p.n > reg_max_n<T>()) return hipErrorInvalidValue;
    if (!solve) return launch_reg_nr<T, 0>(p, s);
    if (p.nrhs <= 1) return launch_reg_nr<T, 1>(p, s);
    if (p.nrhs <= 8) return launch_reg_nr<T, 8>(p, s);
    if (p.nrhs <= 16) return launch_reg_nr<T, 16>(p, s);
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_potrf_blocked(const Problem& p, hipStream_t s) {
    const int n = p.n;
    if (n < 1 || n > panel_max_rows<T>()) return hipErrorInvalidValue;
    hipError_t e;
    for (int j0 = 0; j0 < n; j0 += NBP) {
        const int w = min(NBP, n - j0);
        const int threads = ((n - j0 + 63) / 64) * 64;
        hipLaunchKernelGGL((chol_panel_kernel<T>), dim3((unsigned)p.batch), dim3(threads), 0, s, p, j0, w);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int M = n - j0 - NBP;
        if (M <= 0) break;
        if constexpr (cops<T>::is_complex) {
            using R = typename cops<T>::R;
            constexpr int SH = HerkStrip<R>::SH;
            const int ms = (M + SH - 1) / SH;
            hipLaunchKernelGGL((chol_herk_kernel<R>), dim3((unsigned)((long long)ms * p.batch)), dim3(256), 0, s,
                               p, j0, ms);
        } else {
            const int ms = (M + 63) / 64;
            hipLaunchKernelGGL((chol_syrk_kernel<T>), dim3((unsigned)((long long)ms * p.batch)), dim3(256), 0, s,
                               p, j0, ms);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T, int NRT>
hipError_t launch_solve_nrt(const Problem& p, hipStream_t s) {
    const int threads = ((p.n + 63) / 64) * 64;
    const int rt = (p.nrhs + NRT - 1) / NRT;
    hipLaunchKernelGGL((chol_solve_kernel<T, NRT>), dim3((unsigned)((long long)p.batch * rt)), dim3(threads), 0, s,
                       p, rt);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_solve(const Problem& p, hipStream_t s) {
    if (p.n < 1 || p.n > 1024) return hipErrorInvalidValue;
    if (p.nrhs <= 1) return launch_solve_nrt<T, 1>(p, s);
    if constexpr (sizeof(T) == 16) return launch_solve_nrt<T, 2>(p, s);
    else return launch_solve_nrt<T, 4>(p, s);
}

}  // namespace chol

}  // namespace batchlu
