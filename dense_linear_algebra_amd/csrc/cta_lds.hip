// cta_lds.hip -- the LDS-staged work-group tier: LU with partial pivoting
// (and the fused solve of gesv) of one matrix per work-group, the matrix
// held in LDS.
//
// BatchLAS "LU" page, family table, cta row (a local-memory getf2 whose
// capacity is what fits the local-memory budget at a target occupancy) and
// the gesv rows (factor and solve fused for small n); redesigned for gfx950:
//   - A (n x n) and B (n x nrhs) sit in LDS row-major, row i of [A | B] at
//     i * LDR, so that the threads of a wavefront, one per column, touch
//     consecutive words;
//   - step j: wavefront 0 searches column j (keys as the register tiers:
//     |a| or |re| + |im|, NaN above every number, lowest row on ties), forms
//     r = 1/pivot (Smith's algorithm for complex) and writes the multipliers
//     of column j for the rows as they will stand after the interchange;
//     after one barrier every other column belongs to one thread, which
//     exchanges its two entries of rows j and p and then runs the rank-1
//     update down its column (B's columns too: the forward solve), so the
//     interchange needs no second barrier;
//   - back substitution with U: for k descending, x_k = y_k / u_kk (true
//     division) then y_i -= u_ik x_k, one thread per (row, right-hand side).
// Per element the operations are the unblocked getf2 / getrs order, so L,
// U, ipiv, info and X are bit-identical to the plain computation.  n <= 64
// for complex double, else n <= 128; nrhs <= 16 fused.
#include "device_ops.h"
#include "internal.h"

namespace batchlu {

namespace {

constexpr int CT = 256;                  // threads per work-group
constexpr size_t LDS_MAX = 160 * 1024;   // LDS of one compute unit (gfx950)

// LDS holds NB + CH rows: the rows past n are zero, so a column's update
// runs whole chunks of CH rows with no per-row test (a zero row's update
// stays zero; it is never a pivot candidate and never stored).
template <typename T, int NB, int NRP>
struct CtaShape {
    static constexpr int LDR = NB + NRP + 1;      // LDS row stride (odd: rows on distinct banks)
    // rows of a column updated per round: 16, or 8 where 16 would not fit
    static constexpr int CH = (size_t)(NB + 16) * LDR * sizeof(T) + 512 <= LDS_MAX ? 16 : 8;
    static constexpr int ROWS = NB + CH;
    static constexpr size_t bytes = (size_t)ROWS * LDR * sizeof(T);
    static constexpr bool fits = bytes + 512 <= LDS_MAX;
};

template <typename T, int NB, int NRP>
__global__ void __launch_bounds__(CT) cta_lds_kernel(Problem p, int mode)
{
    using O = ops<T>;
    using R = typename O::R;
    using K = typename O::K;
    constexpr int LDR = CtaShape<T, NB, NRP>::LDR;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int ROWS = CtaShape<T, NB, NRP>::ROWS;
    constexpr int CH = CtaShape<T, NB, NRP>::CH;
    T* S = reinterpret_cast<T*>(smem);             // [ROWS][LDR]
    __shared__ int s_piv;
    __shared__ int s_zero;
    __shared__ T s_x[NRP > 0 ? NRP : 1];

    const long long m = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = p.n;
    const bool solve = NRP > 0 && mode == MODE_GESV;
    const int nr = solve ? p.nrhs : 0;
    const int ncol = n + nr;
    T* A = (T*)p.A + m * p.sA;
    T* B = (T*)p.B + m * p.sB;
    const long long lda = p.lda, ldb = p.ldb;

    // [A | B] into LDS (column-major reads, coalesced down each column);
    // rows n .. ROWS-1 zero
    for (int c = wave; c < ncol; c += CT / 64)
        for (int i = lane; i < n; i += 64) S[i * LDR + c] = c < n ? A[i + c * lda] : B[i + (c - n) * ldb];
    for (int e = tid; e < (ROWS - n) * LDR; e += CT) S[n * LDR + e] = O::zero();
    int info = 0;
    __syncthreads();

    for (int j = 0; j < n; ++j) {
        if (wave == 0) {
            // a1: first argmax of the metric over rows j .. n-1 of column j
            K key = 0;
            int kp = 0x7fffffff;
            for (int i = j + lane; i < n; i += 64) {
                const K kq = (K)pivot_key(O::metric(S[i * LDR + j]));
                if (kq > key) {        // rows of a lane ascend: ties keep the first
                    key = kq;
                    kp = i;
                }
            }
            K kmax;
            int win;
            wave_argmax(key, kp, kmax, win);
            const int pr = __builtin_amdgcn_readlane(kp, win);
            const T piv = S[pr * LDR + j];
            const R pm = O::metric(piv);
            const bool zero = pm == R(0);
            // a3: multipliers of column j, rows as they stand after the
            // interchange (row pr takes old row j's entry)
            if (!zero) {
                const bool small = !(pm >= O::sfmin());
                const T r = O::recip(piv);
                for (int i = j + 1 + lane; i < n; i += 64) {
                    const T a = (i == pr) ? S[j * LDR + j] : S[i * LDR + j];
                    S[i * LDR + j] = small ? O::div(a, piv) : O::mul(a, r);
                }
            } else if (pr != j) {
                // no scaling, but the interchange of column j still happens
                if (lane == 0) S[pr * LDR + j] = S[j * LDR + j];
            }
            if (lane == 0) {
                S[j * LDR + j] = piv;
                s_piv = pr;
                s_zero = zero ? 1 : 0;
            }
        }
        __syncthreads();
        const int pr = s_piv;
        const bool zero = s_zero != 0;
        if (zero && info == 0) info = j + 1;
        if (tid == 0) p.ipiv[m * p.sP + j] = pr + 1;
        // a2 + a4: each column other than j: its interchange, then its update
        for (int c = tid; c < ncol; c += CT) {
            if (c == j) continue;
            T u = S[pr * LDR + c];
            if (pr != j) {
                S[pr * LDR + c] = S[j * LDR + c];
                S[j * LDR + c] = u;
            }
            if (c > j && !zero) {
                // whole chunks of CH rows (zero rows past n): a chunk's
                // loads are in flight together, at constant offsets
                for (int i0 = j + 1; i0 < n; i0 += CH) {
                    T* col = S + i0 * LDR + c;
                    const T* lc = S + i0 * LDR + j;
                    T a[CH], l[CH];
#pragma unroll
                    for (int q = 0; q < CH; ++q) {
                        a[q] = col[q * LDR];
                        l[q] = lc[q * LDR];
                    }
#pragma unroll
                    for (int q = 0; q < CH; ++q) O::fms(a[q], l[q], u);
#pragma unroll
                    for (int q = 0; q < CH; ++q) col[q * LDR] = a[q];
                }
            }
        }
        __syncthreads();
    }

    // a10: back substitution U x = y, k descending, one thread per (row, rhs)
    if (solve && info == 0) {
        for (int k = n - 1; k >= 0; --k) {
            if (tid < nr) {
                T x = O::div(S[k * LDR + n + tid], S[k * LDR + k]);
                S[k * LDR + n + tid] = x;
                s_x[tid] = x;
            }
            __syncthreads();
            for (int e = tid; e < k * NRP; e += CT) {
                const int i = e / NRP, c = e % NRP;      // NRP is a power of two
                if (c >= nr) continue;
                T y = S[i * LDR + n + c];
                O::fms(y, S[i * LDR + k], s_x[c]);
                S[i * LDR + n + c] = y;
            }
            __syncthreads();
        }
    }
    // factors (and X where info == 0) back to memory, down each column
    for (int c = wave; c < ncol; c += CT / 64) {
        if (c >= n && info != 0) break;
        for (int i = lane; i < n; i += 64) {
            if (c < n) A[i + c * lda] = S[i * LDR + c];
            else B[i + (c - n) * ldb] = S[i * LDR + c];
        }
    }
    if (tid == 0) p.info[m] = info;
}

template <typename T, int NB, int NRP>
hipError_t launch_nb(const Problem& p, int mode, hipStream_t s) {
    static_assert(CtaShape<T, NB, NRP>::fits, "the LDS stage must fit one compute unit");
    const size_t smem = CtaShape<T, NB, NRP>::bytes;
    hipLaunchKernelGGL((cta_lds_kernel<T, NB, NRP>), dim3((unsigned)p.batch), dim3(CT), smem, s, p, mode);
    return hipGetLastError();
}

template <typename T, int NRP>
hipError_t launch_nrp(const Problem& p, int mode, hipStream_t s) {
    if (p.n <= 64) return launch_nb<T, 64, NRP>(p, mode, s);
    if constexpr (sizeof(T) < 16) {
        if (p.n <= 128) return launch_nb<T, 128, NRP>(p, mode, s);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_t(const Problem& p, int mode, hipStream_t s) {
    if (mode != MODE_GESV || p.nrhs == 0) return launch_nrp<T, 0>(p, MODE_GETRF, s);
    if (p.nrhs <= 4) return launch_nrp<T, 4>(p, mode, s);
    if (p.nrhs <= 16) return launch_nrp<T, 16>(p, mode, s);
    return hipErrorInvalidValue;
}

}  // namespace

bool cta_lds_supported(int dtype, int n, int nrhs, int mode) {
    if (n < 1 || n > (dtype == C128 ? 64 : 128)) return false;
    return mode != MODE_GESV || (nrhs >= 0 && nrhs <= 16);
}

hipError_t cta_lds_launch(int dtype, const Problem& p, int mode, hipStream_t s) {
    if (!cta_lds_supported(dtype, p.n, p.nrhs, mode)) return hipErrorInvalidValue;
    switch (dtype) {
    case R32: return launch_t<float>(p, mode, s);
    case R64: return launch_t<double>(p, mode, s);
    case C64: return launch_t<cplx<float>>(p, mode, s);
    case C128: return launch_t<cplx<double>>(p, mode, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace batchlu
