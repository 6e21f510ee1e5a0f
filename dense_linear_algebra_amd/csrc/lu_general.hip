// lu_general.hip -- LU with partial pivoting of m x n matrices, and batches
// whose matrices differ in size (pointer arrays with per-matrix m, n, lda),
// plus the matching solve for square variable-size batches.
//
// BatchLAS "LU" page, family table: getrf on a non-square A, and a batch
// whose members differ in shape, have no native route there (only the
// vendor's LAPACK-style getrf, or one call per member).  Here one
// work-group of 256 threads factors one matrix of any shape with m <= 1024
// (complex double 512) and n <= 1024, reading its own sizes, so one launch
// serves a whole heterogeneous batch:
//   panel   the (m - j0) x 32 panel in VGPRs (RPT rows per thread), one
//           work-group barrier per column: each wavefront's argmax (DPP and
//           readlane) with its candidate row goes to a double-buffered LDS
//           slot, every thread picks the winner; rows are relabelled lazily
//           and written once to their final places;
//   swaps   the panel's interchanges reach every other column as one gather
//           of the new top rows and one move of the displaced rows (the
//           composition of the panel's transpositions, traced backwards);
//   U12     one thread per column solves with the panel's unit-lower L11
//           (staged in LDS), ascending k;
//   update  A22 -= L21 U12: one thread per row keeps its L21 row in
//           registers, U12 comes through LDS eight columns at a time, one
//           fused multiply-add per k in ascending order.
// A step whose pivot is exactly zero is left out of the U12 solve and the
// update, as the unblocked order does.  Per element the operation sequence
// is that of the unblocked right-looking getf2 on m x n, so L, U and ipiv
// are bit-identical to it.
#include <type_traits>

#include "device_ops.h"
#include "internal.h"

namespace batchlu {

namespace {

constexpr int GNT = 256;   // threads per work-group
constexpr int GNB = 32;    // panel width
constexpr int GNW = GNT / 64;
constexpr int GCC = 8;     // U12 columns staged per round of the update

struct GenArgs {
    // strided batch (ptrs == nullptr): every matrix m x n
    void* A = nullptr; int m = 0, n = 0, lda = 0; long long sA = 0;
    int* ipiv = nullptr; long long sP = 0;
    // variable-size batch: device arrays of per-matrix values
    void* const* Aptrs = nullptr; const int* ms = nullptr; const int* ns = nullptr; const int* ldas = nullptr;
    int* const* ipivptrs = nullptr;
    int* info = nullptr;
    int cap_m = 0;          // rows the launch's RPT covers
};

template <typename T>
struct GenMat {
    T* A; int m, n, lda; int* ipiv;
};

// The matrix of work-group b; false (and info = -1) for sizes outside what
// the launch covers or an lda below m, so that nothing out of range is read.
template <typename T>
__device__ inline bool gen_desc(const GenArgs& g, long long b, GenMat<T>& d) {
    if (g.Aptrs) {
        d.A = (T*)g.Aptrs[b]; d.m = g.ms[b]; d.n = g.ns[b]; d.lda = g.ldas[b]; d.ipiv = g.ipivptrs[b];
    } else {
        d.A = (T*)g.A + b * g.sA; d.m = g.m; d.n = g.n; d.lda = g.lda; d.ipiv = g.ipiv + b * g.sP;
    }
    return d.m >= 0 && d.n >= 0 && d.m <= g.cap_m && d.n <= 1024 && d.lda >= (d.m > 1 ? d.m : 1) &&
           (d.m == 0 || d.n == 0 || (d.A != nullptr && d.ipiv != nullptr));
}

// Float with one row per thread is budgeted for four wavefronts per SIMD:
// left alone the compiler takes 131 VGPRs (three per SIMD); at 128 it
// spills 8 bytes per lane, and the variable-size gesv (n in [16, 256],
// batch 4096) runs 6.25 -> 5.65 ms.  Two rows per thread spill heavily at
// three or four per SIMD and keep the default.
template <typename T, int RPT>
constexpr int general_waves() { return (sizeof(T) == 4 && RPT == 1) ? 4 : 1; }

template <typename T, int RPT>
__global__ void __launch_bounds__(GNT) __attribute__((amdgpu_waves_per_eu(general_waves<T, RPT>())))
getrf_general_kernel(GenArgs g)
{
    using O = ops<T>;
    using R = typename O::R;
    using K = typename O::K;
    __shared__ K skey[2][GNW];
    __shared__ int spos[2][GNW];
    __shared__ __attribute__((aligned(16))) T cand[2][GNW][GNB];
    __shared__ int srec[GNB];
    __shared__ int src_top[GNB], src_low[GNB], dst_low[GNB];
    __shared__ int nlow;
    __shared__ unsigned zmask;
    __shared__ T l11[GNB][GNB + 1];
    __shared__ T ust[2][GNB][GCC];

    const long long b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    GenMat<T> d;
    if (!gen_desc<T>(g, b, d)) {
        if (tid == 0) g.info[b] = -1;
        return;
    }
    const int m = d.m, n = d.n;
    const long long lda = d.lda;
    T* A = d.A;
    const int kmin = m < n ? m : n;
    int info = 0;

    for (int j0 = 0; j0 < kmin; j0 += GNB) {
        const int w = min(GNB, kmin - j0);
        const int mp = m - j0;                          // panel height
        T* P = A + j0 + j0 * lda;                       // panel origin
        // ---- panel: rows in VGPRs, lazy relabel --------------------------
        T a[RPT][GNB];
        int pos[RPT];
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            const int r = tid + q * GNT;
            pos[q] = r < mp ? r : 0x3fffffff;
#pragma unroll
            for (int c = 0; c < GNB; ++c) a[q][c] = (r < mp && c < w) ? P[r + c * lda] : O::zero();
        }
        if (tid == 0) zmask = 0;
#pragma unroll
        for (int jj = 0; jj < GNB; ++jj) {
            if (jj >= w) continue;
            const int buf = jj & 1;
            K key = 0;
            int kp = 0x7fffffff, ks = 0;
#pragma unroll
            for (int q = 0; q < RPT; ++q) {
                const K kq = (pos[q] >= jj && pos[q] < mp) ? (K)pivot_key(O::metric(a[q][jj])) : (K)0;
                const bool take = kq > key || (kq == key && pos[q] < kp);
                key = take ? kq : key;
                kp = take ? pos[q] : kp;
                ks = take ? q : ks;
            }
            K kmax;
            int win;
            wave_argmax(key, kp, kmax, win);
            if (win < 0) {
                if (lane == 0) {
                    skey[buf][wave] = 0;
                    spos[buf][wave] = 0x7fffffff;
                }
            } else if (lane == win) {
                skey[buf][wave] = kmax;
                spos[buf][wave] = kp;
#pragma unroll
                for (int q = 0; q < RPT; ++q)
                    if (q == ks)
#pragma unroll
                        for (int c = 0; c < GNB; ++c) cand[buf][wave][c] = a[q][c];
            }
            __syncthreads();
            K best = skey[buf][0];
            int ppos = spos[buf][0], vb = 0;
#pragma unroll
            for (int v = 1; v < GNW; ++v) {
                const K kv = skey[buf][v];
                const int pv = spos[buf][v];
                const bool take = kv > best || (kv == best && pv < ppos);
                best = take ? kv : best;
                ppos = take ? pv : ppos;
                vb = take ? v : vb;
            }
            T u[GNB];
#pragma unroll
            for (int c = 0; c < GNB; ++c) u[c] = c >= jj ? cand[buf][vb][c] : O::zero();
#pragma unroll
            for (int q = 0; q < RPT; ++q) {
                if (pos[q] == ppos) srec[jj] = ppos;
                pos[q] = (pos[q] == ppos) ? jj : (pos[q] == jj ? ppos : pos[q]);
            }
            const T piv = u[jj];
            const R pm = O::metric(piv);
            const bool zero = pm == R(0);
            if (zero) {
                if (info == 0) info = j0 + jj + 1;
                if (tid == 0) zmask |= 1u << jj;
                continue;
            }
            const T r = O::recip(piv);
            const bool small = !(pm >= O::sfmin());
#pragma unroll
            for (int q = 0; q < RPT; ++q) {
                if (pos[q] > jj && pos[q] < mp) {
                    const T l = small ? O::div(a[q][jj], piv) : O::mul(a[q][jj], r);
                    a[q][jj] = l;
#pragma unroll
                    for (int c = 0; c < GNB; ++c)
                        if (c > jj && c < w) O::fms(a[q][c], l, u[c]);
                }
            }
        }
        __syncthreads();
        // rows to their final places; ipiv global and 1-based
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            if (tid + q * GNT < mp)
#pragma unroll
                for (int c = 0; c < GNB; ++c)
                    if (c < w) P[pos[q] + c * lda] = a[q][c];
        }
        if (tid < w) d.ipiv[j0 + tid] = j0 + srec[tid] + 1;
        // ---- the interchanges of this panel for every other column ---------
        if (tid == 0) nlow = 0;
        __syncthreads();
        if (tid < w) {
            int x = tid;                                 // new top row tid: a backward trace
            for (int s2 = w - 1; s2 >= 0; --s2) {
                const int ps2 = srec[s2];
                x = (x == s2) ? ps2 : (x == ps2 ? s2 : x);
            }
            src_top[tid] = x;
            const int ps = srec[tid];
            bool first = ps >= w;                        // a row below the top that some step takes
            for (int s2 = 0; s2 < tid; ++s2) first = first && srec[s2] != ps;
            if (first) {
                int y = ps;
                for (int s2 = w - 1; s2 >= 0; --s2) {
                    const int ps2 = srec[s2];
                    y = (y == s2) ? ps2 : (y == ps2 ? s2 : y);
                }
                const int slot = atomicAdd(&nlow, 1);
                dst_low[slot] = ps;
                src_low[slot] = y;
            }
        }
        // L11 into LDS for the U12 solve
        for (int e = tid; e < GNB * GNB; e += GNT) {
            const int f = e % GNB, c = e / GNB;
            l11[f][c] = (f < w && c < w) ? P[f + c * lda] : O::zero();
        }
        __syncthreads();
        const int nl = nlow;
        const unsigned zm = zmask;
        for (int c = tid; c < n; c += GNT) {
            // L11 is read from LDS per column, not held in registers across
            // the loop (the compiler would otherwise hoist all its entries)
            asm volatile("" ::: "memory");
            if (c >= j0 && c < j0 + w) continue;        // the panel itself is done
            T* col = A + j0 + c * lda;
            T top[GNB];
#pragma unroll
            for (int f = 0; f < GNB; ++f) top[f] = f < w ? col[src_top[f]] : O::zero();
            T mv[GNB];
#pragma unroll
            for (int f = 0; f < GNB; ++f) mv[f] = f < nl ? col[src_low[f]] : O::zero();
#pragma unroll
            for (int f = 0; f < GNB; ++f)
                if (f < nl) col[dst_low[f]] = mv[f];
            if (c >= j0 + w) {
                // U12 = L11^-1 (P A12), ascending k, zero pivots left out
#pragma unroll
                for (int k = 0; k < GNB; ++k) {
                    if (k >= w || ((zm >> k) & 1u)) continue;
#pragma unroll
                    for (int f = 0; f < GNB; ++f)
                        if (f > k && f < w) O::fms(top[f], l11[f][k], top[k]);
                }
            }
#pragma unroll
            for (int f = 0; f < GNB; ++f)
                if (f < w) col[f] = top[f];
        }
        __syncthreads();
        // ---- trailing update A22 -= L21 U12 ---------------------------------
        const int r0 = j0 + w;                          // first row and column of A22
        if (r0 < m && r0 < n && zm != (w == 32 ? 0xffffffffu : ((1u << w) - 1u))) {
            T l[RPT][GNB];
#pragma unroll
            for (int q = 0; q < RPT; ++q) {
                const int i = r0 + tid + q * GNT;
#pragma unroll
                for (int k = 0; k < GNB; ++k) l[q][k] = (i < m && k < w) ? A[i + (j0 + k) * lda] : O::zero();
            }
            int round = 0;
            for (int c0 = r0; c0 < n; c0 += GCC, ++round) {
                const int sb = round & 1;
                {   // stage U12[0..w) x [c0, c0 + GCC)
                    const int k = tid % GNB, cc = tid / GNB;
                    ust[sb][k][cc] = (k < w && c0 + cc < n) ? A[j0 + k + (c0 + cc) * lda] : O::zero();
                }
                __syncthreads();
                const int ncc = min(GCC, n - c0);
#pragma unroll 1
                for (int cc = 0; cc < ncc; ++cc) {       // one staged column live at a time
                    asm volatile("" ::: "memory");
                    T acc[RPT];
#pragma unroll
                    for (int q = 0; q < RPT; ++q) {
                        const int i = r0 + tid + q * GNT;
                        acc[q] = i < m ? A[i + (c0 + cc) * lda] : O::zero();
                    }
#pragma unroll
                    for (int k = 0; k < GNB; ++k) {
                        if (k >= w || ((zm >> k) & 1u)) continue;
                        const T uk = ust[sb][k][cc];
#pragma unroll
                        for (int q = 0; q < RPT; ++q) O::fms(acc[q], l[q][k], uk);
                    }
#pragma unroll
                    for (int q = 0; q < RPT; ++q) {
                        const int i = r0 + tid + q * GNT;
                        if (i < m) A[i + (c0 + cc) * lda] = acc[q];
                    }
                }
            }
            __syncthreads();
        }
    }
    if (tid == 0) g.info[b] = info;
}

// Solve A X = B for a square variable-size batch with the factors and ipiv
// of getrf_general_kernel: one work-group per matrix, one row per thread,
// the interchanges as one gather (backward trace of ipiv), forward with the
// unit-lower L and back with U (true division by u_kk) a 32-row block at a
// time, NRT right-hand sides per pass.  With info given, matrices whose
// info is not 0 keep their B.
// x_c = y_c / u_cc for the NRT right-hand sides held by diagonal lane dl,
// broadcast in xc (lane dl keeps them in y): lane r divides right-hand side
// r by the broadcast diagonal (the same operands, so the same bits), so the
// wavefront pays for one division per step rather than NRT.
template <typename T, int NRT>
__device__ inline void spread_divide(T (&y)[NRT], T (&xc)[NRT], T diag, int dl, int lane) {
    using O = ops<T>;
    T yc[NRT];
#pragma unroll
    for (int r = 0; r < NRT; ++r) yc[r] = readlane_t(y[r], dl);
    const T d = readlane_t(diag, dl);
    T v = yc[0];
#pragma unroll
    for (int r = 1; r < NRT; ++r)
        if (lane == r) v = yc[r];
    const T q = O::div(v, d);
#pragma unroll
    for (int r = 0; r < NRT; ++r) xc[r] = readlane_t(q, r);
    if (lane == dl)
#pragma unroll
        for (int r = 0; r < NRT; ++r) y[r] = xc[r];
}

template <typename T, int NRT>
__global__ void __launch_bounds__(1024) getrs_general_kernel(GenArgs g, const int* nrhs_arr,
                                                            void* const* Bptrs, const int* ldbs, int check_info)
{
    using O = ops<T>;
    constexpr int BS = 32;
    __shared__ T ybuf[2][BS][NRT];
    extern __shared__ int sipiv[];
    const long long b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = g.ns[b], nrhs = nrhs_arr[b], ldb = ldbs[b], lda = g.ldas[b];
    if (n <= 0 || nrhs <= 0 || n > (int)blockDim.x || lda < n || ldb < n) return;
    if (check_info && g.info[b] != 0) return;
    const T* F = (const T*)g.Aptrs[b];
    const int* ipiv = g.ipivptrs[b];
    T* B = (T*)Bptrs[b];
    for (int i = tid; i < n; i += blockDim.x) {
        const int v = ipiv[i] - 1;
        sipiv[i] = (v >= 0 && v < n) ? v : i;
    }
    __syncthreads();
    const int row = tid;
    const bool have = row < n;
    int src = row;
    if (have)
        for (int k = n - 1; k >= 0; --k) {
            const int pk = sipiv[k];
            src = (src == k) ? pk : (src == pk ? k : src);
        }
    const int P = (n + BS - 1) / BS;
    for (int c0 = 0; c0 < nrhs; c0 += NRT) {
        T y[NRT];
#pragma unroll
        for (int r = 0; r < NRT; ++r)
            y[r] = (have && c0 + r < nrhs) ? B[src + (long long)(c0 + r) * ldb] : O::zero();
        __syncthreads();   // every row of this tile read before any is written
        for (int kb = 0; kb < P; ++kb) {
            const int r0 = kb * BS, wd = min(BS, n - r0);
            T(*yb)[NRT] = ybuf[kb & 1];
            if (wave == r0 / 64) {
                const int base = r0 % 64, mrow = lane - base;
                const bool inb = mrow >= 0 && mrow < wd;
#pragma unroll
                for (int c = 0; c < BS; ++c) {
                    if (c >= wd) continue;
                    const T lv = (inb && mrow > c) ? F[row + (long long)(r0 + c) * lda] : O::zero();
                    T xc[NRT];
#pragma unroll
                    for (int r = 0; r < NRT; ++r) xc[r] = readlane_t(y[r], base + c);
                    if (inb && mrow > c)
#pragma unroll
                        for (int r = 0; r < NRT; ++r) O::fms(y[r], lv, xc[r]);
                }
                if (inb)
#pragma unroll
                    for (int r = 0; r < NRT; ++r) yb[mrow][r] = y[r];
            }
            __syncthreads();
            if (have && row >= r0 + wd)
                for (int c = 0; c < wd; ++c) {
                    const T lv = F[row + (long long)(r0 + c) * lda];
#pragma unroll
                    for (int r = 0; r < NRT; ++r) O::fms(y[r], lv, yb[c][r]);
                }
        }
        __syncthreads();
        for (int kb = P - 1; kb >= 0; --kb) {
            const int r0 = kb * BS, wd = min(BS, n - r0);
            T(*yb)[NRT] = ybuf[kb & 1];
            if (wave == r0 / 64) {
                const int base = r0 % 64, mrow = lane - base;
                const bool inb = mrow >= 0 && mrow < wd;
#pragma unroll
                for (int c = BS - 1; c >= 0; --c) {
                    if (c >= wd) continue;
                    const T uv = (inb && mrow <= c) ? F[row + (long long)(r0 + c) * lda] : O::zero();
                    T xc[NRT];
                    if constexpr (NRT == 1) {
                        if (mrow == c) y[0] = O::div(y[0], uv);
                        xc[0] = readlane_t(y[0], base + c);
                    } else {
                        spread_divide(y, xc, uv, base + c, lane);
                    }
                    if (inb && mrow < c)
#pragma unroll
                        for (int r = 0; r < NRT; ++r) O::fms(y[r], uv, xc[r]);
                }
                if (inb)
#pragma unroll
                    for (int r = 0; r < NRT; ++r) yb[mrow][r] = y[r];
            }
            __syncthreads();
            if (have && row < r0)
                for (int c = wd - 1; c >= 0; --c) {
                    const T uv = F[row + (long long)(r0 + c) * lda];
#pragma unroll
                    for (int r = 0; r < NRT; ++r) O::fms(y[r], uv, yb[c][r]);
                }
        }
        if (have)
#pragma unroll
            for (int r = 0; r < NRT; ++r)
                if (c0 + r < nrhs) B[row + (long long)(c0 + r) * ldb] = y[r];
        __syncthreads();
    }
}

// rows per work-group: RPT x 256 rows of 32 panel entries stay in VGPRs;
// beyond these the panel would spill
template <typename T>
constexpr int general_max_m() { return sizeof(T) == 16 ? 256 : (sizeof(T) == 8 ? 512 : 1024); }

template <typename T>
hipError_t launch_general(const GenArgs& g0, int max_m, int batch, hipStream_t s) {
    GenArgs g = g0;
    const dim3 grid((unsigned)batch), block(GNT);
    if (max_m > general_max_m<T>()) return hipErrorInvalidValue;
    if (max_m <= 256) {
        g.cap_m = 256;
        hipLaunchKernelGGL((getrf_general_kernel<T, 1>), grid, block, 0, s, g);
    } else if constexpr (general_max_m<T>() >= 512) {
        if (max_m <= 512) {
            g.cap_m = 512;
            hipLaunchKernelGGL((getrf_general_kernel<T, 2>), grid, block, 0, s, g);
        } else if constexpr (general_max_m<T>() >= 1024) {
            g.cap_m = 1024;
            hipLaunchKernelGGL((getrf_general_kernel<T, 4>), grid, block, 0, s, g);
        }
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_general_solve(const GenArgs& g, const int* nrhs, void* const* B, const int* ldb, int max_n,
                                int batch, bool check_info, hipStream_t s) {
    const int threads = ((max_n + 63) / 64) * 64;
    const size_t smem = (size_t)threads * sizeof(int);   // ipiv of a matrix of up to `threads` rows
    const dim3 grid((unsigned)batch), block(threads);
    if constexpr (sizeof(T) == 16)
        hipLaunchKernelGGL((getrs_general_kernel<T, 2>), grid, block, smem, s, g, nrhs, B, ldb, check_info ? 1 : 0);
    else
        hipLaunchKernelGGL((getrs_general_kernel<T, 4>), grid, block, smem, s, g, nrhs, B, ldb, check_info ? 1 : 0);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_getrf(const GenArgs& g, int max_m, int batch, hipStream_t s) {
    return launch_general<T>(g, max_m, batch, s);
}

}  // namespace

int general_max_rows(int dtype) {
    switch (dtype) {
    case R32: return general_max_m<float>();
    case R64: return general_max_m<double>();
    case C64: return general_max_m<cplx<float>>();
    default: return general_max_m<cplx<double>>();
    }
}

hipError_t general_getrf_strided(int dtype, void* A, int m, int n, int lda, long long sA, int* ipiv, long long sP,
                                 int* info, int batch, hipStream_t s) {
    GenArgs g;
    g.A = A; g.m = m; g.n = n; g.lda = lda; g.sA = sA; g.ipiv = ipiv; g.sP = sP; g.info = info;
    switch (dtype) {
    case R32: return dispatch_getrf<float>(g, m, batch, s);
    case R64: return dispatch_getrf<double>(g, m, batch, s);
    case C64: return dispatch_getrf<cplx<float>>(g, m, batch, s);
    case C128: return dispatch_getrf<cplx<double>>(g, m, batch, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t general_getrf_vbatched(int dtype, void* const* A, const int* m, const int* n, const int* lda,
                                  int* const* ipiv, int* info, int max_m, int batch, hipStream_t s) {
    GenArgs g;
    g.Aptrs = A; g.ms = m; g.ns = n; g.ldas = lda; g.ipivptrs = ipiv; g.info = info;
    switch (dtype) {
    case R32: return dispatch_getrf<float>(g, max_m, batch, s);
    case R64: return dispatch_getrf<double>(g, max_m, batch, s);
    case C64: return dispatch_getrf<cplx<float>>(g, max_m, batch, s);
    case C128: return dispatch_getrf<cplx<double>>(g, max_m, batch, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t general_getrs_vbatched(int dtype, void* const* A, const int* n, const int* lda, int* const* ipiv,
                                  const int* nrhs, void* const* B, const int* ldb, int* info, int max_n, int batch,
                                  hipStream_t s) {
    GenArgs g;
    g.Aptrs = A; g.ns = n; g.ldas = lda; g.ipivptrs = ipiv; g.info = info;
    const bool chk = info != nullptr;
    switch (dtype) {
    case R32: return launch_general_solve<float>(g, nrhs, B, ldb, max_n, batch, chk, s);
    case R64: return launch_general_solve<double>(g, nrhs, B, ldb, max_n, batch, chk, s);
    case C64: return launch_general_solve<cplx<float>>(g, nrhs, B, ldb, max_n, batch, chk, s);
    case C128: return launch_general_solve<cplx<double>>(g, nrhs, B, ldb, max_n, batch, chk, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace batchlu
