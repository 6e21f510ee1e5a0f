// blocked_lu_impl.h -- blocked right-looking LU (panel width 32) and the blocked
// LU solve, for matrices too large for the register tiers.
//
// BatchLAS "LU" page, blocked-getrf and register-panel paragraphs, and the
// row-interchange paragraphs; redesigned for gfx950:
//   panel      one work-group per matrix factors the (n - j0) x 32 panel with
//              one row per thread in VGPRs, lazy relabel, and two work-group
//              barriers per column (argmax slots, then the pivot row);
//   right swap the interchanges of the panel are applied to the trailing
//              columns inside the panel TRSM: each column's moved rows are
//              gathered once (never a sequential walk of 32 swaps), the
//              top 32 become U12 = L11^-1 A12 and the displaced rows are
//              written to their new places;
//   gemm       A22 -= L21 * U12 on MFMA 16x16x4 (f32 and f64; complex on the
//              VALU).  An MFMA accumulates its four products like a chain of
//              four fused multiply-adds in k order, so chaining MFMAs in
//              ascending k reproduces the unblocked operation order exactly;
//   left swap  deferred to one pass after the last panel: every earlier
//              panel's L columns are gathered through the composition of the
//              later interchanges.
// getrs: the full row permutation of B is one gather; forward and back
// substitution run block by block (a 32-row triangular solve, then a GEMM
// update of the remaining rows), preserving the plain order of operations
// (ascending k forward, descending k backward, true division by u_kk).
#pragma once

#include <type_traits>

#include "device_ops.h"
#include "internal.h"

namespace batchlu {

namespace {

constexpr int NBP = 32;    // panel width
constexpr int TT = 64;     // GEMM tile (rows and columns)

// ---------------------------------------------------------------------------
// panel factorisation
// ---------------------------------------------------------------------------
template <typename T, int RPT, int MAXT>
__global__ void __launch_bounds__(MAXT) panel_kernel(Problem p, int j0, int w)
{
    using O = ops<T>;
    using R = typename O::R;
    using K = typename O::K;
    const int m = p.n - j0;                 // panel height
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwave = nt >> 6;
    const long long mat = blockIdx.x;

    __shared__ K skey[16];
    __shared__ int spos[16];
    __shared__ T prow[NBP];
    __shared__ int srec[NBP];

    T* A = (T*)p.A + mat * p.sA + j0 + (long long)j0 * p.lda;   // panel origin

    T a[RPT][NBP];
    int pos[RPT];
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
        const int r = tid + q * nt;
        pos[q] = r < m ? r : 0x3fffffff;
#pragma unroll
        for (int c = 0; c < NBP; ++c) a[q][c] = (r < m && c < w) ? A[r + (long long)c * p.lda] : O::zero();
    }

    int info = 0;
#pragma unroll
    for (int jj = 0; jj < NBP; ++jj) {
        if (jj >= w) continue;
        // a1: argmax over rows at positions >= jj
        K key[RPT];
        K kmax = 0;
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            K kk = (pos[q] >= jj && pos[q] < m) ? (K)pivot_key(O::metric(a[q][jj])) : (K)0;
            key[q] = kk;
            kmax = kk > kmax ? kk : kmax;
        }
        kmax = group_max<64>(kmax);
        int qpos = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < RPT; ++q)
            if (key[q] == kmax && pos[q] < qpos) qpos = pos[q];
        qpos = group_min<64>(qpos);
        if (lane == 0) {
            skey[wave] = kmax;
            spos[wave] = qpos;
        }
        __syncthreads();   // B1: per-wave winners visible
        K best = 0;
        int ppos = 0x7fffffff;
        for (int v = 0; v < nwave; ++v) {
            const K kv = skey[v];
            const int pv = spos[v];
            if (kv > best || (kv == best && pv < ppos)) {
                best = kv;
                ppos = pv;
            }
        }
        // the owner publishes the pivot row, then positions jj and ppos swap
#pragma unroll
        for (int q = 0; q < RPT; ++q)
            if (pos[q] == ppos) {
#pragma unroll
                for (int c = 0; c < NBP; ++c)
                    if (c >= jj) prow[c] = a[q][c];
            }
#pragma unroll
        for (int q = 0; q < RPT; ++q)
            pos[q] = (pos[q] == ppos) ? jj : (pos[q] == jj ? ppos : pos[q]);
        if (tid == 0) srec[jj] = ppos;
        __syncthreads();   // B2: pivot row visible
        const T piv = prow[jj];
        const R pm = O::metric(piv);
        const bool zero = pm == R(0);
        if (zero && info == 0) info = j0 + jj + 1;
        const T r = O::recip(piv);
        const bool small = !(pm >= O::sfmin());
        T u[NBP];
#pragma unroll
        for (int c = 0; c < NBP; ++c)
            if (c > jj) u[c] = prow[c];
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            if (pos[q] > jj && pos[q] < m && !zero) {
                T l = O::mul(a[q][jj], r);
                if (__builtin_expect(__builtin_amdgcn_ballot_w64(small) != 0, 0)) {
                    asm volatile("" ::: "memory");
                    if (small) l = O::div(a[q][jj], piv);
                }
                a[q][jj] = l;
#pragma unroll
                for (int c = 0; c < NBP; ++c)
                    if (c > jj) O::fms(a[q][c], l, u[c]);
            }
        }
    }
    __syncthreads();
    // rows to their final positions; ipiv as global 1-based rows
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
        const int r = tid + q * nt;
        if (r < m)
#pragma unroll
            for (int c = 0; c < NBP; ++c)
                if (c < w) A[pos[q] + (long long)c * p.lda] = a[q][c];
    }
    if (tid < w) p.ipiv[mat * p.sP + j0 + tid] = j0 + srec[tid] + 1;
    if (tid == 0) {
        int* ip = p.info + mat;
        if (j0 == 0) *ip = info;
        else if (info != 0 && *ip == 0) *ip = info;
    }
}

// Panels taller than the register-resident kernels reach (at most 4096 rows,
// 1024 threads with up to four rows each): the panel stays in memory, where
// this work-group's own earlier column steps left it (32 columns, L2-resident),
// and each column step reads and updates it there.  Rows keep their storage
// places while the panel is factored; pos[] follows each row's position after
// the interchanges so far, as in the register kernels, and the rows that moved
// go to their final positions at the end.  Per element the operations are
// those of the register kernels: l = a * (1 / pivot) (a / pivot when the
// pivot is below the safe minimum), then a_c -= l u_c column by column, one
// column step at a time.  Two barriers per step: one after the per-wavefront
// argmax, one after the update (the next step reads what this one wrote).
template <typename T>
__global__ void __launch_bounds__(1024) panel_mem_kernel(Problem p, int j0, int w)
{
    using O = ops<T>;
    using R = typename O::R;
    using K = typename O::K;
    constexpr int NT = 1024, NWV = NT / 64, RPT = 4;
    constexpr int CH = sizeof(T) >= 16 ? 2 : sizeof(T) == 8 ? 4 : 8;   // columns per load batch
    const int m = p.n - j0;                 // panel height (<= NT * RPT)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const long long mat = blockIdx.x;
    const long long lda = p.lda;

    __shared__ K skey[NWV];
    __shared__ int spos[NWV];
    __shared__ int sphy[NWV];
    __shared__ int srec[NBP];

    T* A = (T*)p.A + mat * p.sA + j0 + (long long)j0 * lda;   // panel origin

    // element (r, c) of the panel: column c's base (uniform) plus the row's
    // byte offset (32-bit, one register per row for every column)
    auto at = [](T* col, unsigned boff) -> T& { return *(T*)((char*)col + boff); };
    // the offsets, re-read in each iteration: hoisted 64-bit addresses per
    // row and column would not fit the registers
    auto fresh = [](unsigned v) {
        asm volatile("" : "+v"(v));
        return v;
    };
    int pos[RPT];
    unsigned roff[RPT];
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
        const int r = tid + q * NT;
        pos[q] = r < m ? r : 0x3fffffff;
        roff[q] = (unsigned)r * (unsigned)sizeof(T);
    }

    int info = 0;
#pragma unroll 1
    for (int jj = 0; jj < w; ++jj) {
        T* colj = A + (long long)jj * lda;     // uniform column bases, unsigned row offsets
        // a1: the lane's best row (highest key, lowest position among equal
        // keys), then the wavefront's, then the work-group's
        K key = 0;
        int kp = 0x7fffffff, kr = 0;
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            const int r = tid + q * NT;
            if (pos[q] >= jj && pos[q] < m) {
                const K kq = (K)pivot_key(O::metric(at(colj, fresh(roff[q]))));
                if (kq > key || (kq == key && pos[q] < kp)) {
                    key = kq;
                    kp = pos[q];
                    kr = r;
                }
            }
        }
        K kmax;
        int win;
        wave_argmax(key, kp, kmax, win);
        const int wl = win < 0 ? 0 : win;
        const int wpos = __builtin_amdgcn_readlane(kp, wl);
        const int wphy = __builtin_amdgcn_readlane(kr, wl);
        if (lane == 0) {
            skey[wave] = win < 0 ? (K)0 : kmax;
            spos[wave] = win < 0 ? 0x7fffffff : wpos;
            sphy[wave] = wphy;
        }
        __syncthreads();
        K best = 0;
        int ppos = 0x7fffffff, pphy = 0;
#pragma unroll
        for (int v = 0; v < NWV; ++v) {
            const K kv = skey[v];
            const int pv = spos[v];
            if (kv > best || (kv == best && pv < ppos)) {
                best = kv;
                ppos = pv;
                pphy = sphy[v];
            }
        }
        if (tid == 0) srec[jj] = ppos;
#pragma unroll
        for (int q = 0; q < RPT; ++q)
            pos[q] = (pos[q] == ppos) ? jj : (pos[q] == jj ? ppos : pos[q]);
        const unsigned prow = (unsigned)pphy * (unsigned)sizeof(T);   // the pivot row, in its storage place
        const T piv = at(colj, prow);
        const R pm = O::metric(piv);
        const bool zero = pm == R(0);
        if (zero && info == 0) info = j0 + jj + 1;
        if (!zero) {
            const T rcp = O::recip(piv);
            const bool small = !(pm >= O::sfmin());
            bool act[RPT];
            T l[RPT];
#pragma unroll
            for (int q = 0; q < RPT; ++q) {
                act[q] = pos[q] > jj && pos[q] < m;
                if (act[q]) {
                    const unsigned ro = fresh(roff[q]);
                    const T a = at(colj, ro);
                    l[q] = small ? O::div(a, piv) : O::mul(a, rcp);
                    at(colj, ro) = l[q];
                }
            }
            // a4: columns jj+1 .. w-1, CH at a time (their loads issued
            // together, ahead of the stores)
#pragma unroll 1
            for (int c0 = jj + 1; c0 < w; c0 += CH) {
                T u[CH], x[RPT][CH];
                unsigned ro[RPT];
#pragma unroll
                for (int q = 0; q < RPT; ++q) ro[q] = fresh(roff[q]);
                T* cols[CH];
#pragma unroll
                for (int cc = 0; cc < CH; ++cc) cols[cc] = A + (long long)(c0 + cc) * lda;
#pragma unroll
                for (int cc = 0; cc < CH; ++cc)
                    if (c0 + cc < w) u[cc] = at(cols[cc], prow);
#pragma unroll
                for (int q = 0; q < RPT; ++q)
#pragma unroll
                    for (int cc = 0; cc < CH; ++cc)
                        if (act[q] && c0 + cc < w) x[q][cc] = at(cols[cc], ro[q]);
#pragma unroll
                for (int q = 0; q < RPT; ++q)
#pragma unroll
                    for (int cc = 0; cc < CH; ++cc)
                        if (act[q] && c0 + cc < w) {
                            O::fms(x[q][cc], l[q], u[cc]);
                            at(cols[cc], ro[q]) = x[q][cc];
                        }
            }
        }
        __syncthreads();
    }
    // the rows that moved go to their final positions, a few columns at a
    // time: every read of a batch of columns precedes every write to it
    constexpr int CW = 32 / sizeof(T);
#pragma unroll 1
    for (int c0 = 0; c0 < w; c0 += CW) {
        T v[RPT][CW];
        T* cols[CW];
#pragma unroll
        for (int cc = 0; cc < CW; ++cc) cols[cc] = A + (long long)(c0 + cc) * lda;
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            const int r = tid + q * NT;
#pragma unroll
            for (int cc = 0; cc < CW; ++cc)
                if (r < m && pos[q] != r && c0 + cc < w) v[q][cc] = at(cols[cc], fresh(roff[q]));
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            const int r = tid + q * NT;
#pragma unroll
            for (int cc = 0; cc < CW; ++cc)
                if (r < m && pos[q] != r && c0 + cc < w)
                    at(cols[cc], (unsigned)pos[q] * (unsigned)sizeof(T)) = v[q][cc];
        }
        __syncthreads();
    }
    if (tid < w) p.ipiv[mat * p.sP + j0 + tid] = j0 + srec[tid] + 1;
    if (tid == 0) {
        int* ip = p.info + mat;
        if (j0 == 0) *ip = info;
        else if (info != 0 && *ip == 0) *ip = info;
    }
}

// NW wavefronts (four or eight), RPT rows per thread (row = tid + 64 NW q),
// ONE work-group barrier per column: each wavefront finds its argmax (rows of
// a lane first, then DPP and readlane across lanes) and publishes key,
// position and candidate row to a double-buffered LDS slot; every thread reads
// the NW slots and picks the winner.  Fewer, fuller wavefronts than one row
// per thread: the per-step overhead (reduction, exchange, reciprocal) is paid
// by four or eight wavefronts instead of up to sixteen.
template <typename T, int RPT, int NW = 4>
__global__ void __launch_bounds__(64 * NW) panel4_kernel(Problem p, int j0, int w)
{
    using O = ops<T>;
    using R = typename O::R;
    using K = typename O::K;
    constexpr int NT = 64 * NW;
    const int m = p.n - j0;                 // panel height
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const long long mat = blockIdx.x;

    __shared__ K skey[2][NW];
    __shared__ int spos[2][NW];
    __shared__ __attribute__((aligned(16))) T cand[2][NW][NBP];
    __shared__ int srec[NBP];

    T* A = (T*)p.A + mat * p.sA + j0 + (long long)j0 * p.lda;   // panel origin

    T a[RPT][NBP];
    int pos[RPT];
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
        const int r = tid + q * NT;
        pos[q] = r < m ? r : 0x3fffffff;
#pragma unroll
        for (int c = 0; c < NBP; ++c) a[q][c] = (r < m && c < w) ? A[r + (long long)c * p.lda] : O::zero();
    }

    int info = 0;
#pragma unroll
    for (int jj = 0; jj < NBP; ++jj) {
        if (jj >= w) continue;
        const int buf = jj & 1;
        // a1: the lane's best row (lowest position among equal keys), then
        // the wavefront's
        K key = 0;
        int kp = 0x7fffffff, ks = 0;
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            const K kq = (pos[q] >= jj && pos[q] < m) ? (K)pivot_key(O::metric(a[q][jj])) : (K)0;
            const bool take = kq > key || (kq == key && pos[q] < kp);
            key = take ? kq : key;
            kp = take ? pos[q] : kp;
            ks = take ? q : ks;
        }
        K kmax;
        int win;
        wave_argmax(key, kp, kmax, win);
        if (__builtin_expect(win < 0, 0)) {
            if (lane == 0) {
                skey[buf][wave] = 0;
                spos[buf][wave] = 0x7fffffff;
            }
        } else if (lane == win) {
            skey[buf][wave] = kmax;
            spos[buf][wave] = kp;
#pragma unroll
            for (int q = 0; q < RPT; ++q) {
                if (q != ks) continue;
                if constexpr (O::is_complex) {
#pragma unroll
                    for (int c = 0; c < NBP; ++c)
                        if (c >= jj) cand[buf][wave][c] = a[q][c];
                } else {
                    // 16-byte pieces from the piece holding column jj on
                    typedef T vec_t __attribute__((ext_vector_type(16 / sizeof(T))));
                    constexpr int E = 16 / sizeof(T);
#pragma unroll
                    for (int c = 0; c < NBP; c += E) {
                        if (c + E <= jj) continue;
                        vec_t v;
#pragma unroll
                        for (int e = 0; e < E; ++e) v[e] = a[q][c + e];
                        *(vec_t*)&cand[buf][wave][c] = v;
                    }
                }
            }
        }
        lds_barrier();
        K kv[NW];
        int pv[NW];
        T cv[NW];
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            kv[v] = skey[buf][v];
            pv[v] = spos[buf][v];
            cv[v] = cand[buf][v][jj];
        }
        K best = kv[0];
        int ppos = pv[0], vb = 0;
        T piv = cv[0];
#pragma unroll
        for (int v = 1; v < NW; ++v) {
            const bool take = kv[v] > best || (kv[v] == best && pv[v] < ppos);
            best = take ? kv[v] : best;
            ppos = take ? pv[v] : ppos;
            vb = take ? v : vb;
            piv = take ? cv[v] : piv;
        }
        // the pivot row through one VGPR base and immediate offsets
        typedef __attribute__((address_space(3))) const T lds_t;
        uint32_t rowaddr = (uint32_t)(uintptr_t)(lds_t*)&cand[buf][vb][0];
        asm volatile("" : "+v"(rowaddr));
        lds_t* row = (lds_t*)(uintptr_t)rowaddr;
        T u[NBP];
#pragma unroll
        for (int c = 0; c < NBP; ++c) {
            if constexpr (O::is_complex) {
                if (c > jj) u[c] = cand[buf][vb][c];
            } else {
                if (c > jj) u[c] = row[c];
            }
        }
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            if (pos[q] == ppos) srec[jj] = ppos;   // the pivot row's owner records it
            pos[q] = (pos[q] == ppos) ? jj : (pos[q] == jj ? ppos : pos[q]);
        }
        const R pm = O::metric(piv);
        const bool zero = pm == R(0);
        if (zero && info == 0) info = j0 + jj + 1;
        const T r = O::recip(piv);
        const bool small = !(pm >= O::sfmin());
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            if (pos[q] > jj && pos[q] < m && !zero) {
                T l = O::mul(a[q][jj], r);
                if (__builtin_expect(__builtin_amdgcn_ballot_w64(small) != 0, 0)) {
                    asm volatile("" ::: "memory");
                    if (small) l = O::div(a[q][jj], piv);
                }
                a[q][jj] = l;
#pragma unroll
                for (int c = 0; c < NBP; ++c)
                    if (c > jj) O::fms(a[q][c], l, u[c]);
            }
        }
    }
    __syncthreads();
    // rows to their final positions; ipiv as global 1-based rows
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
        const int r = tid + q * NT;
        if (r < m)
#pragma unroll
            for (int c = 0; c < NBP; ++c)
                if (c < w) A[pos[q] + (long long)c * p.lda] = a[q][c];
    }
    if (tid < w) p.ipiv[mat * p.sP + j0 + tid] = j0 + srec[tid] + 1;
    if (tid == 0) {
        int* ip = p.info + mat;
        if (j0 == 0) *ip = info;
        else if (info != 0 && *ip == 0) *ip = info;
    }
}

// ---------------------------------------------------------------------------
// interchange bookkeeping shared by the right-swap solve: destination rows
// of the panel's transpositions and the source row of each (a backward trace
// through the panel's interchange list).  Rows are relative to j0.
// ---------------------------------------------------------------------------
__device__ inline int trace_back(const int* sp, int w, int x) {
    for (int s = w - 1; s >= 0; --s) {
        const int ps = sp[s];
        x = (x == s) ? ps : (x == ps ? s : x);
    }
    return x;
}

// Solve with the 32 x 32 diagonal block of op(T) for columns [c0, c0 + 64)
// of X, where op(T) is T (aop 0), T^T (aop 1) or T^H (aop 2):
//   lower, unit diagonal: x_f -= t_fm x_m, m ascending;
//   lower: x_m /= t_mm then x_f -= t_fm x_m, m ascending;
//   upper: x_m /= t_mm then x_f -= t_fm x_m, m descending;
//   upper, unit diagonal: x_f -= t_fm x_m, m descending.
// With `swap` the rows of X are first permuted by the w transpositions in
// ipiv[j0 .. j0 + w) (getrf right-hand interchange): rows j0.. j0+w-1 get the
// solved values, displaced rows below are copied to their new places.
template <typename T, bool UPPER, bool UNIT>
__global__ void __launch_bounds__(64) trsm_block_kernel(const void* Tmat, int ldt, long long sT, void* Xmat,
                                                        int ldx, long long sX, int r0, int w, int ncols,
                                                        int ctiles, const int* ipiv, long long sP, bool swap,
                                                        const int* info, int aop)
{
    using O = ops<T>;
    __shared__ T tri[NBP][NBP + 1];
    __shared__ int sp[NBP];
    __shared__ int dst2[NBP];
    __shared__ int src_top[NBP], src_low[NBP];
    __shared__ int n2;
    const long long mat = blockIdx.x / ctiles;
    const int c0 = (int)(blockIdx.x % ctiles) * 64;
    const int tid = threadIdx.x;
    if (info && info[mat] != 0) return;   // composed gesv: failed factorisation keeps B
    const T* Tp = (const T*)Tmat + mat * sT + r0 + (long long)r0 * ldt;
    T* Xp = (T*)Xmat + mat * sX + r0;

    for (int e0 = tid; e0 < w * w; e0 += 64 * 8) {   // loads batched
        T v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + u * 64;
            if (e < w * w) v[u] = Tp[(e % w) + (long long)(e / w) * ldt];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + u * 64;
            if (e >= w * w) continue;
            if (aop == 0) {
                tri[e % w][e / w] = v[u];
            } else {
                T x = v[u];
                if constexpr (O::is_complex) {
                    if (aop == 2) x.im = -x.im;
                }
                tri[e / w][e % w] = x;
            }
        }
    }
    if (swap) {
        if (tid < w) sp[tid] = ipiv[mat * sP + r0 + tid] - 1 - r0;
        if (tid == 0) n2 = 0;
        __syncthreads();
        if (tid < w) {
            src_top[tid] = trace_back(sp, w, tid);
            const int ps = sp[tid];
            bool first = ps >= w;
            for (int s = 0; s < tid && first; ++s) first = sp[s] != ps;
            if (first) {
                const int slot = atomicAdd(&n2, 1);
                dst2[slot] = ps;
                src_low[slot] = trace_back(sp, w, ps);
            }
        }
    }
    __syncthreads();

    const int c = c0 + tid;
    if (c >= ncols) return;
    T* col = Xp + (long long)c * ldx;
    T x[NBP];
    T moved[NBP];
    const int nmove = swap ? n2 : 0;
#pragma unroll
    for (int f = 0; f < NBP; ++f) {
        if (f < w) x[f] = swap ? col[src_top[f]] : col[f];
        if (f < nmove) moved[f] = col[src_low[f]];
    }
    if (!UPPER) {
        // in getrf (swap), a step whose pivot is exactly zero took no rank-1
        // update in the unblocked order, so its column of L11 is left out
#pragma unroll
        for (int mm = 0; mm < NBP; ++mm) {
            if (mm >= w) continue;
            if (swap && O::metric(tri[mm][mm]) == typename O::R(0)) continue;
            if (!UNIT) x[mm] = O::div(x[mm], tri[mm][mm]);
#pragma unroll
            for (int f = 0; f < NBP; ++f)
                if (f > mm && f < w) O::fms(x[f], tri[f][mm], x[mm]);
        }
    } else {
#pragma unroll
        for (int mm = NBP - 1; mm >= 0; --mm) {
            if (mm >= w) continue;
            if (!UNIT) x[mm] = O::div(x[mm], tri[mm][mm]);
#pragma unroll
            for (int f = 0; f < NBP; ++f)
                if (f < mm) O::fms(x[f], tri[f][mm], x[mm]);
        }
    }
#pragma unroll
    for (int f = 0; f < NBP; ++f) {
        if (f < w) col[f] = x[f];
        if (f < nmove) col[dst2[f]] = moved[f];
    }
}

// ---------------------------------------------------------------------------
// C[M x N] -= A[M x K] * B[K x N], K <= 32, per matrix of the batch.  k runs
// ascending (kdir > 0) or descending (kdir < 0); each element sees one fused
// multiply-add per k in that order.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));
// row inside a 16x16 MFMA output block held by (lane group lk, register r)
template <typename T>
__device__ inline int mfma_row_t(int lk, int r) {
    return sizeof(T) == 4 ? 4 * lk + r : lk + 4 * r;
}
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ inline void tile_load(T (*As)[TT], T (*Bs)[TT], const T* Ap, int lda_, const T* Bp, int ldb_,
                                 int M, int N, int K, int tid, int nthr, bool negate, int aop = 0)
{
    using O = ops<T>;
    // op(A) element (i, k) is Ap[i + k lda] (aop 0), or Ap[k + i lda] (aop 1),
    // conjugated for aop 2; the transposed read walks k fastest so that it
    // stays coalesced.  Loads issued in batches of eight per thread before
    // their LDS stores.
    for (int e0 = tid; e0 < TT * K; e0 += nthr * 8) {
        T va[8], vb[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + u * nthr;
            if (e < TT * K) {
                if (aop == 0) {
                    const int i = e % TT, k = e / TT;
                    va[u] = i < M ? Ap[i + (long long)k * lda_] : O::zero();
                } else {
                    const int k = e % K, i = e / K;
                    va[u] = i < M ? Ap[k + (long long)i * lda_] : O::zero();
                }
                const int k2 = e % K, j = e / K;
                vb[u] = j < N ? Bp[k2 + (long long)j * ldb_] : O::zero();
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + u * nthr;
            if (e < TT * K) {
                T v = va[u];
                if constexpr (O::is_complex) {
                    if (aop == 2) v.im = -v.im;
                }
                if (negate) {
                    if constexpr (O::is_complex) { v.re = -v.re; v.im = -v.im; }
                    else v = -v;
                }
                if (aop == 0) As[e / TT][e % TT] = v;
                else As[e % K][e / K] = v;
                Bs[e % K][e / K] = vb[u];
            }
        }
    }
}

// MFMA version for float and double: 4 waves, each a 32 x 32 quarter of the
// 64 x 64 tile made of 2 x 2 blocks of 16 x 16.
// U12 = L11^-1 (P A12) for the getrf trailing columns, through an LDS stage:
// the new top rows are gathered 32 lanes down each column (coalesced), the
// displaced rows move with one lane per moved row, one thread per column
// solves with L11 from LDS (ascending m; a zero pivot's column is left out,
// as in the unblocked order), and the stage is written back down each column.
// One wavefront per 32-column tile (its first 32 lanes solve; all 64 gather
// and write back): many small work-groups per compute unit overlap each
// other's memory latency, and the barriers are a wavefront's.  32 columns
// rather than 64 double the work-groups of the late, narrow steps (getrf
// 0.7 - 1.3 % faster at n = 384 - 2048).
template <typename T>
struct StageTile {
    static constexpr int TC = 32;   // columns per work-group (64 threads)
};

template <typename T>
__global__ void __launch_bounds__(64) trsm_stage_kernel(Problem p, int r0, int ncols, int ctiles)
{
    using O = ops<T>;
    using R = typename O::R;
    constexpr int NT = 64;
    constexpr int TC = StageTile<T>::TC;
    __shared__ T S[NBP][TC + 1];
    __shared__ T l11[NBP][NBP];              // transposed: l11[m][f] = l_fm
    __shared__ int src_top[NBP], src_low[NBP], dst_low[NBP];
    __shared__ int nlow;
    __shared__ unsigned zmask;
    const int tid = threadIdx.x;
    const long long mat = blockIdx.x / ctiles;
    const int c0 = (int)(blockIdx.x % ctiles) * TC;
    const int ct = min(TC, ncols - c0);
    const long long lda = p.lda;
    T* A = (T*)p.A + mat * p.sA;
    T* X = A + r0 + (long long)(r0 + NBP + c0) * lda;        // top-left of this tile's P A12 block
    const T* D = A + r0 + (long long)r0 * lda;                // L11 / U11 block
    if (tid == 0) {
        nlow = 0;
        zmask = 0;
    }
    {
        constexpr int PER = NBP * NBP / NT;   // loads per thread, issued together
        T v[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + u * NT;
            v[u] = D[(e % NBP) + (e / NBP) * lda];
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + u * NT;
            l11[e / NBP][e % NBP] = v[u];
        }
    }
    __syncthreads();
    if (tid < NBP) {
        int sp[NBP];
#pragma unroll
        for (int s2 = 0; s2 < NBP; ++s2) sp[s2] = p.ipiv[mat * p.sP + r0 + s2] - 1 - r0;
        int x = tid;
#pragma unroll
        for (int s2 = NBP - 1; s2 >= 0; --s2) x = (x == s2) ? sp[s2] : (x == sp[s2] ? s2 : x);
        src_top[tid] = x;
        const int ps = p.ipiv[mat * p.sP + r0 + tid] - 1 - r0;
        bool first = ps >= NBP;
#pragma unroll
        for (int s2 = 0; s2 < NBP; ++s2)
            if (s2 < tid && sp[s2] == ps) first = false;
        if (first) {
            int y = ps;
#pragma unroll
            for (int s2 = NBP - 1; s2 >= 0; --s2) y = (y == s2) ? sp[s2] : (y == sp[s2] ? s2 : y);
            const int slot = atomicAdd(&nlow, 1);
            dst_low[slot] = ps;
            src_low[slot] = y;
        }
        if (O::metric(l11[tid][tid]) == R(0)) atomicOr(&zmask, 1u << tid);
    }
    __syncthreads();
    // (1) the new top rows into the stage (loads batched: one round trip
    //     per eight elements per thread, not one per element)
    for (int e0 = tid; e0 < NBP * ct; e0 += NT * 8) {
        T v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + u * NT;
            if (e < NBP * ct) v[u] = X[src_top[e % NBP] + (long long)(e / NBP) * lda];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + u * NT;
            if (e < NBP * ct) S[e % NBP][e / NBP] = v[u];
        }
    }
    __syncthreads();
    // (2) displaced rows: old top rows to their new places below
    {
        const int nl = nlow;
        const int q = tid & (NBP - 1);
        if (q < nl) {
            const int srow = src_low[q], drow = dst_low[q];
            for (int c00 = tid >> 5; c00 < ct; c00 += (NT / NBP) * 8) {
                T v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int c = c00 + u * (NT / NBP);
                    if (c < ct) v[u] = X[srow + (long long)c * lda];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int c = c00 + u * (NT / NBP);
                    if (c < ct) X[drow + (long long)c * lda] = v[u];
                }
            }
        }
    }
    // (3) one thread per column
    const unsigned zm = zmask;
    if (tid < ct) {
        T x[NBP];
#pragma unroll
        for (int f = 0; f < NBP; ++f) x[f] = S[f][tid];
        if (zm == 0) {
#pragma unroll
            for (int mm = 0; mm < NBP; ++mm) {
#pragma unroll
                for (int f = 0; f < NBP; ++f)
                    if (f > mm) O::fms(x[f], l11[mm][f], x[mm]);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int mm = 0; mm < NBP; ++mm) {
                const bool skip = (zm >> mm) & 1u;
#pragma unroll
                for (int f = 0; f < NBP; ++f)
                    if (f > mm && !skip) O::fms(x[f], l11[mm][f], x[mm]);
            }
        }
#pragma unroll
        for (int f = 0; f < NBP; ++f) S[f][tid] = x[f];
    }
    __syncthreads();
    // (4) U12 down each column
    for (int e = tid; e < NBP * ct; e += NT) {
        const int f = e % NBP, c = e / NBP;
        X[f + (long long)c * lda] = S[f][c];
    }
}

template <typename T>
__global__ void __launch_bounds__(256) gemm_mfma_kernel(const void* Am, int lda_, long long sA, const void* Bm,
                                                        int ldb_, long long sB, void* Cm, int ldc, long long sC,
                                                        int M, int N, int K, int mtiles, int ntiles, int kdir,
                                                        const int* info, int aop)
{
    __shared__ T As[NBP][TT];
    __shared__ T Bs[NBP][TT];
    const int tiles = mtiles * ntiles;
    const long long mat = blockIdx.x / tiles;
    const int t = (int)(blockIdx.x % tiles);
    const int i0 = (t % mtiles) * TT, jt0 = (t / mtiles) * TT;
    if (info && info[mat] != 0) return;
    const T* Ap = (const T*)Am + mat * sA + (aop ? (long long)i0 * lda_ : (long long)i0);
    const T* Bp = (const T*)Bm + mat * sB + (long long)jt0 * ldb_;
    T* Cp = (T*)Cm + mat * sC + i0 + (long long)jt0 * ldc;
    const int Mt = min(TT, M - i0), Nt = min(TT, N - jt0);
    tile_load<T>(As, Bs, Ap, lda_, Bp, ldb_, Mt, Nt, K, threadIdx.x, 256, true, aop);
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wr = (wave & 1) * 32, wc = (wave >> 1) * 32;
    const int li = lane & 15, lk = lane >> 4;
    using V = typename std::conditional<sizeof(T) == 4, f32x4, f64x4>::type;
    V acc[2][2];
    // load C into the accumulator layout
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = wr + bi * 16 + (sizeof(T) == 4 ? 4 * lk + r : lk + 4 * r);
                const int j = wc + bj * 16 + li;
                acc[bi][bj][r] = (i < Mt && j < Nt) ? Cp[i + (long long)j * ldc] : T(0);
            }
    const int K4 = K & ~3;
    for (int s = 0; s < K4 / 4; ++s) {
        // ascending: k groups 0..; descending: from the top, reversed inside
        const int kk = kdir > 0 ? 4 * s + lk : K - 1 - (4 * s + lk);
        T av[2], bv[2];
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) av[bi] = As[kk][wr + bi * 16 + li];
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) bv[bj] = Bs[kk][wc + bj * 16 + li];
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < 2; ++bj) {
                if constexpr (sizeof(T) == 4)
                    acc[bi][bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[bi], bv[bj], acc[bi][bj], 0, 0, 0);
                else
                    acc[bi][bj] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[bi], bv[bj], acc[bi][bj], 0, 0, 0);
            }
    }
    // remaining k (fewer than 4) on the VALU, continuing the same order
    for (int s = K4; s < K; ++s) {
        const int kk = kdir > 0 ? s : K - 1 - s;
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < 2; ++bj)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = wr + bi * 16 + (sizeof(T) == 4 ? 4 * lk + r : lk + 4 * r);
                    const int j = wc + bj * 16 + li;
                    if constexpr (sizeof(T) == 4) acc[bi][bj][r] = __builtin_fmaf(As[kk][i], Bs[kk][j], acc[bi][bj][r]);
                    else acc[bi][bj][r] = __builtin_fma(As[kk][i], Bs[kk][j], acc[bi][bj][r]);
                }
    }
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = wr + bi * 16 + (sizeof(T) == 4 ? 4 * lk + r : lk + 4 * r);
                const int j = wc + bj * 16 + li;
                if (i < Mt && j < Nt) Cp[i + (long long)j * ldc] = acc[bi][bj][r];
            }
}

// Work-group -> (matrix, strip).  Work-groups are dealt to the eight XCDs in
// turn; when the batch is a multiple of eight, the strips of one matrix go
// to one XCD, so they read its U12 through one L2.
__device__ inline void strip_of(int mstrips, long long& mat, int& strip) {
    const unsigned b = blockIdx.x, batch = gridDim.x / (unsigned)mstrips;
    if (mstrips > 1 && (batch & 7) == 0) {
        const unsigned slot = b >> 3;
        mat = (long long)(slot / (unsigned)mstrips) * 8 + (b & 7);
        strip = (int)(slot % (unsigned)mstrips);
    } else {
        mat = b / (unsigned)mstrips;
        strip = (int)(b % (unsigned)mstrips);
    }
}

// getrf trailing update A22 -= L21 U12 (real types, K = 32, ascending k): one
// work-group per 64-row strip of one matrix walks the strip's 64-column
// tiles.  L21 stays in registers as MFMA operands for the whole strip; the
// next U12 tile is staged into LDS and the next C tile loaded while the
// current one runs on the matrix cores.  Computed as C^T += U12^T (-L21)^T so
// that an accumulator register holds 16 consecutive rows of one column.  A
// zero pivot among the panel's 32 (a zero diagonal entry of U11) leaves its
// k out, on the VALU, as in the unblocked order.
// The update covers the columns [c0, c0 + N) of A22 (all M rows), so that
// the next panel's columns can be updated first and the rest later.
template <typename T>
__global__ void __launch_bounds__(256) update_strip_kernel(T* A, int lda, long long sA, int j0, int M, int c0, int N,
                                                           int mstrips)
{
    using O = ops<T>;
    using R = typename O::R;
    using V = typename std::conditional<sizeof(T) == 4, f32x4, f64x4>::type;
    constexpr int UP = 64 + (sizeof(T) == 4 ? 4 : 2);       // padded row of the U tile
    __shared__ __attribute__((aligned(16))) T Us[2][NBP][UP];
    __shared__ unsigned zmask;
    const int tid = threadIdx.x;
    long long mat;
    int r0;
    strip_of(mstrips, mat, r0);
    r0 *= 64;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave & 1, wc = wave >> 1;
    const int li = lane & 15, lk = lane >> 4;
    T* base = A + mat * sA;
    const T* Lp = base + j0 + NBP + (long long)j0 * lda;             // L21
    const T* Up = base + j0 + (long long)(j0 + NBP + c0) * lda;      // U12, columns c0 ..
    T* Cp = base + j0 + NBP + (long long)(j0 + NBP + c0) * lda;      // A22, columns c0 ..
    const int nct = (N + 63) / 64;
    if (tid == 0) zmask = 0;
    __syncthreads();
    if (tid < NBP && O::metric(base[j0 + tid + (long long)(j0 + tid) * lda]) == R(0)) atomicOr(&zmask, 1u << tid);
    // the first U tile into the stage
    auto load_u = [&](int ct, T (&v)[8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = tid + 256 * u, k = e & (NBP - 1), c = ct * 64 + (e >> 5);
            v[u] = c < N ? Up[k + (long long)c * lda] : O::zero();
        }
    };
    auto put_u = [&](int b, const T (&v)[8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = tid + 256 * u;
            Us[b][e & (NBP - 1)][e >> 5] = v[u];
        }
    };
    {
        T v[8];
        load_u(0, v);
        put_u(0, v);
    }
    __syncthreads();
    if (zmask != 0) {
        // a zero pivot in this panel: plain k loop without that k (rare)
#pragma unroll 1
        for (int e = tid; e < 64 * N; e += 256) {
            const int i = r0 + (e & 63), j = e >> 6;
            if (i >= M) continue;
            T c = Cp[i + (long long)j * lda];
#pragma unroll 1
            for (int k = 0; k < NBP; ++k)
                if (!((zmask >> k) & 1u)) O::fms(c, Lp[i + (long long)k * lda], Up[k + (long long)j * lda]);
            Cp[i + (long long)j * lda] = c;
        }
        return;
    }
    // L21 operands of this wavefront's two 16-row blocks, negated
    T lv[2][NBP / 4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int i = r0 + wr * 32 + t * 16 + li;
#pragma unroll
        for (int s2 = 0; s2 < NBP / 4; ++s2) lv[t][s2] = i < M ? -Lp[i + (long long)(4 * s2 + lk) * lda] : O::zero();
    }
    auto load_c = [&](int ct, V (&c)[2][2]) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = r0 + wr * 32 + t * 16 + li;
                    const int j = ct * 64 + wc * 32 + b * 16 + mfma_row_t<T>(lk, r);
                    c[t][b][r] = (i < M && j < N) ? Cp[i + (long long)j * lda] : O::zero();
                }
    };
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
                    const int j = ct * 64 + wc * 32 + b * 16 + mfma_row_t<T>(lk, r);
                    if (i < M && j < N) Cp[i + (long long)j * lda] = acc[r];
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

// Complex getrf trailing update A22 -= L21 U12 on real MFMAs (K = 32
// complex steps, ascending).  A complex z -= x*y is four real fused
// multiply-adds in a fixed order (GEMM page, POD complex paragraph): the real
// part takes -xr*yr then +xi*yi, the imaginary part -xr*yi then -xi*yr.
// Interleaving each complex k into two real k' = 2k + h turns both parts
// into real products whose terms arrive in exactly that order:
//   re: sum over k' of Ure[c][k'] * Lre[k'][i], Ure = (u.re, u.im), Lre = (-l.re, l.im)
//   im: sum over k' of Uim[c][k'] * Lim[k'][i], Uim = (u.im, u.re), Lim = (-l.re, -l.im)
// and an MFMA chain in ascending k' accumulates like a chain of fused
// multiply-adds in k' order, so every element sees the unblocked operation
// sequence.  Same C^T arrangement and strip walk as update_strip_kernel: one
// work-group per strip of 32*TB rows walks the strip's 64-column tiles, the
// L operands stay in registers, the next U tile is staged into LDS and the
// next C tile loaded while the current one runs.  A zero pivot among the
// panel's 32 leaves its k out on the VALU, as in the unblocked order.
template <typename R>
struct CplxStrip {
    static constexpr int TB = sizeof(R) == 4 ? 2 : 1;   // 16-row blocks per wavefront
    static constexpr int SH = 32 * TB;                   // strip height
};

template <typename R>
__global__ void __launch_bounds__(256) update_strip_cplx_kernel(cplx<R>* A, int lda, long long sA, int j0, int M,
                                                                int c0, int N, int mstrips)
{
    using T = cplx<R>;
    using O = ops<T>;
    using V = typename std::conditional<sizeof(R) == 4, f32x4, f64x4>::type;
    constexpr int TB = CplxStrip<R>::TB, SH = CplxStrip<R>::SH;
    constexpr int KP = 2 * NBP;                              // real k' per panel
    constexpr int UP = 64 + (sizeof(R) == 4 ? 2 : 1);         // padded row of a staged U tile
    __shared__ __attribute__((aligned(16))) T Us[2][NBP][UP];
    __shared__ unsigned zmask;
    const int tid = threadIdx.x;
    long long mat;
    int r0;
    strip_of(mstrips, mat, r0);
    r0 *= SH;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave & 1, wc = wave >> 1;
    const int li = lane & 15, lk = lane >> 4;
    const bool hodd = (lk & 1) != 0;                          // this lane's k' = 2k + 1
    T* base = A + mat * sA;
    const T* Lp = base + j0 + NBP + (long long)j0 * lda;             // L21
    const T* Up = base + j0 + (long long)(j0 + NBP + c0) * lda;      // U12, columns c0 ..
    T* Cp = base + j0 + NBP + (long long)(j0 + NBP + c0) * lda;      // A22, columns c0 ..
    const int nct = (N + 63) / 64;
    if (tid == 0) zmask = 0;
    __syncthreads();
    if (tid < NBP && O::metric(base[j0 + tid + (long long)(j0 + tid) * lda]) == R(0)) atomicOr(&zmask, 1u << tid);
    // a U tile (32 complex rows x 64 columns) into the stage
    auto load_u = [&](int ct, T (&v)[8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = tid + 256 * u, k = e & (NBP - 1), c = ct * 64 + (e >> 5);
            v[u] = c < N ? Up[k + (long long)c * lda] : O::zero();
        }
    };
    auto put_u = [&](int b, const T (&v)[8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = tid + 256 * u;
            Us[b][e & (NBP - 1)][e >> 5] = v[u];
        }
    };
    {
        T v[8];
        load_u(0, v);
        put_u(0, v);
    }
    __syncthreads();
    if (zmask != 0) {
        // a zero pivot in this panel: plain k loop without that k (rare)
#pragma unroll 1
        for (int e = tid; e < SH * N; e += 256) {
            const int i = r0 + e % SH, j = e / SH;
            if (i >= M) continue;
            T c = Cp[i + (long long)j * lda];
#pragma unroll 1
            for (int k = 0; k < NBP; ++k)
                if (!((zmask >> k) & 1u)) O::fms(c, Lp[i + (long long)k * lda], Up[k + (long long)j * lda]);
            Cp[i + (long long)j * lda] = c;
        }
        return;
    }
    // L21 operands of this wavefront's row blocks: lane (li, lk) holds row
    // i = block + li at k' = 4 s2 + lk, i.e. complex k = 2 s2 + lk / 2
    R lre[TB][KP / 4], lim[TB][KP / 4];
#pragma unroll
    for (int t = 0; t < TB; ++t) {
        const int i = r0 + wr * 16 * TB + t * 16 + li;
#pragma unroll
        for (int s2 = 0; s2 < KP / 4; ++s2) {
            const int k = 2 * s2 + (lk >> 1);
            const T l = i < M ? Lp[i + (long long)k * lda] : O::zero();
            lre[t][s2] = hodd ? l.im : -l.re;
            lim[t][s2] = hodd ? -l.im : -l.re;
        }
    }
    auto load_c = [&](int ct, V (&cr)[TB][2], V (&ci)[TB][2]) {
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = r0 + wr * 16 * TB + t * 16 + li;
                    const int j = ct * 64 + wc * 32 + b * 16 + mfma_row_t<R>(lk, r);
                    const T z = (i < M && j < N) ? Cp[i + (long long)j * lda] : O::zero();
                    cr[t][b][r] = z.re;
                    ci[t][b][r] = z.im;
                }
    };
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
            // k' = 4 s2 + lk is complex k = 2 s2 + lk / 2, part lk % 2
            R ur[KP / 4], ui[KP / 4];
#pragma unroll
            for (int s2 = 0; s2 < KP / 4; ++s2) {
                const T z = Us[buf][2 * s2 + (lk >> 1)][c];
                ur[s2] = hodd ? z.im : z.re;
                ui[s2] = hodd ? z.re : z.im;
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
                    const int j = ct * 64 + wc * 32 + b * 16 + mfma_row_t<R>(lk, r);
                    if (i < M && j < N) Cp[i + (long long)j * lda] = T{accr[r], acci[r]};
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

// VALU version (complex types): each thread owns a 4 x 4 block of the tile.
// With Dm (the getrf trailing update) a k whose pivot -- diagonal entry k of
// the K x K block at Dm -- is exactly zero is left out, as in the unblocked
// order, which skips the rank-1 update of such a step.
template <typename T>
__global__ void __launch_bounds__(256) gemm_valu_kernel(const void* Am, int lda_, long long sA, const void* Bm,
                                                        int ldb_, long long sB, void* Cm, int ldc, long long sC,
                                                        int M, int N, int K, int mtiles, int ntiles, int kdir,
                                                        const int* info, const void* Dm, int ldd, long long sD,
                                                        int aop)
{
    using O = ops<T>;
    __shared__ T As[NBP][TT];
    __shared__ T Bs[NBP][TT];
    __shared__ unsigned zmask_s;
    const int tiles = mtiles * ntiles;
    const long long mat = blockIdx.x / tiles;
    const int t = (int)(blockIdx.x % tiles);
    const int i0 = (t % mtiles) * TT, jt0 = (t / mtiles) * TT;
    if (info && info[mat] != 0) return;
    const T* Ap = (const T*)Am + mat * sA + (aop ? (long long)i0 * lda_ : (long long)i0);
    const T* Bp = (const T*)Bm + mat * sB + (long long)jt0 * ldb_;
    T* Cp = (T*)Cm + mat * sC + i0 + (long long)jt0 * ldc;
    const int Mt = min(TT, M - i0), Nt = min(TT, N - jt0);
    if (threadIdx.x < 64) {
        bool z = false;
        if (Dm && (int)threadIdx.x < K) {
            const T* D = (const T*)Dm + mat * sD;
            z = O::metric(D[threadIdx.x + (long long)threadIdx.x * ldd]) == typename O::R(0);
        }
        const uint64_t zb = __builtin_amdgcn_ballot_w64(z);
        if (threadIdx.x == 0) zmask_s = (unsigned)zb;
    }
    tile_load<T>(As, Bs, Ap, lda_, Bp, ldb_, Mt, Nt, K, threadIdx.x, 256, false, aop);
    __syncthreads();
    const unsigned zm = zmask_s;
    const int ti = (threadIdx.x % 16) * 4, tj = (threadIdx.x / 16) * 4;
    T c[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int i = ti + a, j = tj + b;
            c[a][b] = (i < Mt && j < Nt) ? Cp[i + (long long)j * ldc] : O::zero();
        }
    for (int s = 0; s < K; ++s) {
        const int kk = kdir > 0 ? s : K - 1 - s;
        if ((zm >> kk) & 1u) continue;
        T av[4], bv[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) av[a] = As[kk][ti + a];
#pragma unroll
        for (int b = 0; b < 4; ++b) bv[b] = Bs[kk][tj + b];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) O::fms(c[a][b], av[a], bv[b]);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int i = ti + a, j = tj + b;
            if (i < Mt && j < Nt) Cp[i + (long long)j * ldc] = c[a][b];
        }
}

// ---------------------------------------------------------------------------
// deferred left interchanges: after the last panel, the L columns of every
// panel k are gathered through the interchanges of all later steps.  One
// work-group per (matrix, panel): each of its rows at or below the first
// later step finds its source by tracing itself back through those steps
// (LDS copy of ipiv), then the panel's columns move a few at a time, every
// read of a round before any write of it.
// ---------------------------------------------------------------------------
template <typename T, int RPT>
__global__ void __launch_bounds__(1024) left_swap_kernel(Problem p, int npan)
{
    extern __shared__ int sipiv[];   // steps lo .. n-1, 0-based rows
    const int n = p.n;
    const int tid = threadIdx.x, nt = blockDim.x;
    const long long mat = blockIdx.x / npan;
    const int k = (int)(blockIdx.x % npan);        // panel
    const int lo = (k + 1) * NBP;                   // first row the later steps touch
    T* A = (T*)p.A + mat * p.sA;
    for (int i = lo + tid; i < n; i += nt) sipiv[i - lo] = p.ipiv[mat * p.sP + i] - 1;
    __syncthreads();
    int map[RPT];
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
        const int i = lo + tid + q * nt;
        int x = i;
        if (i < n) {
            // eight steps per round: their LDS reads are in flight together
            int s = n - 1;
            for (; s - 7 >= lo; s -= 8) {
                int ps[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) ps[u] = sipiv[s - u - lo];
#pragma unroll
                for (int u = 0; u < 8; ++u) x = (x == s - u) ? ps[u] : (x == ps[u] ? s - u : x);
            }
            for (; s >= lo; --s) {
                const int ps = sipiv[s - lo];
                x = (x == s) ? ps : (x == ps ? s : x);
            }
        }
        map[q] = x;
    }
    const int c0 = k * NBP;
    constexpr int CC = RPT >= 4 ? 4 : 8;   // columns per read/write round (four rows a thread: 4, no spill)
    for (int cb = 0; cb < NBP; cb += CC) {
        T v[RPT][CC];
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            const int i = lo + tid + q * nt;
#pragma unroll
            for (int c = 0; c < CC; ++c)
                if (i < n && map[q] != i) v[q][c] = A[map[q] + (long long)(c0 + cb + c) * p.lda];
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            const int i = lo + tid + q * nt;
#pragma unroll
            for (int c = 0; c < CC; ++c)
                if (i < n && map[q] != i) A[i + (long long)(c0 + cb + c) * p.lda] = v[q][c];
        }
        __syncthreads();
    }
}

// B <- P B: position i receives the row the full interchange sequence brings
// there (a backward trace of ipiv per row), column by column through LDS.
// With `reverse`, B <- P^T B: the interchanges applied last to first, so the
// trace runs forward.
template <typename T>
__global__ void __launch_bounds__(1024) permute_rows_kernel(Problem p, bool reverse)
{
    extern __shared__ int smem[];
    const int n = p.n;
    int* sipiv = smem;
    int* src = smem + n;
    const int tid = threadIdx.x, nt = blockDim.x;
    const long long mat = blockIdx.x;
    if (p.info && p.info[mat] != 0) return;
    for (int i = tid; i < n; i += nt) {   // entries outside 1..n: no interchange
        const int v = p.ipiv[mat * p.sP + i] - 1;
        sipiv[i] = (v >= 0 && v < n) ? v : i;
    }
    __syncthreads();
    for (int i = tid; i < n; i += nt) {
        int x = i;
        for (int q = 0; q < n; ++q) {
            const int s = reverse ? q : n - 1 - q;
            const int ps = sipiv[s];
            x = (x == s) ? ps : (x == ps ? s : x);
        }
        src[i] = x;
    }
    __syncthreads();
    T* B = (T*)p.B + mat * p.sB;
    T* stage = (T*)(smem + 2 * n + ((2 * n) & 3 ? 4 - ((2 * n) & 3) : 0));
    for (int c = 0; c < p.nrhs; ++c) {
        T* col = B + (long long)c * p.ldb;
        for (int i = tid; i < n; i += nt) stage[i] = col[src[i]];
        __syncthreads();
        for (int i = tid; i < n; i += nt) col[i] = stage[i];
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// host drivers
// ---------------------------------------------------------------------------
inline int panel_threads(int m) {
    const int t = ((m + 63) / 64) * 64;
    return t > 1024 ? 1024 : t;
}

// Threads per panel work-group: one row per thread up to a per-type cap that
// keeps the panel rows (32 elements each) and the pivot row in VGPRs; taller
// panels give each thread up to four rows.
template <typename T>
constexpr int panel_cap() { return sizeof(T) == 4 ? 1024 : sizeof(T) == 8 ? 512 : 256; }

template <typename T>
hipError_t launch_panel(const Problem& p, int j0, int w, hipStream_t s) {
    constexpr int CAP = panel_cap<T>();
    const int m = p.n - j0;
    // four wavefronts with up to two rows per thread to 512 rows; real types
    // then eight wavefronts, two rows per thread to 1024 rows (float: four to
    // 2048).  Measured against four wavefronts with four rows: getrf n = 1024,
    // batch 64, 3.78 ms against 3.97 (float), 6.27 against 6.48 (double);
    // float n = 2048, batch 16, 8.83 against 9.77 (1024 threads, two rows each)
    if constexpr (sizeof(T) <= 8) {
        constexpr int CAP4 = ops<T>::is_complex ? 512 : sizeof(T) == 4 ? 2048 : 1024;
        if (m <= CAP4) {
            if (m <= 256) hipLaunchKernelGGL((panel4_kernel<T, 1>), dim3(p.batch), dim3(256), 0, s, p, j0, w);
            else if (m <= 512) hipLaunchKernelGGL((panel4_kernel<T, 2>), dim3(p.batch), dim3(256), 0, s, p, j0, w);
            else if constexpr (!ops<T>::is_complex) {
                if (m <= 1024)
                    hipLaunchKernelGGL((panel4_kernel<T, 2, 8>), dim3(p.batch), dim3(512), 0, s, p, j0, w);
                else if constexpr (sizeof(T) == 4)
                    hipLaunchKernelGGL((panel4_kernel<T, 4, 8>), dim3(p.batch), dim3(512), 0, s, p, j0, w);
            }
            return hipGetLastError();
        }
    }
    int nt = ((m + 63) / 64) * 64;
    if (nt > CAP) nt = CAP;
    const int rpt = (m + nt - 1) / nt;
    // beyond the registers the panel stays in memory (up to 4096 rows); for
    // complex double also where four rows a thread would spill (measured:
    // n = 1024, batch 32: 13.5 ms against 15.2; for the other types the
    // spilling register panel stays faster, by 3 - 30 %)
    if (rpt > (sizeof(T) >= 16 ? 2 : 4)) {
        if (m > 4096) return hipErrorInvalidValue;
        hipLaunchKernelGGL((panel_mem_kernel<T>), dim3(p.batch), dim3(1024), 0, s, p, j0, w);
        return hipGetLastError();
    }
    if (nt <= 256) {
        if (rpt <= 1) hipLaunchKernelGGL((panel_kernel<T, 1, 256>), dim3(p.batch), dim3(nt), 0, s, p, j0, w);
        else if (rpt <= 2) hipLaunchKernelGGL((panel_kernel<T, 2, 256>), dim3(p.batch), dim3(nt), 0, s, p, j0, w);
        else if (rpt <= 4) hipLaunchKernelGGL((panel_kernel<T, 4, 256>), dim3(p.batch), dim3(nt), 0, s, p, j0, w);
        else return hipErrorInvalidValue;
    } else {
        if (rpt <= 1) hipLaunchKernelGGL((panel_kernel<T, 1, CAP>), dim3(p.batch), dim3(nt), 0, s, p, j0, w);
        else if (rpt <= 2) hipLaunchKernelGGL((panel_kernel<T, 2, CAP>), dim3(p.batch), dim3(nt), 0, s, p, j0, w);
        else if (rpt <= 4) hipLaunchKernelGGL((panel_kernel<T, 4, CAP>), dim3(p.batch), dim3(nt), 0, s, p, j0, w);
        else return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_trsm(const void* Tm, int ldt, long long sT, void* X, int ldx, long long sX, int r0, int w,
                       int ncols, int batch, const int* ipiv, long long sP, bool swap, bool upper,
                       const int* info, hipStream_t s, bool unit, int aop = 0) {
    const int ct = (ncols + 63) / 64;
    const dim3 grid((unsigned)((long long)ct * batch));
    if (upper && !unit)
        hipLaunchKernelGGL((trsm_block_kernel<T, true, false>), grid, dim3(64), 0, s, Tm, ldt, sT, X, ldx, sX, r0,
                           w, ncols, ct, ipiv, sP, swap, info, aop);
    else if (upper)
        hipLaunchKernelGGL((trsm_block_kernel<T, true, true>), grid, dim3(64), 0, s, Tm, ldt, sT, X, ldx, sX, r0,
                           w, ncols, ct, ipiv, sP, swap, info, aop);
    else if (unit)
        hipLaunchKernelGGL((trsm_block_kernel<T, false, true>), grid, dim3(64), 0, s, Tm, ldt, sT, X, ldx, sX, r0,
                           w, ncols, ct, ipiv, sP, swap, info, aop);
    else
        hipLaunchKernelGGL((trsm_block_kernel<T, false, false>), grid, dim3(64), 0, s, Tm, ldt, sT, X, ldx, sX, r0,
                           w, ncols, ct, ipiv, sP, swap, info, aop);
    return hipGetLastError();
}

// Dm (complex getrf trailing update only): the panel's K x K diagonal block,
// whose exactly-zero diagonal entries mark the k to leave out.
template <typename T>
hipError_t launch_gemm(const void* Am, int lda_, long long sA, const void* Bm, int ldb_, long long sB, void* Cm,
                       int ldc, long long sC, int M, int N, int K, int batch, int kdir, const int* info,
                       hipStream_t s, const void* Dm = nullptr, int ldd = 0, long long sD = 0, int aop = 0) {
    if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
    const int mt = (M + TT - 1) / TT, nt = (N + TT - 1) / TT;
    const dim3 grid((unsigned)((long long)mt * nt * batch));
    if constexpr (ops<T>::is_complex)
        hipLaunchKernelGGL((gemm_valu_kernel<T>), grid, dim3(256), 0, s, Am, lda_, sA, Bm, ldb_, sB, Cm, ldc, sC, M,
                           N, K, mt, nt, kdir, info, Dm, ldd, sD, aop);
    else
        hipLaunchKernelGGL((gemm_mfma_kernel<T>), grid, dim3(256), 0, s, Am, lda_, sA, Bm, ldb_, sB, Cm, ldc, sC, M,
                           N, K, mt, nt, kdir, info, aop);
    return hipGetLastError();
}

// U12 = L11^-1 (P A12) for the `rest` columns right of panel j0, displaced
// rows moved
template <typename T>
hipError_t launch_right_solve(const Problem& p, int j0, int rest, hipStream_t s) {
    T* A = (T*)p.A;
    if constexpr (sizeof(T) <= 8) {
        constexpr int TC = StageTile<T>::TC;
        const int ct = (rest + TC - 1) / TC;
        hipLaunchKernelGGL((trsm_stage_kernel<T>), dim3((unsigned)((long long)ct * p.batch)), dim3(64), 0, s, p, j0,
                           rest, ct);
        return hipGetLastError();
    } else {   // complex double: the stage would not fit the registers
        return launch_trsm<T>(A, p.lda, p.sA, A + (long long)(j0 + NBP) * p.lda, p.lda, p.sA, j0, NBP, rest, p.batch,
                              p.ipiv, p.sP, true, false, nullptr, s, true);
    }
}

// A22 -= L21 U12 on the columns [c0, c0 + N) of the rest x rest trailing matrix
template <typename T>
hipError_t launch_update(const Problem& p, int j0, int rest, int c0, int N, hipStream_t s) {
    T* A = (T*)p.A;
    if constexpr (!ops<T>::is_complex) {
        const int ms = (rest + 63) / 64;
        hipLaunchKernelGGL((update_strip_kernel<T>), dim3((unsigned)((long long)ms * p.batch)), dim3(256), 0, s, A,
                           p.lda, p.sA, j0, rest, c0, N, ms);
    } else {
        using R = typename ops<T>::R;
        constexpr int SH = CplxStrip<R>::SH;
        const int ms = (rest + SH - 1) / SH;
        hipLaunchKernelGGL((update_strip_cplx_kernel<R>), dim3((unsigned)((long long)ms * p.batch)), dim3(256), 0, s,
                           A, p.lda, p.sA, j0, rest, c0, N, ms);
    }
    return hipGetLastError();
}

// Panel by panel.  With a look-ahead stream, update k covers the next
// panel's 32 columns first; panel k+1 then runs on the side stream while the
// rest of update k runs on the caller's stream, and the caller's stream waits
// for the panel before the next right-hand solve.  The panel writes only its
// own columns (and ipiv, info) and the remaining update only the columns
// beyond them, so the two touch disjoint data; every element still takes its
// updates in the same order.  The fork and join cost several microseconds per
// panel, which pays only for long panels while the first trailing update
// leaves compute units idle: real types, n >= 1024, at most one 64-row strip
// per compute unit (256) over the batch, two from n = 1536 (measured: n =
// 2048, batch 8 gains 7 %, batch 16 8 % (double 4 %); n = 1536, batch 16
// 3 %; n = 1024 at batch 32 loses 6 %, n = 1024 and 512 at batch 64 lose 3 %
// and 16 %; complex n = 96 - 256 at batch <= 64 lose 5 - 15 %).
template <typename T>
hipError_t getrf_t(const Problem& p, hipStream_t s) {
    const int n = p.n;
    hipError_t e;
    LookAhead la;
    const long long strips = (long long)((n - NBP + 63) / 64) * p.batch;
    const bool ahead = !ops<T>::is_complex && n >= 1024 && strips <= (n >= 1536 ? 512 : 256) && lookahead_begin(la);
    if ((e = launch_panel<T>(p, 0, min(NBP, n), s)) != hipSuccess) return lookahead_end(la, e);
    for (int j0 = 0; j0 + NBP < n; j0 += NBP) {
        const int rest = n - j0 - NBP;
        const int nw = min(NBP, rest);          // width of the next panel
        if ((e = launch_right_solve<T>(p, j0, rest, s)) != hipSuccess) return lookahead_end(la, e);
        if (!ahead || rest == nw) {
            if ((e = launch_update<T>(p, j0, rest, 0, rest, s)) != hipSuccess) return lookahead_end(la, e);
            if ((e = launch_panel<T>(p, j0 + NBP, nw, s)) != hipSuccess) return lookahead_end(la, e);
            continue;
        }
        if ((e = launch_update<T>(p, j0, rest, 0, nw, s)) != hipSuccess) return lookahead_end(la, e);
        if ((e = lookahead_fork(la, s)) != hipSuccess) return lookahead_end(la, e);
        if ((e = launch_panel<T>(p, j0 + NBP, nw, la.side)) != hipSuccess) return lookahead_end(la, e);
        if ((e = lookahead_join_record(la)) != hipSuccess) return lookahead_end(la, e);
        if ((e = launch_update<T>(p, j0, rest, nw, rest - nw, s)) != hipSuccess) return lookahead_end(la, e);
        if ((e = lookahead_join_wait(la, s)) != hipSuccess) return lookahead_end(la, e);
    }
    if (n > NBP) {
        // panels 0 .. npan-1 have later steps; rows lo .. n-1 of panel k,
        // at most n - NBP of them
        const int npan = (n - 1) / NBP;
        const int nt = panel_threads(n - NBP);
        const int rpt = (n - NBP + nt - 1) / nt;
        const size_t smem = (size_t)(n - NBP) * sizeof(int);
        const dim3 grid((unsigned)((long long)npan * p.batch));
        if (rpt <= 1) hipLaunchKernelGGL((left_swap_kernel<T, 1>), grid, dim3(nt), smem, s, p, npan);
        else if (rpt <= 2) hipLaunchKernelGGL((left_swap_kernel<T, 2>), grid, dim3(nt), smem, s, p, npan);
        else if (rpt <= 4) hipLaunchKernelGGL((left_swap_kernel<T, 4>), grid, dim3(nt), smem, s, p, npan);
        else return lookahead_end(la, hipErrorInvalidValue);
        if ((e = hipGetLastError()) != hipSuccess) return lookahead_end(la, e);
    }
    return lookahead_end(la, hipSuccess);
}

template <typename T>
hipError_t launch_permute(const Problem& p, bool reverse, hipStream_t s) {
    const int nt = panel_threads(p.n);
    const size_t smem = (size_t)2 * p.n * sizeof(int) + 16 + (size_t)p.n * sizeof(T);
    hipLaunchKernelGGL((permute_rows_kernel<T>), dim3(p.batch), dim3(nt), smem, s, p, reverse);
    return hipGetLastError();
}

// Solve with the factors block row by block row: a 32-row triangular-block
// solve, then a GEMM update of the rows still to come, which takes each k of
// the block in substitution order, so every element of X sees the
// substitutions' operation sequence.
//   A X = B:   B <- P B; L Y = B, blocks ascending; U X = Y, blocks descending.
//   A^T X = B, A^H X = B (op = T or H, conjugated factors for H):
//              op(U) W = B, blocks ascending, dividing by the diagonal;
//              op(L) Z = W, blocks descending, unit diagonal; X = P^T Z.
// The block of op(L) or op(U) at rows [i0, ..) and columns [k0, ..) is read
// transposed from the stored factor at rows [k0, ..), columns [i0, ..).
template <typename T>
hipError_t getrs_t(const Problem& p, hipStream_t s) {
    const int n = p.n, nrhs = p.nrhs, aop = p.trans;
    const long long lda = p.lda;
    hipError_t e;
    if (aop == 0 && (e = launch_permute<T>(p, false, s)) != hipSuccess) return e;
    const T* A = (const T*)p.A;
    T* B = (T*)p.B;
    // forward: L Y = P B or op(U) W = B, block rows ascending
    for (int r0 = 0; r0 < n; r0 += NBP) {
        const int w = min(NBP, n - r0);
        if ((e = launch_trsm<T>(A, p.lda, p.sA, B, p.ldb, p.sB, r0, w, nrhs, p.batch, nullptr, 0, false, false,
                                p.info, s, aop == 0, aop)) != hipSuccess)
            return e;
        const int rest = n - r0 - w;
        if (rest <= 0) continue;
        const T* blk = aop ? A + r0 + (r0 + w) * lda : A + r0 + w + r0 * lda;
        if ((e = launch_gemm<T>(blk, p.lda, p.sA, B + r0, p.ldb, p.sB, B + r0 + w, p.ldb, p.sB, rest, nrhs, w,
                                p.batch, 1, p.info, s, nullptr, 0, 0, aop)) != hipSuccess)
            return e;
    }
    // back: U X = Y or op(L) Z = W, block rows descending
    const int last = ((n - 1) / NBP) * NBP;
    for (int r0 = last; r0 >= 0; r0 -= NBP) {
        const int w = min(NBP, n - r0);
        if ((e = launch_trsm<T>(A, p.lda, p.sA, B, p.ldb, p.sB, r0, w, nrhs, p.batch, nullptr, 0, false, true,
                                p.info, s, aop != 0, aop)) != hipSuccess)
            return e;
        if (r0 == 0) continue;
        const T* blk = aop ? A + r0 : A + r0 * lda;
        if ((e = launch_gemm<T>(blk, p.lda, p.sA, B + r0, p.ldb, p.sB, B, p.ldb, p.sB, r0, nrhs, w, p.batch, -1,
                                p.info, s, nullptr, 0, 0, aop)) != hipSuccess)
            return e;
    }
    if (aop != 0 && (e = launch_permute<T>(p, true, s)) != hipSuccess) return e;
    return hipSuccess;
}

// C = I, one work-group per (column, matrix)
template <typename T>
__global__ void __launch_bounds__(256) identity_kernel(T* C, int ldc, long long sC, int n)
{
    using O = ops<T>;
    const int j = (int)(blockIdx.x % (unsigned)n);
    const long long mat = blockIdx.x / (unsigned)n;
    T* col = C + mat * sC + (long long)j * ldc;
    for (int i = threadIdx.x; i < n; i += 256) col[i] = i == j ? O::one() : O::zero();
}

// getri above the one-launch solve's order: C = I, then the blocked NoTrans
// solve on it
template <typename T>
hipError_t getri_t(const Problem& p, hipStream_t s) {
    hipLaunchKernelGGL((identity_kernel<T>), dim3((unsigned)((long long)p.n * p.batch)), dim3(256), 0, s, (T*)p.B,
                       p.ldb, p.sB, p.n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    Problem q = p;
    q.nrhs = p.n;
    q.trans = 0;
    q.info = nullptr;
    return getrs_t<T>(q, s);
}

}  // namespace

}  // namespace batchlu
