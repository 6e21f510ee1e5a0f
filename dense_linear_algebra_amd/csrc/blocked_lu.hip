// blocked_lu.hip -- blocked right-looking LU (panel width 32) and the blocked
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
                if (__builtin_amdgcn_ballot_w64(small) != 0) {
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

// Solve with the 32 x 32 diagonal block of T for columns [c0, c0 + 64) of X.
//   lower unit (UPPER = false): x_f -= l_fm x_m, m ascending;
//   upper (UPPER = true): x_m /= u_mm then x_f -= u_fm x_m, m descending.
// With `swap` the rows of X are first permuted by the w transpositions in
// ipiv[j0 .. j0 + w) (getrf right-hand interchange): rows j0.. j0+w-1 get the
// solved values, displaced rows below are copied to their new places.
template <typename T, bool UPPER>
__global__ void __launch_bounds__(64) trsm_block_kernel(const void* Tmat, int ldt, long long sT, void* Xmat,
                                                        int ldx, long long sX, int r0, int w, int ncols,
                                                        int ctiles, const int* ipiv, long long sP, bool swap,
                                                        const int* info)
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

    for (int e = tid; e < w * w; e += 64) {
        const int i = e % w, k = e / w;
        tri[i][k] = Tp[i + (long long)k * ldt];
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
#pragma unroll
        for (int mm = 0; mm < NBP; ++mm) {
            if (mm >= w) continue;
#pragma unroll
            for (int f = 0; f < NBP; ++f)
                if (f > mm && f < w) O::fms(x[f], tri[f][mm], x[mm]);
        }
    } else {
#pragma unroll
        for (int mm = NBP - 1; mm >= 0; --mm) {
            if (mm >= w) continue;
            x[mm] = O::div(x[mm], tri[mm][mm]);
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
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ inline void tile_load(T (*As)[TT], T (*Bs)[TT], const T* Ap, int lda_, const T* Bp, int ldb_,
                                 int M, int N, int K, int tid, int nthr, bool negate)
{
    using O = ops<T>;
    for (int e = tid; e < TT * K; e += nthr) {
        const int i = e % TT, k = e / TT;
        T v = i < M ? Ap[i + (long long)k * lda_] : O::zero();
        if (negate) {
            if constexpr (O::is_complex) { v.re = -v.re; v.im = -v.im; }
            else v = -v;
        }
        As[k][i] = v;
    }
    for (int e = tid; e < TT * K; e += nthr) {
        const int k = e % K, j = e / K;
        Bs[k][j] = j < N ? Bp[k + (long long)j * ldb_] : O::zero();
    }
}

// MFMA version for float and double: 4 waves, each a 32 x 32 quarter of the
// 64 x 64 tile made of 2 x 2 blocks of 16 x 16.
template <typename T>
__global__ void __launch_bounds__(256) gemm_mfma_kernel(const void* Am, int lda_, long long sA, const void* Bm,
                                                        int ldb_, long long sB, void* Cm, int ldc, long long sC,
                                                        int M, int N, int K, int mtiles, int ntiles, int kdir,
                                                        const int* info)
{
    __shared__ T As[NBP][TT];
    __shared__ T Bs[NBP][TT];
    const int tiles = mtiles * ntiles;
    const long long mat = blockIdx.x / tiles;
    const int t = (int)(blockIdx.x % tiles);
    const int i0 = (t % mtiles) * TT, jt0 = (t / mtiles) * TT;
    if (info && info[mat] != 0) return;
    const T* Ap = (const T*)Am + mat * sA + i0;
    const T* Bp = (const T*)Bm + mat * sB + (long long)jt0 * ldb_;
    T* Cp = (T*)Cm + mat * sC + i0 + (long long)jt0 * ldc;
    const int Mt = min(TT, M - i0), Nt = min(TT, N - jt0);
    tile_load<T>(As, Bs, Ap, lda_, Bp, ldb_, Mt, Nt, K, threadIdx.x, 256, true);
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

// VALU version (complex types): each thread owns a 4 x 4 block of the tile.
template <typename T>
__global__ void __launch_bounds__(256) gemm_valu_kernel(const void* Am, int lda_, long long sA, const void* Bm,
                                                        int ldb_, long long sB, void* Cm, int ldc, long long sC,
                                                        int M, int N, int K, int mtiles, int ntiles, int kdir,
                                                        const int* info)
{
    using O = ops<T>;
    __shared__ T As[NBP][TT];
    __shared__ T Bs[NBP][TT];
    const int tiles = mtiles * ntiles;
    const long long mat = blockIdx.x / tiles;
    const int t = (int)(blockIdx.x % tiles);
    const int i0 = (t % mtiles) * TT, jt0 = (t / mtiles) * TT;
    if (info && info[mat] != 0) return;
    const T* Ap = (const T*)Am + mat * sA + i0;
    const T* Bp = (const T*)Bm + mat * sB + (long long)jt0 * ldb_;
    T* Cp = (T*)Cm + mat * sC + i0 + (long long)jt0 * ldc;
    const int Mt = min(TT, M - i0), Nt = min(TT, N - jt0);
    tile_load<T>(As, Bs, Ap, lda_, Bp, ldb_, Mt, Nt, K, threadIdx.x, 256, false);
    __syncthreads();
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
// panel k are gathered through the interchanges of all later steps.
// ---------------------------------------------------------------------------
template <typename T, int RPT>
__global__ void __launch_bounds__(1024) left_swap_kernel(Problem p)
{
    extern __shared__ int sipiv[];   // n entries, 0-based
    const int n = p.n;
    const int tid = threadIdx.x, nt = blockDim.x;
    const long long mat = blockIdx.x;
    T* A = (T*)p.A + mat * p.sA;
    for (int i = tid; i < n; i += nt) sipiv[i] = p.ipiv[mat * p.sP + i] - 1;
    __syncthreads();
    const int P = (n + NBP - 1) / NBP;
    int map[RPT];
#pragma unroll
    for (int q = 0; q < RPT; ++q) map[q] = tid + q * nt;
    for (int k = P - 2; k >= 0; --k) {
        const int lo = (k + 1) * NBP;                   // first row the later steps touch
        const int hi = min(n, lo + NBP);                // steps of panel k + 1
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            int x = map[q];
            if (tid + q * nt >= lo && tid + q * nt < n)
                for (int s = hi - 1; s >= lo; --s) {
                    const int ps = sipiv[s];
                    x = (x == s) ? ps : (x == ps ? s : x);
                }
            map[q] = x;
        }
        const int c0 = k * NBP, w = min(NBP, n - c0);
        constexpr int CC = 8;   // columns per read/write round
        for (int cb = 0; cb < w; cb += CC) {
            T v[RPT][CC];
#pragma unroll
            for (int q = 0; q < RPT; ++q) {
                const int i = tid + q * nt;
#pragma unroll
                for (int c = 0; c < CC; ++c)
                    if (i >= lo && i < n && cb + c < w && map[q] != i)
                        v[q][c] = A[map[q] + (long long)(c0 + cb + c) * p.lda];
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < RPT; ++q) {
                const int i = tid + q * nt;
#pragma unroll
                for (int c = 0; c < CC; ++c)
                    if (i >= lo && i < n && cb + c < w && map[q] != i)
                        A[i + (long long)(c0 + cb + c) * p.lda] = v[q][c];
            }
            __syncthreads();
        }
    }
}

// B <- P B: position i receives the row the full interchange sequence brings
// there (a backward trace of ipiv per row), column by column through LDS.
template <typename T>
__global__ void __launch_bounds__(1024) permute_rows_kernel(Problem p)
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
        for (int s = n - 1; s >= 0; --s) {
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
    int nt = ((m + 63) / 64) * 64;
    if (nt > CAP) nt = CAP;
    const int rpt = (m + nt - 1) / nt;
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
                       const int* info, hipStream_t s) {
    const int ct = (ncols + 63) / 64;
    const dim3 grid((unsigned)((long long)ct * batch));
    if (upper)
        hipLaunchKernelGGL((trsm_block_kernel<T, true>), grid, dim3(64), 0, s, Tm, ldt, sT, X, ldx, sX, r0, w,
                           ncols, ct, ipiv, sP, swap, info);
    else
        hipLaunchKernelGGL((trsm_block_kernel<T, false>), grid, dim3(64), 0, s, Tm, ldt, sT, X, ldx, sX, r0, w,
                           ncols, ct, ipiv, sP, swap, info);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_gemm(const void* Am, int lda_, long long sA, const void* Bm, int ldb_, long long sB, void* Cm,
                       int ldc, long long sC, int M, int N, int K, int batch, int kdir, const int* info,
                       hipStream_t s) {
    if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
    const int mt = (M + TT - 1) / TT, nt = (N + TT - 1) / TT;
    const dim3 grid((unsigned)((long long)mt * nt * batch));
    if constexpr (ops<T>::is_complex)
        hipLaunchKernelGGL((gemm_valu_kernel<T>), grid, dim3(256), 0, s, Am, lda_, sA, Bm, ldb_, sB, Cm, ldc, sC, M,
                           N, K, mt, nt, kdir, info);
    else
        hipLaunchKernelGGL((gemm_mfma_kernel<T>), grid, dim3(256), 0, s, Am, lda_, sA, Bm, ldb_, sB, Cm, ldc, sC, M,
                           N, K, mt, nt, kdir, info);
    return hipGetLastError();
}

template <typename T>
hipError_t getrf_t(const Problem& p, hipStream_t s) {
    const int n = p.n;
    hipError_t e;
    for (int j0 = 0; j0 < n; j0 += NBP) {
        const int w = min(NBP, n - j0);
        if ((e = launch_panel<T>(p, j0, w, s)) != hipSuccess) return e;
        const int rest = n - j0 - w;
        if (rest <= 0) break;
        T* A = (T*)p.A;
        // U12 = L11^-1 * (P A12), displaced rows moved
        if ((e = launch_trsm<T>(A, p.lda, p.sA, A + (long long)(j0 + w) * p.lda, p.lda, p.sA, j0, w, rest,
                                p.batch, p.ipiv, p.sP, true, false, nullptr, s)) != hipSuccess)
            return e;
        // A22 -= L21 * U12
        if ((e = launch_gemm<T>(A + j0 + w + (long long)j0 * p.lda, p.lda, p.sA,
                                A + j0 + (long long)(j0 + w) * p.lda, p.lda, p.sA,
                                A + j0 + w + (long long)(j0 + w) * p.lda, p.lda, p.sA, rest, rest, w, p.batch, 1,
                                nullptr, s)) != hipSuccess)
            return e;
    }
    if (n > NBP) {
        const int nt = panel_threads(n);
        const int rpt = (n + nt - 1) / nt;
        const size_t smem = (size_t)n * sizeof(int);
        if (rpt <= 1) hipLaunchKernelGGL((left_swap_kernel<T, 1>), dim3(p.batch), dim3(nt), smem, s, p);
        else if (rpt <= 2) hipLaunchKernelGGL((left_swap_kernel<T, 2>), dim3(p.batch), dim3(nt), smem, s, p);
        else if (rpt <= 4) hipLaunchKernelGGL((left_swap_kernel<T, 4>), dim3(p.batch), dim3(nt), smem, s, p);
        else return hipErrorInvalidValue;
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T>
hipError_t getrs_t(const Problem& p, hipStream_t s) {
    const int n = p.n, nrhs = p.nrhs;
    hipError_t e;
    {
        const int nt = panel_threads(n);
        const size_t smem = (size_t)2 * n * sizeof(int) + 16 + (size_t)n * sizeof(T);
        hipLaunchKernelGGL((permute_rows_kernel<T>), dim3(p.batch), dim3(nt), smem, s, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const T* A = (const T*)p.A;
    T* B = (T*)p.B;
    // forward: L Y = P B, block rows ascending
    for (int r0 = 0; r0 < n; r0 += NBP) {
        const int w = min(NBP, n - r0);
        if ((e = launch_trsm<T>(A, p.lda, p.sA, B, p.ldb, p.sB, r0, w, nrhs, p.batch, nullptr, 0, false, false,
                                p.info, s)) != hipSuccess)
            return e;
        const int rest = n - r0 - w;
        if (rest > 0 &&
            (e = launch_gemm<T>(A + r0 + w + (long long)r0 * p.lda, p.lda, p.sA, B + r0, p.ldb, p.sB, B + r0 + w,
                                p.ldb, p.sB, rest, nrhs, w, p.batch, 1, p.info, s)) != hipSuccess)
            return e;
    }
    // back: U X = Y, block rows descending
    const int last = ((n - 1) / NBP) * NBP;
    for (int r0 = last; r0 >= 0; r0 -= NBP) {
        const int w = min(NBP, n - r0);
        if ((e = launch_trsm<T>(A, p.lda, p.sA, B, p.ldb, p.sB, r0, w, nrhs, p.batch, nullptr, 0, false, true,
                                p.info, s)) != hipSuccess)
            return e;
        if (r0 > 0 &&
            (e = launch_gemm<T>(A + (long long)r0 * p.lda, p.lda, p.sA, B + r0, p.ldb, p.sB, B, p.ldb, p.sB, r0,
                                nrhs, w, p.batch, -1, p.info, s)) != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace

bool blocked_supported(int dtype, int n) {
    // four panel rows per thread at the per-type work-group cap
    const int cap = dtype == R32 ? 4096 : (dtype == C128 ? 1024 : 2048);
    return n >= 1 && n <= cap;
}

hipError_t blocked_getrf(int dtype, const Problem& p, hipStream_t s) {
    if (!blocked_supported(dtype, p.n)) return hipErrorInvalidValue;
    // real orders up to 256: the whole blocked sequence in one work-group
    if (blocked_fused_supported(dtype, p.n, p.lda)) return blocked_fused_getrf(dtype, p, s);
    switch (dtype) {
    case R32: return getrf_t<float>(p, s);
    case R64: return getrf_t<double>(p, s);
    case C64: return getrf_t<cplx<float>>(p, s);
    case C128: return getrf_t<cplx<double>>(p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t blocked_getrs(int dtype, const Problem& p, hipStream_t s) {
    if (!blocked_supported(dtype, p.n)) return hipErrorInvalidValue;
    switch (dtype) {
    case R32: return getrs_t<float>(p, s);
    case R64: return getrs_t<double>(p, s);
    case C64: return getrs_t<cplx<float>>(p, s);
    case C128: return getrs_t<cplx<double>>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace batchlu
