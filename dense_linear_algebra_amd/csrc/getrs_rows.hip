// getrs_rows.hip -- the whole LU solve of one matrix and one tile of
// right-hand sides in a single work-group: one row per thread, n <= 1024,
// for A X = B (also A C = I, the inverse of getri) and (second kernel,
// below) A^T X = B and A^H X = B.
//
// BatchLAS "LU" page, fused getrs paragraph (one work-group per matrix does
// the permutation and both substitutions in one launch) and blocked getrs
// (block solves then updates); here the two are combined for gfx950:
//   - the interchange list is applied as one gather (a backward trace of
//     ipiv per row), so no row is written before every row has been read;
//   - forward: per block of 32 rows, the wavefront holding those rows solves
//     the 32 x 32 unit-lower block on its own (x_m broadcast by readlane, no
//     barrier), publishes the block's solution in LDS, and after one barrier
//     every lower row subtracts l_ik * y_k for the block's 32 k;
//   - back: the same with U, blocks descending, true division by u_kk.
// Per element the order of operations is the plain one (ascending k forward,
// descending k backward), so X equals the unblocked substitution bit for bit.
#include "device_ops.h"
#include "internal.h"

namespace batchlu {

namespace {

constexpr int BS = 32;   // rows per diagonal block
constexpr int CK = 16;   // columns of L or U loaded per round
// entries of the next block prefetched per thread: the first half of its
// block row, for double with right-hand-side tiles of at most four columns
// (measured: 8 % faster at n = 256, nrhs = 1, batch 1024; 10 % at n = 512
// and 1024).  None elsewhere: float and complex float measured slower with
// it (n = 1024, nrhs = 32, batch 64 float: 0.65 -> 0.94 ms; complex float
// n = 256 and 512: 11 - 16 %), where the solve is bound by reading the
// factors once per tile and the prefetch adds reads; wider tiles and complex
// double would spill (the prefetch and the block in use are live together,
// within 128 VGPRs per thread for 1024 threads).
template <typename T, int NRT>
constexpr int pf_count() { return (sizeof(T) == 8 && !ops<T>::is_complex && NRT <= 4) ? CK : 0; }

// Work-group -> (matrix, RHS tile).  Work-groups are dealt to the eight
// XCDs in turn; when the batch is a multiple of eight, the tiles of one
// matrix go to one XCD, so they read its factors through one L2.
__device__ inline void tile_of(int batch, int rtiles, long long& m, int& tile) {
    const unsigned b = blockIdx.x;
    if (rtiles > 1 && (batch & 7) == 0) {
        const unsigned slot = b >> 3;
        m = (long long)(slot / (unsigned)rtiles) * 8 + (b & 7);
        tile = (int)(slot % (unsigned)rtiles);
    } else {
        m = b / (unsigned)rtiles;
        tile = (int)(b % (unsigned)rtiles);
    }
}

// x_c = y_c / u_cc for the NRT right-hand sides held by diagonal lane dl,
// broadcast to the whole wavefront in xc; lane dl keeps them in y.  Lane r
// divides right-hand side r (the same operands as the diagonal lane's, so
// the same quotient bits), so the wavefront pays for one division rather
// than NRT in a row: the divisions were half of the solve's time (complex
// float n = 64, 16 right-hand sides, batch 8192: 0.70 ms, 0.35 without
// them).  Every lane of the wavefront is active here.
template <typename T, int NRT>
__device__ inline void diag_divide(T (&y)[NRT], T (&xc)[NRT], const T& diag, int dl, int lane) {
    using O = ops<T>;
    static_assert(NRT > 1, "one right-hand side divides in the diagonal lane");
    {
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
}

// IDENT: getri.  B is not read; the right-hand sides are the identity's
// columns, so row `row` of P*I is e_src (one where the column is src).
template <typename T, int NRT, bool IDENT>
__global__ void __launch_bounds__(1024) getrs_rows_kernel(Problem p, int rtiles)
{
    using O = ops<T>;
    extern __shared__ uint4 smem_raw[];
    int* sipiv = (int*)smem_raw;                                             // n entries
    T* ybuf = (T*)((char*)smem_raw + ((p.n * 4 + 15) / 16) * 16);            // [2][BS][NRT]

    const int n = p.n;
    long long m;
    int c0;
    tile_of(p.batch, rtiles, m, c0);
    c0 *= NRT;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    if (p.info && p.info[m] != 0) return;   // composed gesv: failed factorisation keeps B

    const T* LU = (const T*)p.A + m * p.sA;
    const int* ipiv = p.ipiv + m * p.sP;
    T* B = (T*)p.B + m * p.sB;

    for (int i = tid; i < n; i += blockDim.x) {   // entries outside 1..n: no interchange
        const int v = ipiv[i] - 1;
        sipiv[i] = (v >= 0 && v < n) ? v : i;
    }
    __syncthreads();

    // a8: row tid of P*B is original row src
    const int row = tid;
    const bool have = row < n;
    T y[NRT];
    {
        int src = row;
        if (have)
            for (int k = n - 1; k >= 0; --k) {
                const int pk = sipiv[k];
                src = (src == k) ? pk : (src == pk ? k : src);
            }
#pragma unroll
        for (int r = 0; r < NRT; ++r) {
            if constexpr (IDENT)
                y[r] = (have && c0 + r < p.nrhs && src == c0 + r) ? O::one() : O::zero();
            else
                y[r] = (have && c0 + r < p.nrhs) ? B[src + (long long)(c0 + r) * p.ldb] : O::zero();
        }
    }

    const int P = (n + BS - 1) / BS;
    // Each thread holds the PF entries of its row in the current block's
    // columns, loaded during the previous block (the next block's are
    // requested right after each barrier and arrive while the update runs),
    // so the wavefront that solves the next diagonal block does not wait for
    // memory on its way there.  Entries a thread does not use are loaded
    // anyway where they lie inside the matrix, and never read.
    constexpr int PF = pf_count<T, NRT>();
    T pf[PF > 0 ? PF : 1];
    // a9: forward, L unit lower
#pragma unroll
    for (int e = 0; e < PF; ++e) pf[e] = (have && e < n) ? LU[row + (long long)e * p.lda] : O::zero();
    for (int kb = 0; kb < P; ++kb) {
        const int r0 = kb * BS;
        const int w = min(BS, n - r0);
        T* yb = ybuf + (size_t)(kb & 1) * BS * NRT;
        if (wave == r0 / 64) {
            // the 32 rows of the block are lanes r0%64 .. r0%64+w-1 of this wavefront
            const int base = r0 % 64;
            const int mrow = lane - base;      // row inside the block when in [0, w)
#pragma unroll
            for (int cc = 0; cc < BS; cc += CK) {
                T lrow[CK];
#pragma unroll
                for (int e = 0; e < CK; ++e) {
                    const int c = cc + e;
                    if (c < PF) lrow[e] = pf[c];
                    else lrow[e] = (mrow > c && mrow < w) ? LU[row + (long long)(r0 + c) * p.lda] : O::zero();
                }
#pragma unroll
                for (int e = 0; e < CK; ++e) {
                    const int c = cc + e;
                    if (c >= w) continue;
                    T xc[NRT];
#pragma unroll
                    for (int r = 0; r < NRT; ++r) xc[r] = readlane_t(y[r], base + c);
                    if (mrow > c && mrow < w)
#pragma unroll
                        for (int r = 0; r < NRT; ++r) O::fms(y[r], lrow[e], xc[r]);
                }
            }
            if (mrow >= 0 && mrow < w)
#pragma unroll
                for (int r = 0; r < NRT; ++r) yb[mrow * NRT + r] = y[r];
        }
        __syncthreads();
        // the next block's entries: rows at or below that block use them
        const int r1 = r0 + BS;
        const bool nneed = have && row >= r1;
        T nx[PF > 0 ? PF : 1];
#pragma unroll
        for (int e = 0; e < PF; ++e) nx[e] = (nneed && r1 + e < n) ? LU[row + (long long)(r1 + e) * p.lda] : O::zero();
        if (have && row >= r0 + w) {
#pragma unroll
            for (int cc = 0; cc < BS; cc += CK) {
                T lrow[CK];
#pragma unroll
                for (int e = 0; e < CK; ++e) {
                    const int c = cc + e;
                    if (c < PF) lrow[e] = pf[c];
                    else lrow[e] = c < w ? LU[row + (long long)(r0 + c) * p.lda] : O::zero();
                }
#pragma unroll
                for (int e = 0; e < CK; ++e) {
                    if (cc + e >= w) continue;
#pragma unroll
                    for (int r = 0; r < NRT; ++r) O::fms(y[r], lrow[e], yb[(cc + e) * NRT + r]);
                }
            }
        }
#pragma unroll
        for (int e = 0; e < PF; ++e) pf[e] = nx[e];
    }
    __syncthreads();
    // a10: back, U upper; blocks descending.  The prefetch covers the rows
    // at or above each block (the block's own rows and those it updates).
    {
        const int rl = (P - 1) * BS;
        const bool need = have && row < n;
#pragma unroll
        for (int e = 0; e < PF; ++e) pf[e] = (need && rl + e < n) ? LU[row + (long long)(rl + e) * p.lda] : O::zero();
    }
    for (int kb = P - 1; kb >= 0; --kb) {
        const int r0 = kb * BS;
        const int w = min(BS, n - r0);
        T* yb = ybuf + (size_t)(kb & 1) * BS * NRT;
        if (wave == r0 / 64) {
            const int base = r0 % 64;
            const int mrow = lane - base;
#pragma unroll
            for (int cc = BS - CK; cc >= 0; cc -= CK) {
                T urow[CK];
#pragma unroll
                for (int e = 0; e < CK; ++e) {
                    const int c = cc + e;
                    if (c < PF) urow[e] = pf[c];
                    else urow[e] = (mrow >= 0 && mrow <= c && c < w) ? LU[row + (long long)(r0 + c) * p.lda] : O::zero();
                }
#pragma unroll
                for (int e = CK - 1; e >= 0; --e) {
                    const int c = cc + e;
                    if (c >= w) continue;
                    T xc[NRT];
                    if constexpr (NRT == 1) {
                        if (mrow == c) y[0] = O::div(y[0], urow[e]);
                        xc[0] = readlane_t(y[0], base + c);
                    } else {
                        diag_divide(y, xc, urow[e], base + c, lane);
                    }
                    if (mrow >= 0 && mrow < c)
#pragma unroll
                        for (int r = 0; r < NRT; ++r) O::fms(y[r], urow[e], xc[r]);
                }
            }
            if (mrow >= 0 && mrow < w)
#pragma unroll
                for (int r = 0; r < NRT; ++r) yb[mrow * NRT + r] = y[r];
        }
        __syncthreads();
        const int rp = r0 - BS;   // the next block (descending)
        const bool nneed = have && kb > 0 && row < r0;
        T nx[PF > 0 ? PF : 1];
#pragma unroll
        for (int e = 0; e < PF; ++e) nx[e] = nneed ? LU[row + (long long)(rp + e) * p.lda] : O::zero();
        if (have && row < r0) {
#pragma unroll
            for (int cc = BS - CK; cc >= 0; cc -= CK) {
                T urow[CK];
#pragma unroll
                for (int e = 0; e < CK; ++e) {
                    const int c = cc + e;
                    if (c < PF) urow[e] = pf[c];
                    else urow[e] = c < w ? LU[row + (long long)(r0 + c) * p.lda] : O::zero();
                }
#pragma unroll
                for (int e = CK - 1; e >= 0; --e) {
                    if (cc + e >= w) continue;
#pragma unroll
                    for (int r = 0; r < NRT; ++r) O::fms(y[r], urow[e], yb[(cc + e) * NRT + r]);
                }
            }
        }
#pragma unroll
        for (int e = 0; e < PF; ++e) pf[e] = nx[e];
    }
    if (have)
#pragma unroll
        for (int r = 0; r < NRT; ++r)
            if (c0 + r < p.nrhs) B[row + (long long)(c0 + r) * p.ldb] = y[r];
}

// op(A) = A^T (CONJ false) or A^H (CONJ true).  With A = P^T L U,
// A^T = U^T L^T P: forward against U^T (lower, true division by u_kk),
// back against L^T (unit upper), then x = P^T z.  Row `row` of U^T and L^T
// is column `row` of the stored factors, so each thread walks its own
// column.  The interchanges are undone by a scatter: z_row goes to row
// src(row), the same backward trace that the NoTrans gather uses (P b has
// b_src at row `row`, so P^T z has z_row at row src).  B is read at the
// start and written at the end, with barriers between, so the scatter needs
// no second buffer.
template <bool CONJ, typename T>
__device__ inline T op_entry(const T& v) {
    if constexpr (CONJ && ops<T>::is_complex) return T{v.re, -v.im};
    else return v;
}

// CK consecutive entries of one stored column, op_entry applied, read as
// 16-byte vectors (src 16-byte aligned): a quarter of the load instructions
// of element loads for float, which matters because the lanes of a
// wavefront each read a different column.
template <bool CONJ, typename T>
__device__ inline void load_column_run(T (&dst)[CK], const T* src) {
    constexpr int PER = 16 / (int)sizeof(T);
    static_assert(CK % PER == 0, "run length");
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
    for (int q = 0; q < CK / PER; ++q) {
        const uint4 v = s4[q];
        T tmp[PER];
        __builtin_memcpy(tmp, &v, 16);
#pragma unroll
        for (int i = 0; i < PER; ++i) dst[q * PER + i] = op_entry<CONJ>(tmp[i]);
    }
}

template <typename T, int NRT, bool CONJ>
__global__ void __launch_bounds__(1024) getrs_rows_trans_kernel(Problem p, int rtiles)
{
    using O = ops<T>;
    extern __shared__ uint4 smem_raw[];
    int* sipiv = (int*)smem_raw;                                             // n entries
    T* ybuf = (T*)((char*)smem_raw + ((p.n * 4 + 15) / 16) * 16);            // [2][BS][NRT]

    const int n = p.n;
    long long m;
    int c0;
    tile_of(p.batch, rtiles, m, c0);
    c0 *= NRT;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    const T* LU = (const T*)p.A + m * p.sA;
    const int* ipiv = p.ipiv + m * p.sP;
    T* B = (T*)p.B + m * p.sB;

    for (int i = tid; i < n; i += blockDim.x) {
        const int v = ipiv[i] - 1;
        sipiv[i] = (v >= 0 && v < n) ? v : i;
    }
    __syncthreads();

    const int row = tid;
    const bool have = row < n;
    int dst = row;   // row of X that receives z_row
    if (have)
        for (int k = n - 1; k >= 0; --k) {
            const int pk = sipiv[k];
            dst = (dst == k) ? pk : (dst == pk ? k : dst);
        }
    T y[NRT];
#pragma unroll
    for (int r = 0; r < NRT; ++r)
        y[r] = (have && c0 + r < p.nrhs) ? B[row + (long long)(c0 + r) * p.ldb] : O::zero();
    const T* col = LU + (long long)row * p.lda;   // column `row`: row `row` of U^T and L^T
    // every run col[r0 + cc .. +CK) of a full block starts 16-byte aligned
    const bool vec = (reinterpret_cast<uintptr_t>(LU) % 16 == 0) && (p.lda % (16 / (int)sizeof(T)) == 0);

    const int P = (n + BS - 1) / BS;
    // U^T w = b, blocks ascending
    for (int kb = 0; kb < P; ++kb) {
        const int r0 = kb * BS;
        const int w = min(BS, n - r0);
        T* yb = ybuf + (size_t)(kb & 1) * BS * NRT;
        if (wave == r0 / 64) {
            const int base = r0 % 64;
            const int mrow = lane - base;
#pragma unroll
            for (int cc = 0; cc < BS; cc += CK) {
                T urow[CK];   // (U^T)_{mrow,c} = u_{c,mrow}, diagonal included
#pragma unroll
                for (int e = 0; e < CK; ++e) {
                    const int c = cc + e;
                    urow[e] = (mrow >= c && mrow < w) ? op_entry<CONJ>(col[r0 + c]) : O::zero();
                }
#pragma unroll
                for (int e = 0; e < CK; ++e) {
                    const int c = cc + e;
                    if (c >= w) continue;
                    T xc[NRT];
                    if constexpr (NRT == 1) {
                        if (mrow == c) y[0] = O::div(y[0], urow[e]);
                        xc[0] = readlane_t(y[0], base + c);
                    } else {
                        diag_divide(y, xc, urow[e], base + c, lane);
                    }
                    if (mrow > c && mrow < w)
#pragma unroll
                        for (int r = 0; r < NRT; ++r) O::fms(y[r], urow[e], xc[r]);
                }
            }
            if (mrow >= 0 && mrow < w)
#pragma unroll
                for (int r = 0; r < NRT; ++r) yb[mrow * NRT + r] = y[r];
        }
        __syncthreads();
        if (have && row >= r0 + w) {
#pragma unroll
            for (int cc = 0; cc < BS; cc += CK) {
                T urow[CK];
                if (vec && w == BS) {
                    load_column_run<CONJ>(urow, col + r0 + cc);
                } else {
#pragma unroll
                    for (int e = 0; e < CK; ++e)
                        urow[e] = cc + e < w ? op_entry<CONJ>(col[r0 + cc + e]) : O::zero();
                }
#pragma unroll
                for (int e = 0; e < CK; ++e) {
                    if (cc + e >= w) continue;
#pragma unroll
                    for (int r = 0; r < NRT; ++r) O::fms(y[r], urow[e], yb[(cc + e) * NRT + r]);
                }
            }
        }
    }
    __syncthreads();
    // L^T z = w (unit diagonal), blocks descending
    for (int kb = P - 1; kb >= 0; --kb) {
        const int r0 = kb * BS;
        const int w = min(BS, n - r0);
        T* yb = ybuf + (size_t)(kb & 1) * BS * NRT;
        if (wave == r0 / 64) {
            const int base = r0 % 64;
            const int mrow = lane - base;
#pragma unroll
            for (int cc = BS - CK; cc >= 0; cc -= CK) {
                T lrow[CK];   // (L^T)_{mrow,c} = l_{c,mrow}, strictly above the diagonal
#pragma unroll
                for (int e = 0; e < CK; ++e) {
                    const int c = cc + e;
                    lrow[e] = (mrow >= 0 && mrow < c && c < w) ? op_entry<CONJ>(col[r0 + c]) : O::zero();
                }
#pragma unroll
                for (int e = CK - 1; e >= 0; --e) {
                    const int c = cc + e;
                    if (c >= w) continue;
                    T xc[NRT];
#pragma unroll
                    for (int r = 0; r < NRT; ++r) xc[r] = readlane_t(y[r], base + c);
                    if (mrow >= 0 && mrow < c)
#pragma unroll
                        for (int r = 0; r < NRT; ++r) O::fms(y[r], lrow[e], xc[r]);
                }
            }
            if (mrow >= 0 && mrow < w)
#pragma unroll
                for (int r = 0; r < NRT; ++r) yb[mrow * NRT + r] = y[r];
        }
        __syncthreads();
        if (have && row < r0) {
#pragma unroll
            for (int cc = BS - CK; cc >= 0; cc -= CK) {
                T lrow[CK];
                if (vec && w == BS) {
                    load_column_run<CONJ>(lrow, col + r0 + cc);
                } else {
#pragma unroll
                    for (int e = 0; e < CK; ++e)
                        lrow[e] = cc + e < w ? op_entry<CONJ>(col[r0 + cc + e]) : O::zero();
                }
#pragma unroll
                for (int e = CK - 1; e >= 0; --e) {
                    if (cc + e >= w) continue;
#pragma unroll
                    for (int r = 0; r < NRT; ++r) O::fms(y[r], lrow[e], yb[(cc + e) * NRT + r]);
                }
            }
        }
    }
    if (have)
#pragma unroll
        for (int r = 0; r < NRT; ++r)
            if (c0 + r < p.nrhs) B[dst + (long long)(c0 + r) * p.ldb] = y[r];
}

template <typename T, int NRT>
hipError_t launch_t(const Problem& p, hipStream_t s) {
    const int threads = ((p.n + 63) / 64) * 64;
    const int rt = (p.nrhs + NRT - 1) / NRT;
    const size_t smem = ((p.n * 4 + 15) / 16) * 16 + 2 * BS * NRT * sizeof(T);
    const dim3 grid((unsigned)((long long)p.batch * rt));
    if (p.inverse) {
        hipLaunchKernelGGL((getrs_rows_kernel<T, NRT, true>), grid, dim3(threads), smem, s, p, rt);
    } else if (p.trans == 0) {
        hipLaunchKernelGGL((getrs_rows_kernel<T, NRT, false>), grid, dim3(threads), smem, s, p, rt);
    } else if constexpr (ops<T>::is_complex) {
        if (p.trans == 2)
            hipLaunchKernelGGL((getrs_rows_trans_kernel<T, NRT, true>), grid, dim3(threads), smem, s, p, rt);
        else
            hipLaunchKernelGGL((getrs_rows_trans_kernel<T, NRT, false>), grid, dim3(threads), smem, s, p, rt);
    } else {   // A^H = A^T for real data
        hipLaunchKernelGGL((getrs_rows_trans_kernel<T, NRT, false>), grid, dim3(threads), smem, s, p, rt);
    }
    return hipGetLastError();
}

}  // namespace

bool getrs_rows_supported(int dtype, int n) {
    (void)dtype;
    return n >= 1 && n <= 1024;
}

hipError_t getrs_rows_launch(int dtype, const Problem& p, hipStream_t s) {
    if (!getrs_rows_supported(dtype, p.n)) return hipErrorInvalidValue;
    // right-hand sides per work-group (each group streams all of L and U;
    // wider tiles were measured slower at n = 1024, nrhs = 32: fewer groups)
    const int r = p.nrhs;
    if (p.inverse) {
        // getri has n columns, so wide tiles still leave many work-groups;
        // each tile streams the factors once, so wider is fewer passes
        switch (dtype) {
        case R32: return r <= 4 ? launch_t<float, 4>(p, s) : launch_t<float, 16>(p, s);
        case R64: return r <= 4 ? launch_t<double, 4>(p, s) : launch_t<double, 8>(p, s);
        case C64: return r <= 4 ? launch_t<cplx<float>, 4>(p, s) : launch_t<cplx<float>, 8>(p, s);
        case C128: return launch_t<cplx<double>, 4>(p, s);
        default: return hipErrorInvalidValue;
        }
    }
    // orders to 256 with many right-hand sides and batches of 512 or more:
    // wider tiles stream the factors fewer times while the batch still gives
    // enough work-groups (measured, solve alone: double n = 256, nrhs = 16,
    // batch 1024 0.70 -> 0.42 ms; complex double n = 128, nrhs = 16 0.58 ->
    // 0.36; float n = 256 0.38 -> 0.34).  Not above 256 (equal or slower),
    // not for complex float (up to 2x slower), not at batch <= 256 (the gesv
    // that factors then solves, double n = 32 - 64 with 16 right-hand sides,
    // went 27 - 43 % slower), and not where a tile would be half empty
    // (double n = 64 with 8 right-hand sides in 16-wide tiles: 0.27 -> 0.40 ms).
    if (p.n <= 256 && p.batch >= 512) {
        if ((dtype == R32 || dtype == R64) && r > 8)
            return dtype == R32 ? launch_t<float, 16>(p, s) : launch_t<double, 16>(p, s);
        if (dtype == C128 && r > 4) return launch_t<cplx<double>, 8>(p, s);
    }
    switch (dtype) {
    case R32: return r <= 1 ? launch_t<float, 1>(p, s) : launch_t<float, 4>(p, s);
    case R64: return r <= 1 ? launch_t<double, 1>(p, s) : launch_t<double, 4>(p, s);
    case C64: return r <= 1 ? launch_t<cplx<float>, 1>(p, s) : r <= 2 ? launch_t<cplx<float>, 2>(p, s)
                                                              : launch_t<cplx<float>, 4>(p, s);
    case C128: return r <= 1 ? launch_t<cplx<double>, 1>(p, s) : launch_t<cplx<double>, 2>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace batchlu
