// getrs_direct.hip -- solve A X = B from packed LU factors and ipiv, one
// work-group per (matrix, tile of right-hand-side columns), any order n.
//
// BatchLAS "LU" page, fused getrs paragraph: one work-group per matrix does
// the permutation, the forward substitution against unit-lower L and the back
// substitution against U in one launch, without a GEMM or a separate
// interchange kernel.  Here the right-hand sides live in registers (a thread
// owns rows tid, tid + T, ...), the row of the step is broadcast through LDS,
// and the permutation is a per-row backward trace of the interchange list
// (the getri paragraph of the same page), so nothing is written before every
// row has been read.  The operation order per element is the plain one:
// forward y_i -= l_ik y_k in ascending k, back x_k = y_k / u_kk then
// y_i -= u_ik x_k in descending k.
#include "device_ops.h"
#include "internal.h"

namespace batchlu {

namespace {

constexpr int kThreads = 256;

template <typename T, int NRT, int MAXQ>
__global__ void __launch_bounds__(kThreads) getrs_direct_kernel(Problem p)
{
    using O = ops<T>;
    extern __shared__ uint4 smem_raw[];
    int* sipiv = (int*)smem_raw;                                   // n entries
    T* yk = (T*)((char*)smem_raw + ((p.n * 4 + 15) / 16) * 16);    // NRT entries

    const int n = p.n;
    const long long m = blockIdx.x;
    const int c0 = blockIdx.y * NRT;
    const int tid = threadIdx.x;
    const int nt = blockDim.x;

    // composed gesv passes info: a matrix whose factorisation failed keeps B
    if (p.info && p.info[m] != 0) return;

    const T* LU = (const T*)p.A + m * p.sA;
    const int* ipiv = p.ipiv + m * p.sP;
    T* B = (T*)p.B + m * p.sB;

    for (int i = tid; i < n; i += nt) sipiv[i] = ipiv[i] - 1;
    __syncthreads();

    // a8: position i of P*B holds original row perm(i); trace each row back
    T y[MAXQ][NRT];
#pragma unroll
    for (int q = 0; q < MAXQ; ++q) {
        const int i = tid + q * nt;
        int src = i;
        if (i < n) {
            for (int k = n - 1; k >= 0; --k) {
                const int pk = sipiv[k];
                src = (src == k) ? pk : (src == pk ? k : src);
            }
        }
#pragma unroll
        for (int r = 0; r < NRT; ++r) {
            T v = O::zero();
            if (i < n && c0 + r < p.nrhs) v = B[src + (long long)(c0 + r) * p.ldb];
            y[q][r] = v;
        }
    }
    __syncthreads();   // every read of B is done before any write below

    // a9: forward substitution, L unit-lower
    for (int k = 0; k < n; ++k) {
        const int owner = k % nt, oq = k / nt;
        if (tid == owner) {
#pragma unroll
            for (int q = 0; q < MAXQ; ++q)
                if (q == oq)
#pragma unroll
                    for (int r = 0; r < NRT; ++r) yk[r] = y[q][r];
        }
        __syncthreads();
        T x[NRT];
#pragma unroll
        for (int r = 0; r < NRT; ++r) x[r] = yk[r];
#pragma unroll
        for (int q = 0; q < MAXQ; ++q) {
            const int i = tid + q * nt;
            if (i > k && i < n) {
                const T l = LU[i + (long long)k * p.lda];
#pragma unroll
                for (int r = 0; r < NRT; ++r) O::fms(y[q][r], l, x[r]);
            }
        }
        __syncthreads();
    }

    // a10: back substitution, U upper with its diagonal
    for (int k = n - 1; k >= 0; --k) {
        const int owner = k % nt, oq = k / nt;
        if (tid == owner) {
            const T d = LU[k + (long long)k * p.lda];
#pragma unroll
            for (int q = 0; q < MAXQ; ++q)
                if (q == oq)
#pragma unroll
                    for (int r = 0; r < NRT; ++r) {
                        y[q][r] = O::div(y[q][r], d);
                        yk[r] = y[q][r];
                    }
        }
        __syncthreads();
        T x[NRT];
#pragma unroll
        for (int r = 0; r < NRT; ++r) x[r] = yk[r];
#pragma unroll
        for (int q = 0; q < MAXQ; ++q) {
            const int i = tid + q * nt;
            if (i < k) {
                const T u = LU[i + (long long)k * p.lda];
#pragma unroll
                for (int r = 0; r < NRT; ++r) O::fms(y[q][r], u, x[r]);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int q = 0; q < MAXQ; ++q) {
        const int i = tid + q * nt;
        if (i < n)
#pragma unroll
            for (int r = 0; r < NRT; ++r)
                if (c0 + r < p.nrhs) B[i + (long long)(c0 + r) * p.ldb] = y[q][r];
    }
}

template <typename T, int NRT>
hipError_t launch_t(const Problem& p, hipStream_t s) {
    const int threads = p.n <= 64 ? 64 : (p.n <= 128 ? 128 : kThreads);
    const int q = (p.n + threads - 1) / threads;
    const size_t smem = ((p.n * 4 + 15) / 16) * 16 + NRT * sizeof(T);
    dim3 grid((unsigned)p.batch, (unsigned)((p.nrhs + NRT - 1) / NRT));
#define BATCHLU_Q(QV)                                                                        \
    if (q <= QV) {                                                                           \
        hipLaunchKernelGGL((getrs_direct_kernel<T, NRT, QV>), grid, dim3(threads), smem, s, p); \
        return hipGetLastError();                                                            \
    }
    BATCHLU_Q(1) BATCHLU_Q(2) BATCHLU_Q(4) BATCHLU_Q(8) BATCHLU_Q(16)
#undef BATCHLU_Q
    return hipErrorInvalidValue;
}

}  // namespace

bool getrs_direct_supported(int dtype, int n, int nrhs) {
    (void)dtype;
    (void)nrhs;
    return n >= 1 && n <= 16 * kThreads;
}

hipError_t getrs_direct_launch(int dtype, const Problem& p, hipStream_t s) {
    if (!getrs_direct_supported(dtype, p.n, p.nrhs)) return hipErrorInvalidValue;
    switch (dtype) {
    case R32: return launch_t<float, 4>(p, s);
    case R64: return launch_t<double, 2>(p, s);
    case C64: return launch_t<cplx<float>, 2>(p, s);
    case C128: return launch_t<cplx<double>, 1>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace batchlu
