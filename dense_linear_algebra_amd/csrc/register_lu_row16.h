// register_lu_row16.h -- register-resident LU and fused gesv for float
// matrices of order 9..32, one matrix per 16-lane DPP row.
//
// Same method and operation order as register_lu_kernel.h (lazy relabel,
// DPP argmax with lowest-position ties, one fma per element and step), with
// the pivot row moved by DPP instead of LDS broadcast reads:
//   - the owner lane writes the pivot row to a per-matrix LDS row; each of
//     the 16 lanes of the matrix reads back ONE 16-byte chunk of it (one
//     ds_read_b128 per step instead of one per chunk);
//   - every element of the pivot row then reaches the whole matrix by a
//     row_newbcast DPP move from the lane holding its chunk (the source lane
//     is a compile-time constant because the row chunk index is);
//   - after elimination the rows are put in position order once (through a
//     one-chunk LDS stage), so the back substitution broadcasts x_k from a
//     static lane by DPP as well and needs no LDS round trip per step, and
//     L, U and X are stored with row-contiguous vector writes.
// The pages' tiny tier publishes the pivot row through local memory (LU
// page, local-row broadcast paragraph); here the broadcast itself rides on
// DPP, which a 16-lane row of a wave64 supports natively.
#pragma once

#include <type_traits>

#include "device_ops.h"
#include "internal.h"

namespace batchlu {

namespace row16_detail {

constexpr int kWaves = 4;   // wavefronts per block

// row_newbcast:L broadcasts lane L of every 16-lane row to the whole row
template <int L>
__device__ inline float bcast(float v) {
    static_assert(L >= 0 && L < 16, "lane");
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + L, 0xF, 0xF,
                                                              false));
}

template <int I, int N, typename F>
__device__ inline void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

template <int NB, int NR>
__global__ void __launch_bounds__(64 * kWaves) row16_kernel(Problem p, int mode)
{
    using O = ops<float>;
    constexpr int RPL = NB / 16;                 // rows per lane
    constexpr int GPB = 4 * kWaves;              // matrices per block
    constexpr int NBC = NB / 4;                  // 16-byte chunks of an A row
    constexpr int NRC = (NR + 3) / 4;            // chunks of a B row
    constexpr int NRP = NRC * 4 > 0 ? NRC * 4 : 1;
    constexpr int ROWC = NBC + NRC;              // chunks of a row: at most 16
    static_assert(NB == 16 || NB == 32, "row16 handles buckets 16 and 32");
    static_assert(ROWC <= 16, "a row must fit one chunk per lane");

    __shared__ uint4 rowbuf[GPB][ROWC];          // the pivot row of the step
    __shared__ uint4 stage[GPB][NB];             // one chunk column, rows by position
    __shared__ float diag[GPB][NB];              // 1/u_jj
    __shared__ float dval[GPB][NB];              // u_jj

    const int lane = threadIdx.x & 63;
    const int grp = (threadIdx.x >> 6) * 4 + (lane >> 4);
    const int li = lane & 15;
    const int n = p.n;

    long long m = (long long)blockIdx.x * GPB + grp;
    const bool live = m < p.batch;
    if (!live) m = p.batch - 1;
    float* A = (float*)p.A + m * p.sA;
    float* B = (float*)p.B + m * p.sB;
    const bool solve = (NR > 0) && mode == MODE_GESV;

    float a[RPL][NB];
    float b[RPL][NRP];
    int pos[RPL];

    // ---- load ---------------------------------------------------------------
    const bool full = (n == NB) && ((p.lda & (RPL - 1)) == 0) && (((uintptr_t)A) % (4 * RPL) == 0);
#pragma unroll
    for (int s = 0; s < RPL; ++s) pos[s] = li * RPL + s;
    if (full) {
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            if constexpr (RPL == 2) {
                const float2 w = *(const float2*)(A + li * 2 + (long long)k * p.lda);
                a[0][k] = w.x;
                a[1][k] = w.y;
            } else {
                a[0][k] = A[li + (long long)k * p.lda];
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < NB; ++k)
#pragma unroll
            for (int s = 0; s < RPL; ++s) {
                const int row = li * RPL + s;
                float v = (row == k) ? 1.0f : 0.0f;
                if (k < n && row < n) v = A[row + (long long)k * p.lda];
                a[s][k] = v;
            }
    }
#pragma unroll
    for (int r = 0; r < NRP; ++r)
#pragma unroll
        for (int s = 0; s < RPL; ++s) {
            const int row = li * RPL + s;
            float v = 0.0f;
            if (solve && r < NR && r < p.nrhs && row < n) v = B[row + (long long)r * p.ldb];
            b[s][r] = v;
        }

    int info = 0;
    int pivrec[NB / 16];
#pragma unroll
    for (int t = 0; t < NB / 16; ++t) pivrec[t] = 0;

    // ---- elimination ----------------------------------------------------------
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        if (j >= n) continue;
        uint32_t key[RPL];
        uint32_t kmax = 0;
#pragma unroll
        for (int s = 0; s < RPL; ++s) {
            const uint32_t kk = (pos[s] >= j) ? pivot_key(__builtin_fabsf(a[s][j])) : 0u;
            key[s] = kk;
            kmax = kk > kmax ? kk : kmax;
        }
        kmax = group_max<16>(kmax);
        int q = 0x7fffffff;
#pragma unroll
        for (int s = 0; s < RPL; ++s)
            if (key[s] == kmax && pos[s] < q) q = pos[s];
        const int piv_pos = group_min<16>(q);
        if (li == j % 16) pivrec[j / 16] = piv_pos;

        // the owner writes its row from the chunk holding column j
#pragma unroll
        for (int s = 0; s < RPL; ++s) {
            if (pos[s] == piv_pos) {
#pragma unroll
                for (int c = 0; c < NBC; ++c) {
                    if (c < j / 4) continue;
                    rowbuf[grp][c] = make_uint4(__float_as_uint(a[s][4 * c]), __float_as_uint(a[s][4 * c + 1]),
                                                __float_as_uint(a[s][4 * c + 2]), __float_as_uint(a[s][4 * c + 3]));
                }
                if constexpr (NRC > 0) {
                    if (solve) {
#pragma unroll
                        for (int c = 0; c < NRC; ++c)
                            rowbuf[grp][NBC + c] =
                                make_uint4(__float_as_uint(b[s][4 * c]), __float_as_uint(b[s][4 * c + 1]),
                                           __float_as_uint(b[s][4 * c + 2]), __float_as_uint(b[s][4 * c + 3]));
                    }
                }
            }
        }
#pragma unroll
        for (int s = 0; s < RPL; ++s)
            pos[s] = (pos[s] == piv_pos) ? j : (pos[s] == j ? piv_pos : pos[s]);

        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // lane li holds chunk li of the pivot row
        const uint4 chw = rowbuf[grp][li < ROWC ? li : 0];
        const float ch[4] = {__uint_as_float(chw.x), __uint_as_float(chw.y), __uint_as_float(chw.z),
                             __uint_as_float(chw.w)};
        float u[NB];
        float ub[NRP];
        static_for<0, NB>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            if (k >= j) u[k] = bcast<k / 4>(ch[k % 4]);
        });
        if constexpr (NR > 0) {
            if (solve)
                static_for<0, NR>([&](auto rc) {
                    constexpr int r2 = decltype(rc)::value;
                    ub[r2] = bcast<NBC + r2 / 4>(ch[r2 % 4]);
                });
        }

        const float piv = u[j];
        const float pm = __builtin_fabsf(piv);
        const bool zero = pm == 0.0f;
        if (zero && info == 0) info = j + 1;
        const float r = 1.0f / piv;
        const bool small = !(pm >= O::sfmin());
        if (li == 0) {
            diag[grp][j] = r;
            dval[grp][j] = piv;
        }
        float lm[RPL];
#pragma unroll
        for (int s = 0; s < RPL; ++s) lm[s] = a[s][j] * r;
        if (__builtin_amdgcn_ballot_w64(small) != 0) {
            asm volatile("" ::: "memory");
#pragma unroll
            for (int s = 0; s < RPL; ++s)
                if (small) lm[s] = a[s][j] / piv;
        }
#pragma unroll
        for (int s = 0; s < RPL; ++s) {
            if (pos[s] > j && !zero) {
                const float l = lm[s];
                a[s][j] = l;
#pragma unroll
                for (int k = 0; k < NB; ++k)
                    if (k > j) a[s][k] = __builtin_fmaf(-l, u[k], a[s][k]);
                if constexpr (NR > 0) {
                    if (solve)
#pragma unroll
                        for (int r2 = 0; r2 < NR; ++r2) b[s][r2] = __builtin_fmaf(-l, ub[r2], b[s][r2]);
                }
            }
        }
    }

    // ---- rows into position order (one chunk column at a time) -------------
    // slot s of lane li then holds the row at position li*RPL + s
#pragma unroll
    for (int c = 0; c < ROWC; ++c) {
        if (c >= NBC && !solve) continue;
#pragma unroll
        for (int s = 0; s < RPL; ++s) {
            float* src = c < NBC ? &a[s][4 * c] : &b[s][4 * (c - NBC)];
            stage[grp][pos[s]] = make_uint4(__float_as_uint(src[0]), __float_as_uint(src[1]),
                                            __float_as_uint(src[2]), __float_as_uint(src[3]));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int s = 0; s < RPL; ++s) {
            const uint4 w = stage[grp][li * RPL + s];
            float* dst = c < NBC ? &a[s][4 * c] : &b[s][4 * (c - NBC)];
            dst[0] = __uint_as_float(w.x);
            dst[1] = __uint_as_float(w.y);
            dst[2] = __uint_as_float(w.z);
            dst[3] = __uint_as_float(w.w);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- back substitution, x_k broadcast by DPP from its static lane -------
    if constexpr (NR > 0) {
        if (solve) {
            float rd[RPL], dv[RPL];
#pragma unroll
            for (int s = 0; s < RPL; ++s) {
                rd[s] = diag[grp][li * RPL + s];
                dv[s] = dval[grp][li * RPL + s];
            }
            static_for<0, NB>([&](auto ic) {
                constexpr int k = NB - 1 - decltype(ic)::value;
                constexpr int ks = k % RPL;
                constexpr int kl = k / RPL;
                if (k < n) {
                    // the owner (lane kl, slot ks) forms x_k; every lane reads it by DPP
                    float own[NR];
#pragma unroll
                    for (int r2 = 0; r2 < NR; ++r2) own[r2] = b[ks][r2] * rd[ks];
                    const bool tiny = !(__builtin_fabsf(dv[ks]) >= O::sfmin());
                    if (__builtin_amdgcn_ballot_w64(tiny && li == kl) != 0) {
                        asm volatile("" ::: "memory");
                        if (tiny)
#pragma unroll
                            for (int r2 = 0; r2 < NR; ++r2) own[r2] = b[ks][r2] / dv[ks];
                    }
                    float xk[NR];
#pragma unroll
                    for (int r2 = 0; r2 < NR; ++r2) xk[r2] = bcast<kl>(own[r2]);
                    if (li == kl) {
#pragma unroll
                        for (int r2 = 0; r2 < NR; ++r2) b[ks][r2] = xk[r2];
                    }
#pragma unroll
                    for (int s = 0; s < RPL; ++s) {
                        if (li * RPL + s < k) {
#pragma unroll
                            for (int r2 = 0; r2 < NR; ++r2) b[s][r2] = __builtin_fmaf(-a[s][k], xk[r2], b[s][r2]);
                        }
                    }
                }
            });
        }
    }

    // ---- store (rows now in position order) ----------------------------------
    if (!live) return;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        if (k >= n) continue;
        if (full && RPL == 2) {
            *(float2*)(A + li * 2 + (long long)k * p.lda) = make_float2(a[0][k], a[RPL - 1][k]);
        } else {
#pragma unroll
            for (int s = 0; s < RPL; ++s)
                if (li * RPL + s < n) A[li * RPL + s + (long long)k * p.lda] = a[s][k];
        }
    }
    int* ipiv = p.ipiv + m * p.sP;
#pragma unroll
    for (int t = 0; t < NB / 16; ++t) {
        const int j = t * 16 + li;
        if (j < n) ipiv[j] = pivrec[t] + 1;
    }
    if (li == 0) p.info[m] = info;
    if constexpr (NR > 0) {
        if (solve && info == 0) {
            const bool bfull = full && ((p.ldb & (RPL - 1)) == 0) && (((uintptr_t)B) % (4 * RPL) == 0);
#pragma unroll
            for (int r2 = 0; r2 < NR; ++r2) {
                if (r2 >= p.nrhs) continue;
                if (bfull && RPL == 2) {
                    *(float2*)(B + li * 2 + (long long)r2 * p.ldb) = make_float2(b[0][r2], b[RPL - 1][r2]);
                } else {
#pragma unroll
                    for (int s = 0; s < RPL; ++s)
                        if (li * RPL + s < n) B[li * RPL + s + (long long)r2 * p.ldb] = b[s][r2];
                }
            }
        }
    }
}

template <int NB, int NR>
hipError_t launch(const Problem& p, int mode, hipStream_t s) {
    constexpr int GPB = 4 * kWaves;
    const long long blocks = (p.batch + GPB - 1) / GPB;
    hipLaunchKernelGGL((row16_kernel<NB, NR>), dim3((unsigned)blocks), dim3(64 * kWaves), 0, s, p, mode);
    return hipGetLastError();
}

// float, 9 <= n <= 32; nr is the right-hand-side bucket (0 for getrf)
inline hipError_t launch_row16(const Problem& p, int mode, int nr, hipStream_t s) {
    const int nb = p.n <= 16 ? 16 : 32;
#define BATCHLU_R16(NBV, NRV) \
    if (nb == NBV && nr == NRV) return launch<NBV, NRV>(p, mode, s);
    BATCHLU_R16(16, 0) BATCHLU_R16(16, 1) BATCHLU_R16(16, 8) BATCHLU_R16(16, 16)
    BATCHLU_R16(32, 0) BATCHLU_R16(32, 1) BATCHLU_R16(32, 8) BATCHLU_R16(32, 16)
#undef BATCHLU_R16
    return hipErrorInvalidValue;
}

}  // namespace row16_detail

}  // namespace batchlu
