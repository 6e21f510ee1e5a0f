// register_lu_kernel.h -- register-resident LU with partial pivoting, and the
// fused factor-and-solve, for small matrices (n <= 64) on gfx950.
//
// Design (BatchLAS "LU" page, tiny-tier paragraph and the gesv-tiny
// paragraph; redesigned for wave64):
//   - A matrix lives in a group of LPM lanes of one wavefront; each lane owns
//     RPL consecutive rows (row = RPL*lane_in_group + slot) of A and of B in
//     VGPRs.  64 / LPM matrices share a wavefront.  Rows and columns past n
//     carry the identity, so the unrolled body needs no per-row guards.
//   - Row interchanges are lazy: each slot carries its current position
//     `pos`; a step relabels two positions and moves no data.
//   - Pivot search: per-slot keys (metric bits + 1, NaN mapped) reduced with
//     DPP / ds_swizzle inside the group; ties go to the lowest position by a
//     second min-reduction over positions.
//   - The pivot row is published through a per-group LDS row (one lane
//     writes, the group reads it back as a broadcast).  All lanes of a group
//     are in one wavefront and LDS operations of a wavefront complete in
//     order, so no barrier is needed.
//   - For gesv the right-hand sides ride along as extra columns of the rank-1
//     update (the forward solve).  The back substitution multiplies by the
//     reciprocal of each diagonal entry, computed once at its elimination
//     step (BatchLAS "Blackwell" page, getrs tiny paragraph); each entry of
//     x_k is formed by one lane and staged in LDS, where the rows above read
//     it back, and X leaves from the stage with row-contiguous vector writes.
// Arithmetic per element is the same operation sequence as the unblocked
// right-looking LU, so L, U and ipiv are bit-identical to it.
#pragma once

#include "device_ops.h"
#include "internal.h"

namespace batchlu {

namespace reg_detail {

constexpr int kWavesPerBlock = 4;

template <int BYTES>
struct vecbits;
template <>
struct vecbits<4> { using type = uint32_t; };
template <>
struct vecbits<8> { using type = uint2; };
template <>
struct vecbits<16> { using type = uint4; };

// Rows of 512 bytes (64 doubles or complex floats, 32 complex doubles) take
// the pivot row a chunk at a time where the update consumes it instead of
// holding it whole; the registers are then budgeted for two wavefronts per
// SIMD wherever that fits without spilling (checked in the compiler's
// resource report), so that one wavefront's latency overlaps another's work.
template <typename T, int NB>
constexpr bool reg_chunked() { return NB * (int)sizeof(T) >= 512; }
template <typename T, int NB, int NR>
constexpr int reg_waves() {
    if (!reg_chunked<T, NB>()) return 1;
    // one matrix per wavefront with its one right-hand side in LDS: three,
    // as without B
    if (NR == 1 && NB == 64 && sizeof(T) == 8) return 3;
    if (sizeof(T) == 8) return (ops<T>::is_complex || NR <= 8) ? 2 : 1;
    return NR <= 1 ? 2 : 1;
}

template <typename T, int NB, int RPL, int NR>
__global__ void __launch_bounds__(64 * kWavesPerBlock) __attribute__((amdgpu_waves_per_eu(reg_waves<T, NB, NR>())))
register_lu_kernel(Problem p, int mode)
{
    using O = ops<T>;
    using R = typename O::R;
    using K = typename O::K;
    constexpr int LPM = NB / RPL;                  // lanes per matrix
    constexpr int GPW = 64 / LPM;                  // matrices per wavefront
    constexpr int GPB = GPW * kWavesPerBlock;      // matrices per block
    constexpr int CH = 16 / (int)sizeof(T);        // elements per 16-byte chunk
    constexpr int NBC = NB / CH;                   // chunks of an A row
    constexpr int NRC = (NR + CH - 1) / CH;        // chunks of a B row
    constexpr int NRP = NRC * CH > 0 ? NRC * CH : 1;
    constexpr int ROWC = NBC + NRC;
    constexpr int NPIV = (NB + LPM - 1) / LPM;     // pivots recorded per lane
    // one matrix per wavefront with 512-byte rows and one right-hand side:
    // B lives in LDS (row i of B at bst row i), not in VGPRs, so that the
    // kernel fits three wavefronts per SIMD like the factorisation alone;
    // x_k then overwrites y_k in place and X leaves from there.  (Measured:
    // complex float n = 64, batch 8192: 0.468 -> 0.407 ms; with 8 or 16
    // right-hand sides the per-step LDS traffic costs more than the third
    // wavefront gains, 0.57 -> 0.59 and 0.72 -> 1.08 ms, so those keep B in
    // VGPRs.)
    constexpr bool BL = NR == 1 && LPM == 64 && RPL == 1 && reg_chunked<T, NB>();
    constexpr int XC = (NR > 0 && !BL) ? NB * NRC : 1;      // chunks of the staged X
    constexpr int DGC = NR > 0 ? (2 * NB + CH - 1) / CH : 1;   // chunks of (1/u_jj, u_jj)
    constexpr int VB = RPL * (int)sizeof(T);       // bytes of a lane's rows in one column
    static_assert(NB % CH == 0 && NB % RPL == 0 && LPM <= 64 && 64 % LPM == 0, "bad shape");

    __shared__ uint4 rowbuf[GPB][ROWC];
    __shared__ uint4 xstage[GPB][XC];   // X row k at chunks [k*NRC, (k+1)*NRC)
    __shared__ uint4 diagbuf[GPB][DGC]; // (1/u_jj, u_jj) of every step j
    __shared__ uint4 bst[BL ? GPB * NB * NRC : 1];   // B rows (BL)

    const int lane = threadIdx.x & 63;
    const int grp = (threadIdx.x >> 6) * GPW + lane / LPM;
    const int li = lane % LPM;
    const int n = p.n;

    long long m = (long long)blockIdx.x * GPB + grp;
    const bool live = m < p.batch;
    if (!live) m = p.batch - 1;   // idle groups factor a copy and store nothing

    T* A = (T*)p.A + m * p.sA;
    T* B = (T*)p.B + m * p.sB;
    const bool solve = (NR > 0) && mode == MODE_GESV;
    T* diag = (T*)&diagbuf[grp][0];

    T a[RPL][NB];
    T b[RPL][NRP];
    int pos[RPL];

    // ---- load (identity padding past n) ----------------------------------
    const bool full = (n == NB) && (VB <= 16) && ((p.lda * sizeof(T)) % VB == 0) &&
                      (((uintptr_t)A) % VB == 0);
#pragma unroll
    for (int s = 0; s < RPL; ++s) pos[s] = li * RPL + s;
    if constexpr (VB <= 16) {
        using V = typename vecbits<VB>::type;
        if (full) {
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                V w = *(const V*)(A + li * RPL + (long long)k * p.lda);
                T tmp[RPL];
                __builtin_memcpy(tmp, &w, sizeof(tmp));
#pragma unroll
                for (int s = 0; s < RPL; ++s) a[s][k] = tmp[s];
            }
        }
    }
    if (!full) {
#pragma unroll
        for (int k = 0; k < NB; ++k) {
#pragma unroll
            for (int s = 0; s < RPL; ++s) {
                const int row = li * RPL + s;
                T v = (row == k) ? O::one() : O::zero();
                if (k < n && row < n) v = A[row + (long long)k * p.lda];
                a[s][k] = v;
            }
        }
    }
    if constexpr (BL) {
        // row li of B into its LDS row (zero past nrhs and n)
#pragma unroll
        for (int c = 0; c < NRC; ++c) {
            T v[CH];
#pragma unroll
            for (int e = 0; e < CH; ++e) {
                const int r = c * CH + e;
                v[e] = (solve && r < NR && r < p.nrhs && li < n) ? B[li + (long long)r * p.ldb] : O::zero();
            }
            uint4 w;
            __builtin_memcpy(&w, v, 16);
            bst[(grp * NB + li) * NRC + c] = w;
        }
    } else {
#pragma unroll
        for (int r = 0; r < NRP; ++r) {
#pragma unroll
            for (int s = 0; s < RPL; ++s) {
                const int row = li * RPL + s;
                T v = O::zero();
                if (solve && r < NR && r < p.nrhs && row < n) v = B[row + (long long)r * p.ldb];
                b[s][r] = v;
            }
        }
    }

    // ---- elimination -------------------------------------------------------
    int info = 0;
    int pivrec[NPIV];
#pragma unroll
    for (int t = 0; t < NPIV; ++t) pivrec[t] = 0;

#pragma unroll
    for (int j = 0; j < NB; ++j) {
        if (j >= n) continue;   // uniform; keeps the trip count constant for full unrolling

        // a1: argmax of the metric over rows at positions >= j
        K key[RPL];
        K kmax = 0;
#pragma unroll
        for (int s = 0; s < RPL; ++s) {
            // rows past n pad the bucket; never candidates (0 * inf in their
            // updates can make them NaN, which would outrank real rows)
            K kk = (pos[s] >= j && pos[s] < n) ? (K)pivot_key(O::metric(a[s][j])) : (K)0;
            key[s] = kk;
            kmax = kk > kmax ? kk : kmax;
        }
        int piv_pos;
        int owner = 0;   // lane holding the pivot row (LPM == 64)
        T piv_early = O::zero();
        if constexpr (LPM == 64) {
            // one matrix per wavefront (one row per lane): DPP inside rows
            // of 16 lanes and readlane across them, no LDS round trips; the
            // position reduction runs only when several rows share the key.
            // The pivot itself is read from the winning lane here, so that
            // its reciprocal does not wait for the pivot row's round trip.
            int win;
            wave_argmax(key[0], pos[0], kmax, win);
            win = win < 0 ? 0 : win;
            owner = win;
            piv_pos = __builtin_amdgcn_readlane(pos[0], win);
            piv_early = readlane_t(a[0][j], win);
        } else {
            kmax = group_max<LPM>(kmax);
            int q = 0x7fffffff;
#pragma unroll
            for (int s = 0; s < RPL; ++s)
                if (key[s] == kmax && pos[s] < q) q = pos[s];
            piv_pos = group_min<LPM>(q);
        }
        if (li == j % LPM) pivrec[j / LPM] = piv_pos;

        // publish the pivot row (chunks from the one holding column j)
#pragma unroll
        for (int s = 0; s < RPL; ++s) {
            if (pos[s] == piv_pos) {
#pragma unroll
                for (int c = 0; c < NBC; ++c) {
                    if (c < j / CH) continue;
                    uint4 w;
                    __builtin_memcpy(&w, &a[s][c * CH], 16);
                    rowbuf[grp][c] = w;
                }
                if constexpr (NRC > 0 && !BL) {
                    if (solve) {
#pragma unroll
                        for (int c = 0; c < NRC; ++c) {
                            uint4 w;
                            __builtin_memcpy(&w, &b[s][c * CH], 16);
                            rowbuf[grp][NBC + c] = w;
                        }
                    }
                }
            }
        }
        // a2: lazy interchange of positions j and piv_pos
#pragma unroll
        for (int s = 0; s < RPL; ++s)
            pos[s] = (pos[s] == piv_pos) ? j : (pos[s] == j ? piv_pos : pos[s]);

        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // the pivot row: held whole in registers, or (when registers are
        // budgeted for two wavefronts per SIMD) read a chunk at a time where
        // the update consumes it
        constexpr bool chunked = reg_chunked<T, NB>();
        T u[NB];
        T ub[NRP];
        if constexpr (!chunked) {
#pragma unroll
            for (int c = 0; c < NBC; ++c) {
                if (c < j / CH) continue;
                uint4 w = rowbuf[grp][c];
                __builtin_memcpy(&u[c * CH], &w, 16);
            }
            if constexpr (NRC > 0) {
                if (solve) {
#pragma unroll
                    for (int c = 0; c < NRC; ++c) {
                        uint4 w = rowbuf[grp][NBC + c];
                        __builtin_memcpy(&ub[c * CH], &w, 16);
                    }
                }
            }
        } else {
            uint4 w = rowbuf[grp][j / CH];
            __builtin_memcpy(&u[(j / CH) * CH], &w, 16);
        }

        const T piv = (LPM == 64) ? piv_early : u[j];
        const R pm = O::metric(piv);
        const bool zero = (pm == R(0));
        if (zero && info == 0) info = j + 1;
        const T r = O::recip(piv);
        const bool small = !(pm >= O::sfmin());
        if constexpr (NR > 0) {
            if (solve && li == 0) {
                diag[2 * j] = r;
                diag[2 * j + 1] = piv;
            }
        }

        // a3: multipliers l = a * r; a pivot below the smallest normal takes
        // l = a / pivot instead.  That path is rare and sits behind a
        // wavefront-uniform branch (the empty asm keeps the compiler from
        // executing the divisions speculatively on every step).
        T lm[RPL];
#pragma unroll
        for (int s = 0; s < RPL; ++s) lm[s] = O::mul(a[s][j], r);
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(small) != 0, 0)) {
            asm volatile("" ::: "memory");
#pragma unroll
            for (int s = 0; s < RPL; ++s)
                if (small) lm[s] = O::div(a[s][j], piv);
        }

        // a4: rank-1 update of the rows below position j
#pragma unroll
        for (int s = 0; s < RPL; ++s) {
            if (pos[s] > j && !zero) {
                const T l = lm[s];
                a[s][j] = l;
                if constexpr (!chunked) {
#pragma unroll
                    for (int k = 0; k < NB; ++k)
                        if (k > j) O::fms(a[s][k], l, u[k]);
                    if constexpr (NR > 0) {
                        if (solve) {
#pragma unroll
                            for (int r2 = 0; r2 < NR; ++r2) O::fms(b[s][r2], l, ub[r2]);
                        }
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < NBC; ++c) {
                        if (c < j / CH) continue;
                        T uc[CH];
                        uint4 w = rowbuf[grp][c];
                        __builtin_memcpy(uc, &w, 16);
#pragma unroll
                        for (int e = 0; e < CH; ++e)
                            if (c * CH + e > j) O::fms(a[s][c * CH + e], l, uc[e]);
                    }
                    if constexpr (BL) {
                        if (solve) {
                            // the pivot row's right-hand sides straight from
                            // its owner's LDS row; this lane's own row updated
                            // in place
                            const uint4* const urow = &bst[(grp * NB + owner) * NRC];
                            uint4* const brow = &bst[(grp * NB + li) * NRC];
                            // a chunk at a time (unrolled, the reads would all
                            // be hoisted and hold registers the factor needs)
#pragma unroll 1
                            for (int c = 0; c < NRC; ++c) {
                                T uc[CH], bc[CH];
                                uint4 w = urow[c];
                                __builtin_memcpy(uc, &w, 16);
                                uint4 v = brow[c];
                                __builtin_memcpy(bc, &v, 16);
#pragma unroll
                                for (int e = 0; e < CH; ++e)
                                    if (c * CH + e < NR) O::fms(bc[e], l, uc[e]);
                                __builtin_memcpy(&v, bc, 16);
                                brow[c] = v;
                            }
                        }
                    } else if constexpr (NR > 0) {
                        if (solve) {
#pragma unroll
                            for (int c = 0; c < NRC; ++c) {
                                T uc[CH];
                                uint4 w = rowbuf[grp][NBC + c];
                                __builtin_memcpy(uc, &w, 16);
#pragma unroll
                                for (int e = 0; e < CH; ++e)
                                    if (c * CH + e < NR) O::fms(b[s][c * CH + e], l, uc[e]);
                            }
                        }
                    }
                }
            }
        }
    }

    // ---- back substitution U x = y (gesv) ---------------------------------
    // Step k: the row at position k publishes y_k; lane r of the group forms
    // x_kr = y_kr * (1/u_kk) (or y_kr / u_kk when u_kk is below the smallest
    // normal) for right-hand sides r = li, li + LPM, ..., and stages it; then
    // every row above position k reads x_k back and subtracts u_ik * x_k.
    // Each x_kr is formed once instead of in every lane of the group.
    if constexpr (BL) {
        // y_k is already in the LDS row of the lane at position k: lane r
        // forms x_kr there in place; after a wavefront sync the rows above
        // read x_k and update their own LDS rows
        if (solve) {
#pragma unroll
            for (int k = NB - 1; k >= 0; --k) {
                if (k >= n) continue;
                const int own = __builtin_ctzll(__builtin_amdgcn_ballot_w64(pos[0] == k));
                T* const xrow = reinterpret_cast<T*>(&bst[(grp * NB + own) * NRC]);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                {
                    const T rk = diag[2 * k];
                    const T dk = diag[2 * k + 1];
                    const bool tiny = !(O::metric(dk) >= O::sfmin());
                    if (li < NR) {
                        const T y = xrow[li];
                        T x = O::mul(y, rk);
                        if (__builtin_expect(__builtin_amdgcn_ballot_w64(tiny) != 0, 0)) {
                            asm volatile("" ::: "memory");
                            if (tiny) x = O::div(y, dk);
                        }
                        xrow[li] = x;
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                if (pos[0] < k) {
                    const uint4* const xr4 = &bst[(grp * NB + own) * NRC];
                    uint4* const brow = &bst[(grp * NB + li) * NRC];
#pragma unroll 1
                    for (int c = 0; c < NRC; ++c) {
                        T xc[CH], bc[CH];
                        uint4 w = xr4[c];
                        __builtin_memcpy(xc, &w, 16);
                        uint4 v = brow[c];
                        __builtin_memcpy(bc, &v, 16);
#pragma unroll
                        for (int e = 0; e < CH; ++e)
                            if (c * CH + e < NR) O::fms(bc[e], a[0][k], xc[e]);
                        __builtin_memcpy(&v, bc, 16);
                        brow[c] = v;
                    }
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    } else if constexpr (NR > 0) {
        if (solve) {
            const T* const ybuf = reinterpret_cast<const T*>(&rowbuf[grp][0]);
#pragma unroll
            for (int k = NB - 1; k >= 0; --k) {
                if (k >= n) continue;
#pragma unroll
                for (int s = 0; s < RPL; ++s) {
                    if (pos[s] == k) {
#pragma unroll
                        for (int c = 0; c < NRC; ++c) {
                            uint4 w;
                            __builtin_memcpy(&w, &b[s][c * CH], 16);
                            rowbuf[grp][c] = w;
                        }
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                {
                    const T rk = diag[2 * k];
                    const T dk = diag[2 * k + 1];
                    const bool tiny = !(O::metric(dk) >= O::sfmin());
                    T* const xs = reinterpret_cast<T*>(&xstage[grp][k * NRC]);
#pragma unroll
                    for (int r0 = 0; r0 < NR; r0 += LPM) {
                        const int r2 = r0 + li;
                        if (r2 < NR) {
                            const T y = ybuf[r2];
                            T x = O::mul(y, rk);
                            if (__builtin_expect(__builtin_amdgcn_ballot_w64(tiny) != 0, 0)) {
                                asm volatile("" ::: "memory");
                                if (tiny) x = O::div(y, dk);
                            }
                            xs[r2] = x;
                        }
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                T xk[NRP];
#pragma unroll
                for (int c = 0; c < NRC; ++c) {
                    uint4 w = xstage[grp][k * NRC + c];
                    __builtin_memcpy(&xk[c * CH], &w, 16);
                }
#pragma unroll
                for (int s = 0; s < RPL; ++s) {
                    if (pos[s] < k) {
#pragma unroll
                        for (int r2 = 0; r2 < NR; ++r2) O::fms(b[s][r2], a[s][k], xk[r2]);
                    }
                }
            }
        }
    }

    // ---- store -------------------------------------------------------------
    if (!live) return;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        if (k >= n) continue;
#pragma unroll
        for (int s = 0; s < RPL; ++s)
            if (pos[s] < n) A[pos[s] + (long long)k * p.lda] = a[s][k];
    }
    int* ipiv = p.ipiv + m * p.sP;
#pragma unroll
    for (int t = 0; t < NPIV; ++t) {
        const int j = t * LPM + li;
        if (j < n) ipiv[j] = pivrec[t] + 1;
    }
    if (li == 0) p.info[m] = info;
    if constexpr (BL) {
        if (solve && info == 0 && pos[0] < n) {
            // each lane stores x at the position of the row it holds
            const uint4* const brow = &bst[(grp * NB + li) * NRC];
#pragma unroll
            for (int c = 0; c < NRC; ++c) {
                T xc[CH];
                uint4 w = brow[c];
                __builtin_memcpy(xc, &w, 16);
#pragma unroll
                for (int e = 0; e < CH; ++e) {
                    const int r2 = c * CH + e;
                    if (r2 < NR && r2 < p.nrhs) B[pos[0] + (long long)r2 * p.ldb] = xc[e];
                }
            }
        }
    } else if constexpr (NR > 0) {
        if (solve && info == 0) {
            // X rows li*RPL .. li*RPL+RPL-1 from the stage
            T xr[RPL][NRP];
#pragma unroll
            for (int s = 0; s < RPL; ++s) {
                const int row = li * RPL + s;
#pragma unroll
                for (int c = 0; c < NRC; ++c) {
                    uint4 w = xstage[grp][row * NRC + c];
                    __builtin_memcpy(&xr[s][c * CH], &w, 16);
                }
            }
            const bool bfull = (n == NB) && (VB <= 16) && ((p.ldb * sizeof(T)) % VB == 0) &&
                               (((uintptr_t)B) % VB == 0);
#pragma unroll
            for (int r2 = 0; r2 < NR; ++r2) {
                if (r2 >= p.nrhs) continue;
                bool done = false;
                if constexpr (VB <= 16) {
                    using V = typename vecbits<VB>::type;
                    if (bfull) {
                        T tmp[RPL];
#pragma unroll
                        for (int s = 0; s < RPL; ++s) tmp[s] = xr[s][r2];
                        V w;
                        __builtin_memcpy(&w, tmp, sizeof(tmp));
                        *(V*)(B + li * RPL + (long long)r2 * p.ldb) = w;
                        done = true;
                    }
                }
                if (!done) {
#pragma unroll
                    for (int s = 0; s < RPL; ++s) {
                        const int row = li * RPL + s;
                        if (row < n) B[row + (long long)r2 * p.ldb] = xr[s][r2];
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// instantiation table
// ---------------------------------------------------------------------------
struct Shape {
    int nb, rpl;
};

// Partition per data type and row bucket: lanes per matrix = nb / rpl.
// Several matrices per wavefront ("tiny") up to n = 32; one wavefront per
// matrix for n in (32, 64] ("cta").
inline Shape pick_shape(int dtype, int n) {
    int nb = n <= 4 ? 4 : n <= 8 ? 8 : n <= 16 ? 16 : n <= 32 ? 32 : 64;
    int rpl;
    switch (dtype) {
    case R32: rpl = nb <= 8 ? 4 : 1; break;
    case R64: rpl = nb <= 16 ? 2 : 1; break;
    case C64: rpl = nb <= 16 ? 2 : 1; break;
    default: rpl = 1; break;
    }
    return Shape{nb, rpl};
}

inline int pick_nr(int nrhs, int mode) {
    if (mode != MODE_GESV) return 0;
    return nrhs <= 1 ? 1 : nrhs <= 8 ? 8 : nrhs <= 16 ? 16 : -1;
}

template <typename T, int NB, int RPL, int NR>
hipError_t launch_one(const Problem& p, int mode, hipStream_t s) {
    constexpr int LPM = NB / RPL;
    constexpr int GPB = (64 / LPM) * kWavesPerBlock;
    const long long blocks = (p.batch + GPB - 1) / GPB;
    hipLaunchKernelGGL((register_lu_kernel<T, NB, RPL, NR>), dim3((unsigned)blocks),
                       dim3(64 * kWavesPerBlock), 0, s, p, mode);
    return hipGetLastError();
}

template <typename T, int NB, int RPL>
hipError_t launch_nr(const Problem& p, int mode, int nr, hipStream_t s) {
    switch (nr) {
    case 0: return launch_one<T, NB, RPL, 0>(p, mode, s);
    case 1: return launch_one<T, NB, RPL, 1>(p, mode, s);
    case 8: return launch_one<T, NB, RPL, 8>(p, mode, s);
    case 16: return launch_one<T, NB, RPL, 16>(p, mode, s);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_type(const Problem& p, int mode, hipStream_t s) {
    constexpr int dtype = sizeof(T) == 4 ? R32 : sizeof(T) == 16 ? C128 : (ops<T>::is_complex ? C64 : R64);
    Shape sh = pick_shape(dtype, p.n);
    const int nr = pick_nr(p.nrhs, mode);
    constexpr bool big = sizeof(T) == 16;
#define BATCHLU_CASE(NBV, RPLV)                                                  \
    if (sh.nb == NBV && sh.rpl == RPLV) return launch_nr<T, NBV, RPLV>(p, mode, nr, s);
    if constexpr (sizeof(T) == 4) {
        // orders 9..32 of float go to the 16-lane-row kernel (register_lu_row16.h)
        BATCHLU_CASE(4, 4) BATCHLU_CASE(8, 4) BATCHLU_CASE(64, 1)
    } else if constexpr (!big) {
        BATCHLU_CASE(4, 2) BATCHLU_CASE(8, 2) BATCHLU_CASE(16, 2) BATCHLU_CASE(32, 1)
        BATCHLU_CASE(64, 1)
    } else {
        BATCHLU_CASE(4, 1) BATCHLU_CASE(8, 1) BATCHLU_CASE(16, 1) BATCHLU_CASE(32, 1)
    }
#undef BATCHLU_CASE
    return hipErrorInvalidValue;
}

}  // namespace reg_detail

}  // namespace batchlu
