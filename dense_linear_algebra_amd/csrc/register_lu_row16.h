// register_lu_row16.h -- register-resident LU and fused gesv for float
// matrices of order 9..32, one matrix per 16-lane DPP row.
//
// Same method and per-element operation order as register_lu_kernel.h
// (lazy relabel of row positions, argmax with lowest-position ties, one fma
// per element and step), arranged so that the rank-1 update runs with every
// lane enabled:
//   - the pivot row of step j is published into a per-matrix LDS record
//     (row j: the 16-byte chunks from the one holding column j onwards, then
//     the right-hand-side chunks); each of the 16 lanes reads back one chunk;
//   - the update a_ik -= l_i u_jk takes u_jk straight from the lane holding
//     its chunk through a row_newbcast DPP operand of v_fmac_f32, so no
//     broadcast copy of the pivot row is made;
//   - rows already chosen as pivots are updated too (their multipliers are
//     meaningless, which saves the per-row exec masks): their U and
//     right-hand-side parts are taken from the record at the end, their L
//     parts are never written after they become pivots;
//   - the back substitution reads U and y from the record, one lane per
//     (matrix, right-hand-side column), with the oracle's descending order of
//     subtractions per entry; X leaves as contiguous columns.
// The pages' tiny tier publishes the pivot row through local memory (LU
// page, local-row broadcast paragraph); here the broadcast rides on DPP,
// which a 16-lane row of a wave64 supports natively, and the local copy
// doubles as the record of U.
#pragma once

#include <type_traits>

#include "device_ops.h"
#include "internal.h"

namespace batchlu {

namespace row16_detail {

constexpr int kWaves = 2;   // wavefronts per block (smaller blocks even out the end of the grid)

// row_newbcast:L broadcasts lane L of every 16-lane row to the whole row
template <int L>
__device__ inline float bcast(float v) {
    static_assert(L >= 0 && L < 16, "lane");
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + L, 0xF, 0xF,
                                                              false));
}

// d_t -= u_t(lane L) * l for the four elements of one chunk, for one or two
// rows (l0, l1).  v_fmac_f32 with a DPP source: d = (-u[lane L]) * l + d, the
// same rounding as fma(-l, u, d).  The leading s_nop gives the two wait
// states a DPP source needs after a VALU write (the compiler's hazard
// tracking does not look inside asm).
template <int L>
__device__ inline void fnma_chunk(float (&d0)[4], const float (&u)[4], float l0) {
    static_assert(L >= 0 && L < 16, "lane");
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, -%4, %8 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, -%5, %8 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, -%6, %8 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, -%7, %8 row_newbcast:%9 row_mask:0xf bank_mask:0xf"
        : "+v"(d0[0]), "+v"(d0[1]), "+v"(d0[2]), "+v"(d0[3])
        : "v"(u[0]), "v"(u[1]), "v"(u[2]), "v"(u[3]), "v"(l0), "n"(L));
}
template <int L>
__device__ inline void fnma_chunk(float (&d0)[4], float (&d1)[4], const float (&u)[4], float l0, float l1) {
    static_assert(L >= 0 && L < 16, "lane");
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, -%8, %12 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, -%9, %12 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, -%10, %12 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, -%11, %12 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, -%8, %13 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, -%9, %13 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, -%10, %13 row_newbcast:%14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, -%11, %13 row_newbcast:%14 row_mask:0xf bank_mask:0xf"
        : "+v"(d0[0]), "+v"(d0[1]), "+v"(d0[2]), "+v"(d0[3]), "+v"(d1[0]), "+v"(d1[1]), "+v"(d1[2]), "+v"(d1[3])
        : "v"(u[0]), "v"(u[1]), "v"(u[2]), "v"(u[3]), "v"(l0), "v"(l1), "n"(L));
}

// The same for elements E..3 of a chunk (the rest of the chunk holding the
// pivot column).
template <int L, int E>
__device__ inline void fnma_tail(float (&d0)[4], const float (&u)[4], float l0) {
    static_assert(L >= 0 && L < 16 && E >= 1 && E <= 3, "lane / element");
    if constexpr (E == 1) {
        asm("s_nop 1\n\t"
            "v_fmac_f32_dpp %0, -%3, %6 row_newbcast:%7 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %1, -%4, %6 row_newbcast:%7 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %2, -%5, %6 row_newbcast:%7 row_mask:0xf bank_mask:0xf"
            : "+v"(d0[1]), "+v"(d0[2]), "+v"(d0[3])
            : "v"(u[1]), "v"(u[2]), "v"(u[3]), "v"(l0), "n"(L));
    } else if constexpr (E == 2) {
        asm("s_nop 1\n\t"
            "v_fmac_f32_dpp %0, -%2, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %1, -%3, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf"
            : "+v"(d0[2]), "+v"(d0[3])
            : "v"(u[2]), "v"(u[3]), "v"(l0), "n"(L));
    } else {
        asm("s_nop 1\n\t"
            "v_fmac_f32_dpp %0, -%1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
            : "+v"(d0[3])
            : "v"(u[3]), "v"(l0), "n"(L));
    }
}
template <int L, int E>
__device__ inline void fnma_tail(float (&d0)[4], float (&d1)[4], const float (&u)[4], float l0, float l1) {
    static_assert(L >= 0 && L < 16 && E >= 1 && E <= 3, "lane / element");
    if constexpr (E == 1) {
        asm("s_nop 1\n\t"
            "v_fmac_f32_dpp %0, -%6, %9 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %1, -%7, %9 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %2, -%8, %9 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %3, -%6, %10 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %4, -%7, %10 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %5, -%8, %10 row_newbcast:%11 row_mask:0xf bank_mask:0xf"
            : "+v"(d0[1]), "+v"(d0[2]), "+v"(d0[3]), "+v"(d1[1]), "+v"(d1[2]), "+v"(d1[3])
            : "v"(u[1]), "v"(u[2]), "v"(u[3]), "v"(l0), "v"(l1), "n"(L));
    } else if constexpr (E == 2) {
        asm("s_nop 1\n\t"
            "v_fmac_f32_dpp %0, -%4, %6 row_newbcast:%8 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %1, -%5, %6 row_newbcast:%8 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %2, -%4, %7 row_newbcast:%8 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %3, -%5, %7 row_newbcast:%8 row_mask:0xf bank_mask:0xf"
            : "+v"(d0[2]), "+v"(d0[3]), "+v"(d1[2]), "+v"(d1[3])
            : "v"(u[2]), "v"(u[3]), "v"(l0), "v"(l1), "n"(L));
    } else {
        asm("s_nop 1\n\t"
            "v_fmac_f32_dpp %0, -%2, %3 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %1, -%2, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf"
            : "+v"(d0[3]), "+v"(d1[3])
            : "v"(u[3]), "v"(l0), "v"(l1), "n"(L));
    }
}

// maximum of a signed value over each 16-lane row (DPP; every source lane
// of these patterns lies inside the row)
__device__ inline int group_max16_i32(int v) {
    int o = (int)exchange32<1>((uint32_t)v, 0x80000000u);
    v = o > v ? o : v;
    o = (int)exchange32<2>((uint32_t)v, 0x80000000u);
    v = o > v ? o : v;
    o = (int)exchange32<4>((uint32_t)v, 0x80000000u);
    v = o > v ? o : v;
    o = (int)exchange32<8>((uint32_t)v, 0x80000000u);
    v = o > v ? o : v;
    return v;
}

template <int I, int N, typename F>
__device__ inline void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Record layout per matrix: row j holds chunks j/4 .. NBC-1 of its A part,
// then its NRC right-hand-side chunks.  rec_off(j) = first chunk of row j.
template <int NBC, int NRC>
__host__ __device__ constexpr int rec_off(int j) {
    int o = 0;
    for (int i = 0; i < j; ++i) o += NBC - i / 4 + NRC;
    return o;
}
template <int NBC, int NRC>
__device__ inline int rec_off_dyn(int j) {
    const int q = j >> 2, t = j & 3;
    return 4 * (q * (NBC + NRC) - (q * (q - 1)) / 2) + t * (NBC + NRC - q);
}

// the reciprocal of a pivot, the same bits wherever it is formed
__device__ inline float recip_step(float piv) {
    float r = recip_fast(piv);
    const bool ok = recip_fast_ok(__builtin_fabsf(piv));
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!ok) != 0, 0)) {
        asm volatile("" ::: "memory");
        if (!ok) r = 1.0f / piv;
    }
    return r;
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
    constexpr int RECC = rec_off<NBC, NRC>(NB);  // record chunks per matrix
    static_assert(NB == 16 || NB == 32, "row16 handles buckets 16 and 32");
    static_assert(ROWC <= 16, "a row must fit one chunk per lane");

    // published pivot rows, by position.  The four matrices of a wavefront
    // sit two chunks apart beyond their records (a record is a multiple of
    // 64 dwords), so that their owners' stores fall on different LDS banks;
    // the padding stays inside the wavefront's share so that three blocks
    // still fit one compute unit.
    constexpr int RSTRIDE = RECC + 2;
    __shared__ uint4 rec[kWaves][3 * RSTRIDE + RECC];
    __shared__ int ppos[GPB];                    // position the pivot row came from

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
#pragma unroll
    for (int s = 0; s < RPL; ++s) pos[s] = li + 16 * s;
    if (n == NB && p.lda == NB) {
#pragma unroll
        for (int k = 0; k < NB; ++k)
#pragma unroll
            for (int s = 0; s < RPL; ++s) a[s][k] = A[li + 16 * s + k * NB];
    } else if (n == NB) {
#pragma unroll
        for (int k = 0; k < NB; ++k)
#pragma unroll
            for (int s = 0; s < RPL; ++s) a[s][k] = A[li + 16 * s + (long long)k * p.lda];
    } else {
#pragma unroll
        for (int k = 0; k < NB; ++k)
#pragma unroll
            for (int s = 0; s < RPL; ++s) {
                const int row = li + 16 * s;
                float v = (row == k) ? 1.0f : 0.0f;
                if (k < n && row < n) v = A[row + (long long)k * p.lda];
                a[s][k] = v;
            }
    }
#pragma unroll
    for (int r = 0; r < NRP; ++r)
#pragma unroll
        for (int s = 0; s < RPL; ++s) {
            const int row = li + 16 * s;
            float v = 0.0f;
            if (solve && r < NR && r < p.nrhs && row < n) v = B[row + (long long)r * p.ldb];
            b[s][r] = v;
        }

    int pivrec[NB / 16];
#pragma unroll
    for (int t = 0; t < NB / 16; ++t) pivrec[t] = 0;
    float rd[NB];                 // 1/u_jj, identical in the 16 lanes of a matrix
    bool wave_zero = false;       // some matrix of the wavefront met a zero pivot
    bool wave_small = false;      // some pivot below the smallest normal
    uint4* const rbase = &rec[grp >> 2][(grp & 3) * RSTRIDE];
    int* const ppos_g = &ppos[grp];
    // lane li reads chunk li of each published row (lanes past the row read
    // its first chunk); rec_off(j) - j/4 >= 0 keeps every address in range
    const uint4* const rread = rbase + (li < ROWC ? li : 0);

    // ---- elimination ----------------------------------------------------------
    static_for<0, NB>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int J4 = j / 4;
        constexpr int RO = rec_off<NBC, NRC>(j) - J4;   // record row j, as chunk J4 + c at RO + c
        if (j >= n) return;
        // candidate keys: the bits of |a| with every NaN clamped just above
        // +inf (so NaNs tie and rank first), -1 for rows already chosen
        int key[RPL];
        int kmax = -1;
#pragma unroll
        for (int s = 0; s < RPL; ++s) {
            const uint32_t bits = __float_as_uint(a[s][j]) & 0x7fffffffu;
            // rows past n pad the bucket and are never candidates (0 * inf in
            // their updates can make them NaN, which would outrank real rows)
            const int kk = (pos[s] >= j && pos[s] < n) ? (int)(bits < 0x7f800001u ? bits : 0x7f800001u) : -1;
            key[s] = kk;
            kmax = kk > kmax ? kk : kmax;
        }
        kmax = group_max16_i32(kmax);
        // |pivot| is the winning key (a NaN for the clamped key): the
        // reciprocal of the magnitude starts here, off the LDS round trip;
        // the sign arrives with the published row (1/(-x) = -(1/x) exactly)
        const float pm = __uint_as_float((uint32_t)kmax);
        const bool zero = pm == 0.0f;
        const bool small = !(pm >= O::sfmin());
        const float rabs = recip_step(pm);
        // one maximal row per matrix (the usual case) needs no position
        // reduction; otherwise the lowest position among the maximal wins.
        // Ownership stays in scalar lane masks.
        uint64_t om[RPL];
        uint64_t hits = 0, both = ~0ull;
#pragma unroll
        for (int s = 0; s < RPL; ++s) {
            om[s] = __builtin_amdgcn_ballot_w64(key[s] == kmax);
            hits |= om[s];
            both &= om[s];
        }
        const bool unique = __builtin_popcountll(hits) == 4 && (RPL == 1 || both == 0);
        if (__builtin_expect(!unique, 0)) {
            int q = 0x7fffffff;
#pragma unroll
            for (int s = 0; s < RPL; ++s)
                if (key[s] == kmax && pos[s] < q) q = pos[s];
            const int pp = group_min<16>(q);
#pragma unroll
            for (int s = 0; s < RPL; ++s) om[s] = __builtin_amdgcn_ballot_w64(pos[s] == pp);
        }
        bool own[RPL];
#pragma unroll
        for (int s = 0; s < RPL; ++s) own[s] = __builtin_amdgcn_inverse_ballot_w64(om[s]);

        // the owner publishes its row (A chunks from the one holding column
        // j, then B) and where it came from.  The row is first selected from
        // the owner's slot into fresh registers, which the compiler places as
        // aligned quads: one 16-byte store per chunk from one exec region
        // (LDS instructions, not bytes, are what the LDS pipe pays for).
        {
            bool anyown = own[0];
            int opos = pos[0];
            float t[NB + 4 * NRC];
#pragma unroll
            for (int k = 4 * J4; k < NB; ++k) t[k] = a[0][k];
#pragma unroll
            for (int r2 = 0; r2 < 4 * NRC; ++r2) t[NB + r2] = b[0][r2];
            if constexpr (RPL == 2) {
                anyown = own[0] || own[1];
                opos = own[1] ? pos[1] : pos[0];
#pragma unroll
                for (int k = 4 * J4; k < NB; ++k) t[k] = own[1] ? a[1][k] : t[k];
#pragma unroll
                for (int r2 = 0; r2 < 4 * NRC; ++r2) t[NB + r2] = own[1] ? b[1][r2] : t[NB + r2];
            }
            if (anyown) {
#pragma unroll
                for (int c = J4; c < ROWC; ++c)
                    rbase[RO + c] = make_uint4(__float_as_uint(t[4 * c]), __float_as_uint(t[4 * c + 1]),
                                               __float_as_uint(t[4 * c + 2]), __float_as_uint(t[4 * c + 3]));
                *ppos_g = opos;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        const uint4 chw = rread[RO];
        const int piv_pos = *ppos_g;
        const float ch[4] = {__uint_as_float(chw.x), __uint_as_float(chw.y), __uint_as_float(chw.z),
                             __uint_as_float(chw.w)};
        if (li == j % 16) pivrec[j / 16] = piv_pos;
#pragma unroll
        for (int s = 0; s < RPL; ++s) pos[s] = own[s] ? j : (pos[s] == j ? piv_pos : pos[s]);

        const float piv = bcast<J4>(ch[j % 4]);
        wave_zero |= __builtin_amdgcn_ballot_w64(zero) != 0;
        const float r = __uint_as_float(__float_as_uint(rabs) ^ (__float_as_uint(piv) & 0x80000000u));
        rd[j] = r;
        wave_small |= __builtin_amdgcn_ballot_w64(small) != 0;
        // every row of the matrix is updated (rows already chosen get values
        // that are never used); a zero pivot skips the step for its matrix
        const bool step_small = __builtin_amdgcn_ballot_w64(small && !zero) != 0;
        if (!zero) {
            // multipliers l = a * r; a / pivot where the pivot is below the
            // smallest normal (rare: a fix-up off the straight path)
            float a0[RPL];
#pragma unroll
            for (int s = 0; s < RPL; ++s) {
                a0[s] = a[s][j];
                a[s][j] = a0[s] * r;
            }
            if (__builtin_expect(step_small, 0)) {
#pragma unroll
                for (int s = 0; s < RPL; ++s)
                    if (small) a[s][j] = a0[s] / piv;
            }
            float lm[RPL];
#pragma unroll
            for (int s = 0; s < RPL; ++s) lm[s] = a[s][j];
            // rest of the chunk holding column j
            if constexpr (j % 4 != 3) {
                if constexpr (RPL == 2) {
                    fnma_tail<J4, j % 4 + 1>(*reinterpret_cast<float(*)[4]>(&a[0][4 * J4]), *reinterpret_cast<float(*)[4]>(&a[1][4 * J4]), ch, lm[0], lm[1]);
                } else {
                    fnma_tail<J4, j % 4 + 1>(*reinterpret_cast<float(*)[4]>(&a[0][4 * J4]), ch, lm[0]);
                }
            }
            // whole chunks after it, then the right-hand sides
            static_for<J4 + 1, ROWC>([&](auto cc) {
                constexpr int c = decltype(cc)::value;
                if constexpr (c < NBC) {
                    if constexpr (RPL == 2) {
                        fnma_chunk<c>(*reinterpret_cast<float(*)[4]>(&a[0][4 * c]), *reinterpret_cast<float(*)[4]>(&a[1][4 * c]), ch, lm[0], lm[1]);
                    } else {
                        fnma_chunk<c>(*reinterpret_cast<float(*)[4]>(&a[0][4 * c]), ch, lm[0]);
                    }
                } else {
                    constexpr int cb = c - NBC;
                    if constexpr (4 * cb + 4 <= NR) {
                        if constexpr (RPL == 2) {
                            fnma_chunk<c>(*reinterpret_cast<float(*)[4]>(&b[0][4 * cb]), *reinterpret_cast<float(*)[4]>(&b[1][4 * cb]), ch, lm[0], lm[1]);
                        } else {
                            fnma_chunk<c>(*reinterpret_cast<float(*)[4]>(&b[0][4 * cb]), ch, lm[0]);
                        }
                    } else {
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            if (4 * cb + t >= NR) continue;
                            const float u = bcast<c>(ch[t]);
#pragma unroll
                            for (int s = 0; s < RPL; ++s) b[s][4 * cb + t] = __builtin_fmaf(-lm[s], u, b[s][4 * cb + t]);
                        }
                    }
                }
            });
        }
    });

    // info: the first step whose pivot is exactly zero (1-based), read back
    // from the diagonal of the record when the wavefront met one
    int info = 0;
    if (wave_zero) {
        for (int k = n - 1; k >= 0; --k) {
            const float* const dk = reinterpret_cast<const float*>(rbase + rec_off_dyn<NBC, NRC>(k)) + (k & 3);
            if (*dk == 0.0f) info = k + 1;
        }
    }

    // ---- L, U and ipiv out ------------------------------------------------------
    // Each row leaves from the lane that held it, to its final position: the
    // L part from registers, the rest (U, from the chunk holding the diagonal
    // on) from the record.  Within one column the 16 lanes of a matrix write
    // one 128-byte line.
    if (live) {
        const bool contig = n == NB && p.lda == NB;
#pragma unroll
        for (int s = 0; s < RPL; ++s) {
            const int pr = pos[s];
            const int q = pr >> 2;
            // chunk c of row pr at rrow[c] for c >= q (in range for every pr)
            const uint4* const rrow = rbase + (rec_off_dyn<NBC, NRC>(pr) - q);
            float v[NB];
#pragma unroll
            for (int c = 0; c < NBC; ++c) {
                const uint4 w = rrow[c];
                // read every chunk, then select: no per-lane branches
                asm volatile("" ::"v"(w.x), "v"(w.y), "v"(w.z), "v"(w.w));
                const bool fromrec = c >= q;
                v[4 * c] = fromrec ? __uint_as_float(w.x) : a[s][4 * c];
                v[4 * c + 1] = fromrec ? __uint_as_float(w.y) : a[s][4 * c + 1];
                v[4 * c + 2] = fromrec ? __uint_as_float(w.z) : a[s][4 * c + 2];
                v[4 * c + 3] = fromrec ? __uint_as_float(w.w) : a[s][4 * c + 3];
            }
            float* const Ar = A + pr;
            if (contig) {
#pragma unroll
                for (int k = 0; k < NB; ++k) Ar[k * NB] = v[k];
            } else if (pr < n) {
#pragma unroll
                for (int k = 0; k < NB; ++k)
                    if (k < n) Ar[(long long)k * p.lda] = v[k];
            }
        }
        int* ipiv = p.ipiv + m * p.sP;
#pragma unroll
        for (int t = 0; t < NB / 16; ++t) {
            const int j = t * 16 + li;
            if (j < n) ipiv[j] = pivrec[t] + 1;
        }
        if (li == 0) p.info[m] = info;
    }

    // ---- back substitution from the record: lane li solves column li ---------
    if constexpr (NR > 0) {
        if (solve) {
            const int rc = li < NR ? li : NR - 1;
            const float* const yb = reinterpret_cast<const float*>(rbase) + rc;
            float x[NB];
            const bool fast = n == NB && !wave_small;
            if (fast) {
                // U row k is read one row ahead into a second register set;
                // each dot product runs as four partial sums (one per element
                // of a chunk), so the chains stay short
                uint4 ub[2][NBC];
                float yv[2];
                auto load_row = [&](auto kc, auto bc) {
                    constexpr int k = decltype(kc)::value;
                    constexpr int bsel = decltype(bc)::value;
                    constexpr int RO = rec_off<NBC, NRC>(k) - k / 4;
#pragma unroll
                    for (int c = k / 4; c < NBC; ++c) ub[bsel][c] = rbase[RO + c];
                    yv[bsel] = yb[4 * (RO + NBC)];
                };
                load_row(std::integral_constant<int, NB - 1>{}, std::integral_constant<int, (NB - 1) & 1>{});
                static_for<0, NB>([&](auto ic) {
                    constexpr int k = NB - 1 - decltype(ic)::value;
                    constexpr int bsel = k & 1;
                    if constexpr (k > 0)
                        load_row(std::integral_constant<int, k - 1>{}, std::integral_constant<int, (k - 1) & 1>{});
                    float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int c = NBC - 1; c >= k / 4; --c) {
                        const float u[4] = {__uint_as_float(ub[bsel][c].x), __uint_as_float(ub[bsel][c].y),
                                            __uint_as_float(ub[bsel][c].z), __uint_as_float(ub[bsel][c].w)};
#pragma unroll
                        for (int t = 3; t >= 0; --t)
                            if (4 * c + t > k) ps[t] = __builtin_fmaf(u[t], x[4 * c + t], ps[t]);
                    }
                    x[k] = (yv[bsel] - ((ps[0] + ps[1]) + (ps[2] + ps[3]))) * rd[k];
                });
            } else {
                static_for<0, NB>([&](auto ic) {
                    constexpr int k = NB - 1 - decltype(ic)::value;
                    constexpr int RO = rec_off<NBC, NRC>(k) - k / 4;
                    if (k < n) {
                        float acc = yb[4 * (RO + NBC)];
#pragma unroll
                        for (int c = NBC - 1; c >= k / 4; --c) {
                            const uint4 w = rbase[RO + c];
                            const float u[4] = {__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z),
                                                __uint_as_float(w.w)};
#pragma unroll
                            for (int t = 3; t >= 0; --t)
                                if (4 * c + t > k && 4 * c + t < n) acc = __builtin_fmaf(-u[t], x[4 * c + t], acc);
                        }
                        const uint4 w = rbase[RO + k / 4];
                        const float u[4] = {__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z),
                                            __uint_as_float(w.w)};
                        if (!(__builtin_fabsf(u[k % 4]) >= O::sfmin()))
                            x[k] = acc / u[k % 4];
                        else
                            x[k] = acc * rd[k];
                    } else {
                        x[k] = 0.0f;
                    }
                });
            }
            if (live && info == 0 && li < NR && li < p.nrhs) {
                float* const Xc = B + (long long)li * p.ldb;
                if (n == NB && (((uintptr_t)Xc) % 16) == 0) {
#pragma unroll
                    for (int c = 0; c < NBC; ++c)
                        *reinterpret_cast<float4*>(Xc + 4 * c) = make_float4(x[4 * c], x[4 * c + 1], x[4 * c + 2],
                                                                             x[4 * c + 3]);
                } else {
#pragma unroll
                    for (int k = 0; k < NB; ++k)
                        if (k < n) Xc[k] = x[k];
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
