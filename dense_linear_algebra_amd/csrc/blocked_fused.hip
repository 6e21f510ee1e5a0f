// blocked_fused.hip -- blocked right-looking LU (panel width 32) of a real
// matrix of order n <= 256 in ONE work-group: panel, right interchange, U12
// solve, MFMA trailing update and the deferred left interchange run as phases
// of a single kernel, so a matrix stays in the caches of its compute unit
// between panels instead of streaming the whole batch through HBM once per
// launch.
//
// BatchLAS "LU" page, blocked-getrf, register-panel and row-interchange
// paragraphs (the same steps and order as the multi-launch blocked tier):
//   panel   one row per thread in VGPRs, lazy relabel; per column ONE
//           work-group barrier: every wavefront finds its argmax (DPP inside
//           rows of 16, readlane across rows, ballot for the winning lane)
//           and publishes key, position and candidate row to a
//           double-buffered LDS slot; every thread then reads the four
//           slots in one round trip and picks the winner;
//   right   the panel's transpositions reach the trailing columns as one
//           gather of the new top rows into an LDS stage; a displaced row is
//           read by the update from the old top row that moves there (the
//           update writes every trailing row anyway), and U12 replaces the
//           top rows only after the update has read them;
//   U12     one thread per trailing column solves in the LDS stage,
//           ascending m, L11 from LDS; the stage then feeds the update and
//           is written back down each column;
//   update  A22 -= L21 U12 on v_mfma_{f32,f64}_16x16x4 chained in ascending
//           k (each MFMA accumulates like four fused multiply-adds in k
//           order, whichever operand is which), L21 negated; K = 32 always,
//           since only the last panel can be narrower and it has no trailing
//           matrix;
//   left    after the last panel, each earlier panel's L columns are gathered
//           through the composition of the later interchanges.
// A zero pivot skips its scaling and its rank-1 update everywhere (U12 solve
// and trailing update included); the update then runs on the VALU with that
// k left out, so signed zeros and infinities behave as in the unblocked order.
#include <type_traits>

#include "device_ops.h"
#include "internal.h"

namespace batchlu {

namespace {

constexpr int NB = 32;        // panel width
constexpr int NT = 256;       // threads per work-group = largest order
constexpr int NW = NT / 64;   // wavefronts
// LDS stage for U12: CW trailing columns at a time.  The widest trailing
// matrix at once where LDS allows; f64 budgeted for three work-groups per
// compute unit stages 112 columns (three 43 KB work-groups fit the 160 KB),
// for four 64 columns (31 KB each).
template <typename T, int WPE> struct Stage {
    static constexpr int CW = (sizeof(T) == 8 && WPE >= 4) ? 64 : (sizeof(T) == 8 && WPE >= 3) ? 112 : NT - NB;
    static constexpr int SLD = CW + 8;   // padded against bank conflicts
};

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef double f64x4_t __attribute__((ext_vector_type(4)));

// Matrix accesses go through a buffer resource over the matrix's own extent:
// 32-bit element offsets (one VGPR per address instead of two), and an
// access outside the extent reads 0 and writes nothing.
struct Buf {
    __amdgpu_buffer_rsrc_t r;
};
__device__ inline Buf make_buf(const void* base, uint32_t bytes) {
    return Buf{__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000)};
}
__device__ inline float ld(const Buf& b, float*, uint32_t e) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(b.r, (int)(e * 4u), 0, 0));
}
__device__ inline double ld(const Buf& b, double*, uint32_t e) {
    return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(b.r, (int)(e * 8u), 0, 0));
}
__device__ inline void st(const Buf& b, uint32_t e, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), b.r, (int)(e * 4u), 0, 0);
}
__device__ inline void st(const Buf& b, uint32_t e, double v) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), b.r, (int)(e * 8u), 0, 0);
}

// row inside a 16x16 MFMA output block held by (lane group lk, register r)
template <typename T>
__device__ inline int mfma_row(int lk, int r) {
    return sizeof(T) == 4 ? 4 * lk + r : lk + 4 * r;
}

// WPE: wavefronts per SIMD the registers are budgeted for (= work-groups per
// compute unit: f32 4; f64 2 with the full-width stage, 3 with the 112-column
// stage (168 VGPRs, no spill), or 4 with the 64-column stage and the pivot
// row read from LDS in the update (128 VGPRs, a 4-byte spill))
template <typename T, int WPE>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WPE)))
lu_fused_kernel(Problem p, uint32_t extent_bytes)
{
    using O = ops<T>;
    using R = typename O::R;
    using K = typename O::K;
    using V = typename std::conditional<sizeof(T) == 4, f32x4_t, f64x4_t>::type;
    T* const tag = nullptr;   // selects the element type of ld()

    __shared__ K skey[2][NW];
    __shared__ int spos[2][NW];
    __shared__ __attribute__((aligned(16))) T cand[2][NW][NB];
    __shared__ T l11[NB][NB];                // L11 transposed: l11[m][f] = l_fm
    __shared__ int sipiv[NT];                 // pivot rows, 0-based, global
    __shared__ int src_top[NB], src_low[NB], dst_low[NB];
    __shared__ int nlow;
    __shared__ int csrc[NT];                  // trailing position -> row holding it (relative to j0)
    constexpr int CW = Stage<T, WPE>::CW, SLD = Stage<T, WPE>::SLD;
    __shared__ T S[NB][SLD];                  // P A12, then U12 (rows of the panel x trailing columns)

    const int n = p.n;
    const uint32_t lda = (uint32_t)p.lda;
    const int tid0 = threadIdx.x;
    const long long mat = blockIdx.x;
    const Buf M = make_buf((T*)p.A + mat * p.sA, extent_bytes);
    auto at = [&](int i, int j) -> uint32_t { return (uint32_t)i + (uint32_t)j * lda; };

    int info = 0;
    for (int j0 = 0; j0 < n; j0 += NB) {
        // the thread index is re-materialised per panel so that no per-thread
        // address arithmetic is hoisted out of this loop and held live
        // across every phase (it would cost more registers than it saves)
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63;
        const int wave = tid >> 6;
        const int w = min(NB, n - j0);
        const int m = n - j0;                  // panel height
        // ---- panel: thread tid holds the row at panel position tid --------
        T a[NB];
        int pos = tid < m ? tid : 0x3fffffff;
#pragma unroll
        for (int c = 0; c < NB; ++c) a[c] = (tid < m && c < w) ? ld(M, tag, at(j0 + tid, j0 + c)) : O::zero();
        unsigned zmask = 0;
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) {
            if (jj >= w) continue;
            const int buf = jj & 1;
            const K key = (pos >= jj && pos < m) ? (K)pivot_key(O::metric(a[jj])) : (K)0;
            K kmax;
            int win;
            wave_argmax(key, pos, kmax, win);
            if (__builtin_expect(win < 0, 0)) {
                // no candidate row in this wavefront
                if (lane == 0) {
                    skey[buf][wave] = 0;
                    spos[buf][wave] = 0x7fffffff;
                }
            } else if (lane == win) {
                skey[buf][wave] = kmax;
                spos[buf][wave] = pos;
                // the candidate row in 16-byte pieces from the piece holding
                // column jj on (lower columns are written but never read)
                typedef T vec_t __attribute__((ext_vector_type(16 / sizeof(T))));
                constexpr int E = 16 / sizeof(T);
#pragma unroll
                for (int c = 0; c < NB; c += E) {
                    if (c + E <= jj) continue;
                    vec_t v;
#pragma unroll
                    for (int e = 0; e < E; ++e) v[e] = a[c + e];
                    *(vec_t*)&cand[buf][wave][c] = v;
                }
            }
            lds_barrier();
            // one LDS round trip: the four keys, positions and pivot values
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
                const bool take = (kv[v] > best) | ((kv[v] == best) & (pv[v] < ppos));   // no short circuit: no branch
                best = take ? kv[v] : best;
                ppos = take ? pv[v] : ppos;
                vb = take ? v : vb;
                piv = take ? cv[v] : piv;
            }
            // the pivot row is read now, through one VGPR base address and
            // immediate offsets, so that its reads overlap the reciprocal
            typedef __attribute__((address_space(3))) const T lds_t;
            uint32_t rowaddr = (uint32_t)(uintptr_t)(lds_t*)&cand[buf][vb][0];
            asm volatile("" : "+v"(rowaddr));
            lds_t* row = (lds_t*)(uintptr_t)rowaddr;
            // the pivot row in registers, except for f64 budgeted for four
            // work-groups per compute unit, which reads it from LDS in the
            // update (128 VGPRs leave no room for a second row)
            constexpr bool ROWREG = !(sizeof(T) == 8 && WPE >= 4);
            T u[ROWREG ? NB : 1];
            if constexpr (ROWREG) {
#pragma unroll
                for (int c = 0; c < NB; ++c)
                    if (c > jj) u[c] = row[c];
            }
            if (pos == ppos) sipiv[j0 + jj] = j0 + ppos;   // the pivot row's owner records it
            pos = (pos == ppos) ? jj : (pos == jj ? ppos : pos);
            const R pm = O::metric(piv);
            const bool zero = pm == R(0);
            if (__builtin_expect(zero, 0)) {
                zmask |= 1u << jj;
                if (info == 0) info = j0 + jj + 1;
            }
            const T r = O::recip(piv);
            const bool small = !(pm >= O::sfmin());
            // rows below the pivot take the update; the others keep their
            // values.  f32 selects (one select per element keeps the step a
            // single block the scheduler can interleave with the next pivot
            // search); f64 masks (a select costs two instructions there)
            const bool upd = pos > jj && pos < m && !zero;
            T l = O::mul(a[jj], r);
            if (__builtin_expect(__builtin_amdgcn_ballot_w64(small && upd) != 0, 0)) {
                asm volatile("" ::: "memory");
                if (small && upd) l = O::div(a[jj], piv);
            }
            if constexpr (sizeof(T) == 4) {
                a[jj] = upd ? l : a[jj];
#pragma unroll
                for (int c = 0; c < NB; ++c)
                    if (c > jj) {
                        T t = a[c];
                        O::fms(t, l, u[c]);
                        a[c] = upd ? t : a[c];
                    }
            } else if (upd) {
                a[jj] = l;
#pragma unroll
                for (int c = 0; c < NB; ++c)
                    if (c > jj) {
                        if constexpr (ROWREG) O::fms(a[c], l, u[c]);
                        else O::fms(a[c], l, (T)row[c]);
                    }
            }
        }
        // rows to their final positions; L11 to LDS for the U12 solve
        if (tid < m) {
#pragma unroll
            for (int c = 0; c < NB; ++c)
                if (c < w) st(M, at(j0 + pos, j0 + c), a[c]);
            if (pos < w) {   // stored transposed: a column of L11 is contiguous
#pragma unroll
                for (int c = 0; c < NB; ++c) l11[c][pos] = a[c];
            }
        }
        if (tid == 0) nlow = 0;
        lds_barrier();   // the row stores drain behind the next phases
        if (tid < w) p.ipiv[mat * p.sP + j0 + tid] = sipiv[j0 + tid] + 1;
        const int rest = n - j0 - w;
        if (rest <= 0) break;

        // ---- right interchange bookkeeping (positions relative to j0) -----
        // (a trailing matrix exists, so this panel is full: w == NB)
        if (tid < NB) {
            int sp[NB];
#pragma unroll
            for (int s2 = 0; s2 < NB; ++s2) sp[s2] = sipiv[j0 + s2] - j0;
            int x = tid;
#pragma unroll
            for (int s2 = NB - 1; s2 >= 0; --s2) x = (x == s2) ? sp[s2] : (x == sp[s2] ? s2 : x);
            src_top[tid] = x;
            const int ps = sipiv[j0 + tid] - j0;
            bool first = ps >= NB;
#pragma unroll
            for (int s2 = 0; s2 < NB; ++s2)
                if (s2 < tid && sp[s2] == ps) first = false;
            if (first) {
                int y = ps;
#pragma unroll
                for (int s2 = NB - 1; s2 >= 0; --s2) y = (y == s2) ? sp[s2] : (y == sp[s2] ? s2 : y);
                const int slot = atomicAdd(&nlow, 1);
                dst_low[slot] = ps;
                src_low[slot] = y;
            }
        }
        csrc[tid] = tid;
        lds_barrier();
        // a displaced trailing row is read by the update from the old top
        // row that moves there (the top rows are overwritten only after it)
        if (tid < nlow) csrc[dst_low[tid]] = src_low[tid];
        lds_barrier();

        // ---- trailing columns, in chunks of CW (the LDS stage) ------------
        const uint32_t Lo = at(j0 + w, j0);
        for (int c0 = 0; c0 < rest; c0 += CW) {
            const int cw = min(CW, rest - c0);
            const int cb = j0 + w + c0;          // first column of the chunk
            // ---- U12 = L11^-1 (P A12) -----------------------------------------
            // (1) the new top rows into the LDS stage, 32 lanes down each column
            for (int e0 = tid; e0 < NB * cw; e0 += NT * 8) {   // loads batched
                T v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int e = e0 + u * NT;
                    v[u] = ld(M, tag, at(j0 + src_top[e % NB], cb + (e < NB * cw ? e / NB : 0)));
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int e = e0 + u * NT;
                    if (e < NB * cw) S[e % NB][e / NB] = v[u];
                }
            }
            lds_barrier();
            // (3) one thread per column solves with L11 (ascending m)
            if (tid < cw) {
                if (zmask == 0) {
                    T x[NB];
#pragma unroll
                    for (int f = 0; f < NB; ++f) x[f] = S[f][tid];
#pragma unroll
                    for (int mm = 0; mm < NB; ++mm) {
#pragma unroll
                        for (int f = 0; f < NB; ++f)
                            if (f > mm) O::fms(x[f], l11[mm][f], x[mm]);
                        __builtin_amdgcn_sched_barrier(0);   // one column of L11 in flight at a time
                    }
#pragma unroll
                    for (int f = 0; f < NB; ++f) S[f][tid] = x[f];
                } else {
                    // a zero pivot: its column of L11 is left out (rare; in LDS)
#pragma unroll 1
                    for (int mm = 0; mm < NB; ++mm) {
                        if ((zmask >> mm) & 1u) continue;
                        const T xm = S[mm][tid];
#pragma unroll 1
                        for (int f = mm + 1; f < NB; ++f) {
                            T v = S[f][tid];
                            O::fms(v, l11[mm][f], xm);
                            S[f][tid] = v;
                        }
                    }
                }
            }
            __syncthreads();   // the stage and L21 visible to all

            // ---- A22[:, chunk] -= L21 U12[:, chunk] ------------------------
            const uint32_t Co = at(j0 + w, cb);
            if (zmask == 0) {
                // computed as C^T += U12^T (-L21)^T so that an output register
                // holds 16 consecutive rows of one column (coalesced C traffic)
                const int nb = (cw + 15) / 16;
                const int li = lane & 15, lk = lane >> 4;
                constexpr int RBP = 2;                   // row blocks per pass
                constexpr int PASSES = NT / 16 / NW / RBP;
#pragma unroll 1
                for (int pass = 0; pass < PASSES; ++pass) {
                    const int rb0 = (wave + NW * pass * RBP) * 16;
                    if (rb0 >= rest) continue;
                    T lv[RBP][NB / 4];
#pragma unroll
                    for (int t = 0; t < RBP; ++t) {
                        const int i = rb0 + NW * 16 * t + li;
#pragma unroll
                        for (int s = 0; s < NB / 4; ++s) lv[t][s] = -ld(M, tag, Lo + at(i, 4 * s + lk));
                    }
                    // C tiles of the next column block are loaded while the
                    // current one runs on the matrix cores
                    // the physical rows of this lane's two output rows (a
                    // displaced position reads its old top row)
                    int crow[RBP];
#pragma unroll
                    for (int t = 0; t < RBP; ++t) {
                        const int i = rb0 + NW * 16 * t + li;
                        crow[t] = i < rest ? csrc[w + i] : w + i;
                    }
                    const uint32_t Cr = at(j0, cb);   // row j0 of the chunk's first column
                    auto load_c = [&](int bj, V (&cc)[RBP]) {
#pragma unroll
                        for (int t = 0; t < RBP; ++t)
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                cc[t][r] = ld(M, tag, Cr + at(crow[t], bj * 16 + mfma_row<T>(lk, r)));
                    };
                    V cc[RBP];
                    load_c(0, cc);
#pragma unroll 1
                    for (int bj = 0; bj < nb; ++bj) {
                        // out-of-range rows and columns read harmless values (or
                        // 0 past the extent); they only reach outputs not stored
                        const int j = bj * 16 + li;
                        T uv[NB / 4];
#pragma unroll
                        for (int s = 0; s < NB / 4; ++s) uv[s] = S[4 * s + lk][j < SLD ? j : 0];
                        V cn[RBP];
                        load_c(bj + 1 < nb ? bj + 1 : bj, cn);
#pragma unroll
                        for (int t = 0; t < RBP; ++t) {
                            const int i = rb0 + NW * 16 * t + li;
                            if (rb0 + NW * 16 * t >= rest) continue;
                            V acc = cc[t];
#pragma unroll
                            for (int s = 0; s < NB / 4; ++s) {
                                if constexpr (sizeof(T) == 4)
                                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(uv[s], lv[t][s], acc, 0, 0, 0);
                                else
                                    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(uv[s], lv[t][s], acc, 0, 0, 0);
                            }
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int jc = bj * 16 + mfma_row<T>(lk, r);
                                if (i < rest && jc < cw) st(M, Co + at(i, jc), (T)acc[r]);
                            }
                        }
#pragma unroll
                        for (int t = 0; t < RBP; ++t) cc[t] = cn[t];
                    }
                }
            } else {
                // a zero pivot in this panel: leave its k out (rare; VALU)
#pragma unroll 1
                for (int e = tid; e < rest * cw; e += NT) {
                    const int i = e % rest, j = e / rest;
                    T c = ld(M, tag, at(j0 + csrc[w + i], cb + j));
#pragma unroll 1
                    for (int k = 0; k < NB; ++k)
                        if (!((zmask >> k) & 1u)) O::fms(c, ld(M, tag, Lo + at(i, k)), S[k][j]);
                    st(M, Co + at(i, j), c);
                }
            }
            __syncthreads();   // every update read of the old top rows is done
            // (4) U12 to the top rows, down each column
            for (int e = tid; e < NB * cw; e += NT) {
                const int f = e % NB, c = e / NB;
                st(M, at(j0 + f, cb + c), S[f][c]);
            }
            lds_barrier();   // the stage is refilled by the next chunk
        }
        __syncthreads();
    }

    // ---- deferred left interchange ------------------------------------------
    const int tid = tid0;
    const int P = (n + NB - 1) / NB;
    int map = tid;
    for (int k = P - 2; k >= 0; --k) {
        const int lo = (k + 1) * NB;
        const int hi = min(n, lo + NB);
        if (tid >= lo && tid < n)
            for (int s = hi - 1; s >= lo; --s) {
                const int ps = sipiv[s];
                map = (map == s) ? ps : (map == ps ? s : map);
            }
        const bool mv = tid >= lo && tid < n && map != tid;
        T v[NB];
        if (mv) {
#pragma unroll
            for (int c = 0; c < NB; ++c) v[c] = ld(M, tag, at(map, k * NB + c));
        }
        __syncthreads();
        if (mv) {
#pragma unroll
            for (int c = 0; c < NB; ++c) st(M, at(tid, k * NB + c), v[c]);
        }
        __syncthreads();
    }
    if (tid == 0) p.info[mat] = info;
}

}  // namespace

// bytes from a matrix's first element to one past its last
static long long extent_of(int dtype, int n, int lda) {
    return ((long long)(n - 1) * lda + n) * elem_bytes(dtype);
}

bool blocked_fused_supported(int dtype, int n, int lda) {
    return (dtype == R32 || dtype == R64) && n >= 1 && n <= NT && extent_of(dtype, n, lda) < (1ll << 31);
}

hipError_t blocked_fused_getrf(int dtype, const Problem& p, hipStream_t s) {
    if (!blocked_fused_supported(dtype, p.n, p.lda)) return hipErrorInvalidValue;
    const uint32_t ext = (uint32_t)extent_of(dtype, p.n, p.lda);
    if (dtype == R32)
        hipLaunchKernelGGL((lu_fused_kernel<float, 4>), dim3((unsigned)p.batch), dim3(NT), 0, s, p, ext);
    else if (p.batch >= 1024)
        // four work-groups per compute unit once the batch fills them:
        // measured against three, n = 96 - 256 at batch 2048 - 4096, 2 - 14 %
        // faster; against two at n = 256, batch 1024, 1.247 -> 1.148 ms
        hipLaunchKernelGGL((lu_fused_kernel<double, 4>), dim3((unsigned)p.batch), dim3(NT), 0, s, p, ext);
    else if (p.batch > 512)
        // three work-groups per unit hold up to 768 matrices at once
        hipLaunchKernelGGL((lu_fused_kernel<double, 3>), dim3((unsigned)p.batch), dim3(NT), 0, s, p, ext);
    else
        // up to two matrices per compute unit: two work-groups per unit with
        // the full-width stage (n = 256, batch 512: 0.635 ms against 0.651
        // with three and 0.742 with four)
        hipLaunchKernelGGL((lu_fused_kernel<double, 2>), dim3((unsigned)p.batch), dim3(NT), 0, s, p, ext);
    return hipGetLastError();
}

}  // namespace batchlu
