// fold.hip -- the damped, equilibrated GPTQ fold on gfx950.
//
// Source of the method: page "cortiq-engine 0.8.41 src/gpu_wgpu/gptq_dev.rs" (module
// documentation steps 1-4; kernels diag_get, build_a, chol_*, inv_*, make_u; driver fold) and
// page "cortiq-cli 0.8.45 src/gptq.rs" (gptq_fold_operator_par: dead channels, damping by
// lambda * mean(diag), the x10 retry, U = upper Cholesky factor of H_d^-1).
//
// Device layout (workspace, caller-owned): n_p = n rounded up to NB = 128.
//   state  FoldState (base, pivot flag, dead count)
//   dinv   [n_p] f32: (H_ii + damp)^-1/2, dead: (1 + damp)^-1/2, indexed by channel
//   MI     [n_p/NB][NB][NB] f32: inverses of the diagonal blocks of L
//   A      [n_p][n_p] f32: reversed equilibrated H_d, then L (lower) in place
//   X      [n_p][n_p] f32: L^-1 (lower), built block row by block row
// The padding rows/columns n..n_p-1 of A are the identity, so L and L^-1 carry an identity
// tail and every tile, panel and K-chunk is full.
//
// Blocked right-looking Cholesky fused with the blocked right-looking inverse, per step k:
//   diag   : L_kk = chol(A_kk), MI_k = L_kk^-1 (one workgroup, LDS resident)
//   panel  : L_ik = A_ik MI_k^T for the rows below;  X_k,<k = MI_k X_k,<k     (one GEMM launch)
//   update : A_ij -= L_ik L_jk^T (lower tiles);      X_i,<=k -= L_ik X_k,<=k
// The pages factor and invert in two separate passes; both are right-looking and the inverse
// of step k only needs L's column block k, so one pass does both.  The update is split with a
// look-ahead of one step: its next block column / block row (needed by step k+1's diag and
// panel) runs on the caller's stream, and the bulk runs on a helper stream, overlapping the
// serial diag / panel chain of the next step.
#include <math.h>
#include <string.h>

#include <utility>

#include <algorithm>
#include <vector>

#include "common.hpp"
#include "fold.hpp"
#include "gemm_mfma.hpp"

namespace gptq {

// Diagonal, dead mask, mean of the diagonal with dead channels counted as 1 (f64, fixed
// reduction order).
__global__ __launch_bounds__(1024) void fold_prep_kernel(HTab ht, int64_t n, float* __restrict__ hdiag,
                                                          uint8_t* __restrict__ dead, FoldState* st,
                                                          int64_t gs) {
    const float* __restrict__ H = ht.H[blockIdx.z];
    const HLayout hl{n, ht.ldh[blockIdx.z]};
    hdiag = gang_ptr(hdiag, gs);
    dead = gang_ptr(dead, gs);
    st = gang_ptr(st, gs);
    __shared__ double ssum[1024];
    __shared__ int scnt[1024];
    const int t = threadIdx.x;
    double s = 0.0;
    int cnt = 0;
    // Unrolled so that several of the strided diagonal loads are in flight at once (the sums
    // keep their order).
#pragma unroll 8
    for (int64_t i = t; i < n; i += 1024) {
        const float d = H[hl.at(i, i)];
        const bool dd = !(d > 0.0f);
        hdiag[i] = d;
        dead[i] = dd ? 1 : 0;
        s += dd ? 1.0 : (double)d;
        cnt += dd ? 1 : 0;
    }
    ssum[t] = s;
    scnt[t] = cnt;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
        if (t < w) {
            ssum[t] += ssum[t + w];
            scnt[t] += scnt[t + w];
        }
        __syncthreads();
    }
    if (t == 0) {
        st->base = fmax(ssum[0] / (double)n, 1e-12);
        st->n_dead = scnt[0];
        st->flag = 0u;
    }
}

// Per attempt: inverse equilibration scales and a cleared pivot flag.
__global__ void fold_scale_kernel(const float* __restrict__ hdiag, const uint8_t* __restrict__ dead,
                                  FoldState* st, double lam, int64_t n, int64_t np,
                                  float* __restrict__ dinv, int64_t gs) {
    hdiag = gang_ptr(hdiag, gs);
    dead = gang_ptr(dead, gs);
    st = gang_ptr(st, gs);
    dinv = gang_ptr(dinv, gs);
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0) {
        __atomic_store_n(&st->flag, 0u, __ATOMIC_RELAXED);
        __atomic_store_n(&st->minp32, 0x7F800000u, __ATOMIC_RELAXED);  // +inf
    }
    if (i >= np) return;
    if (i >= n) {
        dinv[i] = 1.0f;
        return;
    }
    const double damp = lam * st->base;
    const double v = dead[i] ? 1.0 + damp : (double)hdiag[i] + damp;
    dinv[i] = (float)(1.0 / sqrt(v));
}

// A[i][j] (i >= j) = reversed, damped, equilibrated H read from its upper triangle; the
// padding block is the identity; entries above the diagonal inside diagonal 64 x 64 tiles are 0.
// One workgroup per lower 64 x 64 tile (the grid enumerates only those).  VEC (dense H, n and
// ldh multiples of 4, H 16-byte aligned): each thread takes 4 adjacent columns of 4 rows, as
// float4 reads of H (4 adjacent columns of H in reverse order) and float4 writes of A;
// otherwise (also for the packed layout, whose rows start at any float) a row of the tile is
// one wave of single floats.  Both coalesce.
template <bool VEC>
__global__ __launch_bounds__(256) void fold_build_kernel(HTab ht, const float* __restrict__ dinv,
                                                         const uint8_t* __restrict__ dead,
                                                         const FoldState* st, double lam,
                                                         float* __restrict__ A, int64_t n,
                                                         int64_t np, int64_t gs) {
    const float* __restrict__ H = ht.H[blockIdx.z];
    const HLayout hl{n, ht.ldh[blockIdx.z]};
    dinv = gang_ptr(dinv, gs);
    dead = gang_ptr(dead, gs);
    st = gang_ptr(st, gs);
    A = gang_ptr(A, gs);
    const int b = blockIdx.x;
    int ti = (int)((sqrtf(8.0f * (float)b + 1.0f) - 1.0f) * 0.5f);
    while ((ti + 1) * (ti + 2) / 2 <= b) ++ti;
    while (ti * (ti + 1) / 2 > b) --ti;
    const int tj = b - ti * (ti + 1) / 2;
    const double damp = lam * st->base;
    if constexpr (VEC) {
        const int64_t j4 = (int64_t)tj * 64 + (threadIdx.x & 15) * 4;
        const bool jin = j4 < n;  // n % 4 == 0: the 4 columns are all in or all out
        const int64_t bc4 = n - 4 - j4;  // H columns bc4 .. bc4 + 3 are A's columns j4 + 3 .. j4
        f32x4 db = {0.f, 0.f, 0.f, 0.f};
        bool deadb[4] = {false, false, false, false};
        if (jin) {
            db = *reinterpret_cast<const f32x4*>(dinv + bc4);
#pragma unroll
            for (int u = 0; u < 4; ++u) deadb[u] = dead[bc4 + u] != 0;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t i = (int64_t)ti * 64 + (threadIdx.x >> 4) + 16 * q;
            f32x4 v;
            if (i >= n || !jin) {
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = (i == j4 + u) ? 1.0f : 0.0f;
            } else {
                const int64_t a = n - 1 - i;
                const bool dead_a = dead[a] != 0;
                const float da = dinv[a];
                const f32x4 h4 = *reinterpret_cast<const f32x4*>(H + hl.at(a, bc4));
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int64_t j = j4 + u, bcol = n - 1 - j;  // H column of A's column j
                    float x;
                    if (j > i) {
                        x = 0.0f;
                    } else if (dead_a || deadb[3 - u]) {
                        x = (a == bcol) ? 1.0f : 0.0f;
                    } else if (a == bcol) {
                        const double di = (double)da;
                        x = (float)(((double)h4[3 - u] + damp) * di * di);
                    } else {
                        x = h4[3 - u] * da * db[3 - u];
                    }
                    v[u] = x;
                }
            }
            *reinterpret_cast<f32x4*>(A + i * np + j4) = v;
        }
    } else {
        const int64_t j = (int64_t)tj * 64 + (threadIdx.x & 63);
        const int64_t bc = n - 1 - j;  // column of H (valid when j < n)
        const bool jin = j < n;
        const bool dead_b = jin && dead[bc];
        const float db = jin ? dinv[bc] : 0.0f;
#pragma unroll 4
        for (int q = 0; q < 16; ++q) {
            const int64_t i = (int64_t)ti * 64 + (threadIdx.x >> 6) + 4 * q;
            float v;
            if (j > i) {
                v = 0.0f;
            } else if (i >= n || !jin) {
                v = (i == j) ? 1.0f : 0.0f;
            } else {
                const int64_t a = n - 1 - i;  // a <= bc: upper triangle of H
                if (dead[a] || dead_b) {
                    v = (a == bc) ? 1.0f : 0.0f;
                } else if (a == bc) {
                    const double di = (double)db;
                    v = (float)(((double)H[hl.at(a, a)] + damp) * di * di);
                } else {
                    v = H[hl.at(a, bc)] * dinv[a] * db;
                }
            }
            A[i * np + j] = v;
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Diagonal block: L_kk = chol(A_kk) and MI_k = L_kk^-1 for the NB x NB block at k * NB, in one
// workgroup of 4 waves, LDS resident.  The block is factored as 4 sub-panels of 32 columns:
//   wave 0: 32 x 32 Cholesky of the sub-panel's diagonal block in registers (one lane per row,
//           column values broadcast with readlane) and its inverse T_p (one lane per column);
//   waves : panel rows below, L = A T_p^T, and the lower trailing blocks A -= L L^T, each a
//           32 x 32 x 32 product on v_mfma_f32_32x32x2_f32;
// then the off-diagonal blocks of L^-1 by block forward substitution down each block column,
//   M_IJ = -T_I sum_{J <= Q < I} L_IQ M_QJ   (waves 0..2 take block columns 0..2).
// A pivot that is not above tau (the accuracy floor of the "auto" precision, 0 for "f32"), or
// NaN, is replaced by 1 (if not positive) and sets flag bit 1 under "auto" (the damping is then
// factored in f64) or bit 0 under "f32" (the attempt failed).  The smallest pivot of the block,
// as the square of L's smallest diagonal entry, goes to *minp.
constexpr int DLD = NB + 1;  // row stride of the block in LDS (odd: column reads spread banks)
constexpr int SLD = 33;      // row stride of 32 x 32 blocks in LDS

__device__ __forceinline__ float lane_bcast(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// acc += A * B on one wave, 32 x 32 x 32.  A[i][k] = A[i*lda + k];
// B(k, j) = TRANS ? B[j*ldb + k] : B[k*ldb + j].  MFMA k index of lane l in step s: 2 s + l/32.
template <bool TRANS>
__device__ __forceinline__ f32x16 mm32(const float* A, int lda, const float* B, int ldb,
                                       f32x16 acc) {
    const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        const int k = 2 * s + h;
        const float a = A[l32 * lda + k];
        const float b = TRANS ? B[l32 * ldb + k] : B[k * ldb + l32];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    return acc;
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int v = 0; v < 16; ++v) z[v] = 0.0f;
    return z;
}

// Element (i, j) of a 32 x 32 MFMA result held by this lane in slot v.
__device__ __forceinline__ int mrow(int v) { return 8 * (v >> 2) + 4 * ((threadIdx.x & 63) >> 5) + (v & 3); }
__device__ __forceinline__ int mcol() { return threadIdx.x & 31; }

// Step C of the 32 x 32 leaf of the diagonal kernel (the lane layout is described there): the
// pivot x[C] of lane C is tested and turned into 1 / L_CC; x[C] *= 1 / L_CC makes L_sC final on
// lane s of the lower half (L_CC = sqrt(pivot) on lane C itself) and T_C,row final in the upper
// half, (e_row - sum_{k<C} L_Ck T_k,row) / L_CC; then every later x[s] -= x[C] L_sC, with L_sC
// broadcast from lane s.  C is a template parameter so that every loop below has a constant trip
// count and x[] stays in registers; the broadcasts go four at a time into separate scalar
// registers.  Each step's updates are pinned in place so the compiler does not defer them.
template <int C>
__device__ __forceinline__ void leaf_step(float (&x)[32], float tau, int& nbad) {
    float pv = lane_bcast(x[C], C);
    nbad += !(pv > tau) ? 1 : 0;  // not above the floor (tau = 0: not positive), or NaN
    asm volatile("" : "+v"(nbad));
    pv = (pv > 0.0f) ? pv : 1.0f;
    // rsq needs a normal input; a positive subnormal pivot takes the IEEE route (pv is uniform,
    // so this is a scalar branch off the common path).
    float rs;
    if (__builtin_expect(pv < 1.17549435e-38f, 0)) rs = 1.0f / sqrtf(pv);
    else rs = __builtin_amdgcn_rsqf(pv);
    x[C] *= rs;
#pragma unroll
    for (int s0 = (C + 1) & ~3; s0 < 32; s0 += 4) {
        float L[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (s0 + u > C) L[u] = lane_bcast(x[C], s0 + u);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (s0 + u > C) x[s0 + u] -= x[C] * L[u];
    }
#pragma unroll
    for (int s2 = C + 1; s2 < 32; ++s2) asm volatile("" : "+v"(x[s2]));
}

template <int... C>
__device__ __forceinline__ void leaf_steps(float (&x)[32], float tau, int& nbad,
                                           std::integer_sequence<int, C...>) {
    (leaf_step<C>(x, tau, nbad), ...);
}

__global__ __launch_bounds__(256) void fold_diag_kernel(float* __restrict__ A, float* __restrict__ MI,
                                                        int64_t np, int k, unsigned* flag,
                                                        unsigned* minp, float tau, int64_t gs) {
    flag = gang_ptr(flag, gs);
    if (__atomic_load_n(flag, __ATOMIC_RELAXED)) return;
    A = gang_ptr(A, gs);
    MI = gang_ptr(MI, gs);
    minp = gang_ptr(minp, gs);
    __builtin_amdgcn_s_setprio(CHAIN_PRIO);
    // 81 KB of LDS, so that the kernel fits on a CU beside one GEMM workgroup.  The off-diagonal
    // 32-blocks M_IJ (I > J) of L^-1 live in the unused upper triangle of Ls, at block (J, I).
    __shared__ float Ls[NB * DLD];        // the block, L in place (lower)
    __shared__ float Ts[4][32 * SLD];     // T_p = inverse of L's diagonal 32-blocks
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31;
    const int64_t kb = (int64_t)k * NB;
    {
        // 16 float4 per thread, all issued before any is stored (32 threads per 128-float row).
        f32x4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = (tid >> 5) + 8 * i, c = (tid & 31) * 4;
            v[i] = *reinterpret_cast<const f32x4*>(A + (kb + r) * np + kb + c);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = (tid >> 5) + 8 * i, c = (tid & 31) * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) Ls[r * DLD + c + q] = (c + q <= r) ? v[i][q] : 0.0f;
        }
    }
    __syncthreads();
    bool bad = false;
    float pmin = INFINITY;  // lanes 0..31 of wave 0: the smallest L_cc^2 of their rows
    for (int p = 0; p < 4; ++p) {
        const int c0 = 32 * p;
        if (wave == 0) {
            // Factor and invert together: lane r holds row r of the 32 x 32 block (a) and lane
            // r + 32 column r of its inverse T = L^-1 (t), both in x[].  Step c makes column c
            // of L final; its entries L_sc (s > c), broadcast from the lower half, drive the
            // same update x[s] -= x[c] L_sc in both halves: the right-looking Cholesky update of
            // the later columns of a, and the right-looking substitution step c of every column
            // of T.  An opaque copy of the row index keeps comparisons against it inside the
            // sub-panel (instead of hoisted out of the loop and spilled).
            int row = l32;
            asm volatile("" : "+v"(row));
            const bool tpart = lane >= 32;
            float x[32];
#pragma unroll
            for (int c = 0; c < 32; ++c) {
                const float av = Ls[(c0 + row) * DLD + c0 + c];
                x[c] = tpart ? ((c == row) ? 1.0f : 0.0f) : av;
            }
            int nbad = 0;
            leaf_steps(x, tau, nbad, std::make_integer_sequence<int, 32>{});
            if (!tpart) {
#pragma unroll
                for (int c = 0; c < 32; ++c) Ls[(c0 + row) * DLD + c0 + c] = (c <= row) ? x[c] : 0.0f;
                const float lcc = Ls[(c0 + row) * DLD + c0 + row];  // written by this lane
                pmin = fminf(pmin, lcc * lcc);
            } else {
#pragma unroll
                for (int c = 0; c < 32; ++c) Ts[p][c * SLD + row] = x[c];
            }
            bad = bad || nbad != 0;
        }
        __syncthreads();
        // Panel: rows below, L_rb = A_rb T_p^T.
        if (wave < 3 - p) {
            const int r0 = c0 + 32 * (wave + 1);
            f32x16 acc = mm32<true>(&Ls[r0 * DLD + c0], DLD, Ts[p], SLD, zero16());
#pragma unroll
            for (int v = 0; v < 16; ++v) Ls[(r0 + mrow(v)) * DLD + c0 + mcol()] = acc[v];
        }
        __syncthreads();
        // Trailing lower 32-blocks (rb >= cb > p): A_rb,cb -= L_rb,p L_cb,p^T.
        int item = 0;
        for (int rb = p + 1; rb < 4; ++rb)
            for (int cb = p + 1; cb <= rb; ++cb, ++item) {
                if ((item & 3) != wave) continue;
                f32x16 acc = mm32<true>(&Ls[32 * rb * DLD + c0], DLD, &Ls[32 * cb * DLD + c0], DLD,
                                        zero16());
#pragma unroll
                for (int v = 0; v < 16; ++v) Ls[(32 * rb + mrow(v)) * DLD + 32 * cb + mcol()] -= acc[v];
            }
        __syncthreads();
    }
    // Off-diagonal blocks of L^-1, block column J = wave: M_IJ = -T_I sum_{J<=Q<I} L_IQ M_QJ,
    // each kept at block (J, I) of Ls (the partial sum is staged in the same place).
    if (wave < 3) {
        const int J = wave;
        for (int I = J + 1; I < 4; ++I) {
            f32x16 acc = zero16();
            for (int Q = J; Q < I; ++Q) {
                const float* m = (Q == J) ? Ts[J] : &Ls[32 * J * DLD + 32 * Q];
                const int ldm = (Q == J) ? SLD : DLD;
                acc = mm32<false>(&Ls[32 * I * DLD + 32 * Q], DLD, m, ldm, acc);
            }
            float* slot = &Ls[32 * J * DLD + 32 * I];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int v = 0; v < 16; ++v) slot[mrow(v) * DLD + mcol()] = acc[v];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            f32x16 m2 = mm32<false>(Ts[I], SLD, slot, DLD, zero16());
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int v = 0; v < 16; ++v) slot[mrow(v) * DLD + mcol()] = -m2[v];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
    if (wave == 0) {
        // The smallest pivot of the block, as the square of L's smallest diagonal entry.
#pragma unroll
        for (int off = 16; off > 0; off >>= 1) pmin = fminf(pmin, __shfl_xor(pmin, off, 32));
        if (lane == 0) {
            if (bad) atomicOr(flag, tau > 0.0f ? 2u : 1u);
            atomicMin(minp, __float_as_uint(pmin));
        }
    }
    __syncthreads();
    // Output: MI_k as float4 rows (zeros above the diagonal).  Nothing reads L's diagonal block
    // after this kernel (the panel solve multiplies by MI_k), so it is not stored; the inverse's
    // diagonal blocks are copied from MI on the inverse's own stream.
    float* mi = MI + (int64_t)k * NB * NB;
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
        const int r = (tid >> 5) + 8 * i, c = (tid & 31) * 4;
        const int I = r >> 5, J = c >> 5;  // the four columns share one 32-block
        f32x4 m4;
        if (I == J) {
#pragma unroll
            for (int q = 0; q < 4; ++q) m4[q] = Ts[I][(r & 31) * SLD + ((c + q) & 31)];
        } else if (I > J) {
#pragma unroll
            for (int q = 0; q < 4; ++q) m4[q] = Ls[(32 * J + (r & 31)) * DLD + 32 * I + ((c + q) & 31)];
        } else {
            m4 = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        *reinterpret_cast<f32x4*>(mi + r * NB + c) = m4;
    }
}

// U[j][c] = X[n-1-j][n-1-c] * dinv[c] for c >= j, 0 below the diagonal, for the rows
// j0 <= j < j1 of U.  One workgroup per 64 x 64 tile of those rows; tiles wholly below the
// diagonal only store 0.  VEC (n a multiple of 4, U 16-byte aligned): each thread takes 4
// adjacent columns of 4 rows, float4 reads of X (4 adjacent columns in reverse order) and
// float4 writes of U; otherwise a row of the tile per wave, single floats.
template <bool VEC>
__global__ __launch_bounds__(256) void fold_make_u_kernel(const float* __restrict__ X,
                                                          const float* __restrict__ dinv,
                                                          float* __restrict__ U, int64_t n,
                                                          int64_t np, int64_t j0, int64_t j1,
                                                          int64_t gs) {
    X = gang_ptr(X, gs);
    dinv = gang_ptr(dinv, gs);
    U = gang_ptr(U, gs);
    const int64_t jt = j0 + (int64_t)blockIdx.y * 64;  // the tile's first row of U
    const bool below = (int64_t)blockIdx.x * 64 + 63 < jt;  // every column left of every row
    if constexpr (VEC) {
        const int64_t c4 = (int64_t)blockIdx.x * 64 + (threadIdx.x & 15) * 4;
        if (c4 >= n) return;  // n % 4 == 0: the 4 columns are all in or all out
        const f32x4 d4 = below ? f32x4{0.f, 0.f, 0.f, 0.f} : *reinterpret_cast<const f32x4*>(dinv + c4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t j = jt + (threadIdx.x >> 4) + 16 * q;
            if (j >= j1) continue;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (!below && c4 + 3 >= j) {
                // X[n-1-j][n-4-c4 .. n-1-c4] holds the columns c4 + 3 .. c4 of U's row j.
                const f32x4 x4 = *reinterpret_cast<const f32x4*>(X + (n - 1 - j) * np + (n - 4 - c4));
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = (c4 + u >= j) ? x4[3 - u] * d4[u] : 0.0f;
            }
            *reinterpret_cast<f32x4*>(U + j * n + c4) = v;
        }
    } else {
        const int64_t c = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
        const float dc = (!below && c < n) ? dinv[c] : 0.0f;
#pragma unroll 4
        for (int q = 0; q < 16; ++q) {
            const int64_t j = jt + (threadIdx.x >> 6) + 4 * q;
            if (j >= j1 || c >= n) continue;
            U[j * n + c] = (!below && c >= j) ? X[(n - 1 - j) * np + (n - 1 - c)] * dc : 0.0f;
        }
    }
}

__global__ __launch_bounds__(256) void fold_identity_kernel(float* __restrict__ U, int64_t n) {
    for (int e = threadIdx.x; e < 32 * 32; e += 256) {
        const int64_t j = (int64_t)blockIdx.y * 32 + (e >> 5);
        const int64_t c = (int64_t)blockIdx.x * 32 + (e & 31);
        if (j < n && c < n) U[j * n + c] = (j == c) ? 1.0f : 0.0f;
    }
}

// The w x w diagonal block of X at kb before its block forward substitution: the diagonal
// 128-blocks are the inverses MI of L's diagonal blocks, the blocks above are 0 (the blocks
// below are written by the substitution).
__global__ __launch_bounds__(256) void fold_x_diag_kernel(float* __restrict__ X,
                                                          const float* __restrict__ MI,
                                                          int64_t np, int64_t kb, int64_t w,
                                                          int64_t gs) {
    X = gang_ptr(X, gs);
    MI = gang_ptr(MI, gs);
    const int64_t r = blockIdx.y;                // row within the block
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= w) return;
    const int64_t I = r / NB, J = c / NB;
    if (J > I) X[(kb + r) * np + kb + c] = 0.0f;
    else if (J == I) X[(kb + r) * np + kb + c] = MI[((kb / NB + I) * NB + (r % NB)) * NB + (c % NB)];
}

__global__ __launch_bounds__(256) void fold_copy_rows_kernel(const float* __restrict__ src,
                                                             float* __restrict__ dst, int64_t ld,
                                                             int64_t cols, int64_t gs) {
    src = gang_ptr(src, gs);
    dst = gang_ptr(dst, gs);
    const int64_t r = blockIdx.y;
    for (int64_t c = (int64_t)blockIdx.x * 1024 + threadIdx.x * 4; c < cols;
         c += (int64_t)gridDim.x * 1024) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(src + r * ld + c);
        *reinterpret_cast<f32x4*>(dst + r * ld + c) = v;
    }
}

}  // namespace gptq

using namespace gptq;

// The "auto" precision's accuracy floor on the f32 pivots.  The pivots are those of the
// unit-diagonal equilibrated matrix; the f32 factor's error in U D grows as u32 / (smallest
// pivot), so an attempt whose smallest pivot is at or below this floor is repeated in f64.
static constexpr float kF32PivotFloor = 1.0e-2f;

extern "C" size_t gptq_fold_workspace_size_ex(int64_t n, int precision) {
    if (n <= 0 || n > ((int64_t)1 << 20)) return 0;
    if (precision != GPTQ_FOLD_AUTO && precision != GPTQ_FOLD_F32 && precision != GPTQ_FOLD_F64) return 0;
    const FoldLayout L = fold_layout(n);
    return precision == GPTQ_FOLD_F32 ? L.total_f32 : L.total;
}

extern "C" size_t gptq_fold_workspace_size(int64_t n) {
    return gptq_fold_workspace_size_ex(n, GPTQ_FOLD_AUTO);
}

extern "C" int gptq_fold(const float* H, int64_t n, int64_t ldh, double lambda, float* U,
                         float* hdiag, uint8_t* dead, void* workspace, size_t workspace_bytes,
                         void* stream, gptq_fold_report* report) {
    return gptq_fold_ex(H, n, ldh, lambda, GPTQ_FOLD_AUTO, U, hdiag, dead, workspace,
                        workspace_bytes, stream, report);
}

extern "C" int gptq_fold_ex(const float* H, int64_t n, int64_t ldh, double lambda, int precision,
                            float* U, float* hdiag, uint8_t* dead, void* workspace,
                            size_t workspace_bytes, void* stream, gptq_fold_report* report) {
    return fold_run(H, n, ldh, lambda, precision, U, hdiag, dead, workspace, workspace_bytes,
                    (hipStream_t)stream, report, false);
}

namespace gptq {

namespace {

// check_launch over spans listed at run time, then the launch.
template <class F>
int launch_with(hipStream_t s, const char* name, const std::vector<Span>& acc, F&& f) {
    const int rc = check_launch(name, s, acc.data(), (int)acc.size());
    if (rc != GPTQ_OK) return rc;
    if (!dry_run()) f();
    return GPTQ_OK;
}

// The Hessians of the ng groups of ht, read whole: the caller's buffers, one per group.
void push_hessians(std::vector<Span>& acc, const HTab& ht, int ng, int64_t n) {
    for (int g = 0; g < ng; ++g) acc.push_back(fixed(hessian_span(ht.H[g], n, ht.ldh[g], false)));
}

#define FOLD_OK(call)                           \
    do {                                        \
        const int rc_ = (call);                 \
        if (rc_ != GPTQ_OK) return rc_;         \
    } while (0)

// Diagonal, dead flags, base and a cleared flag for the ng groups of ht (the gang open on this
// thread, or one group).
int fold_prep(const HTab& ht, int ng, int64_t n, float* hdiag, uint8_t* dead, FoldState* state,
              hipStream_t st) {
    std::vector<Span> acc;
    push_hessians(acc, ht, ng, n);
    acc.push_back(wr(hdiag, n, 1, n));
    acc.push_back(wr(dead, n, 1, n, 1));
    acc.push_back(wr(state, 1, 1, sizeof(FoldState), 1));
    const int64_t gs = gang_current().gs;
    ProfScope ps(FAM_FOLD_BUILD, st, 0.0, 8.0 * n);
    FOLD_OK(launch_with(st, "fold_prep", acc, [&] {
        fold_prep_kernel<<<gang_grid(1), 1024, 0, st>>>(ht, n, hdiag, dead, state, gs);
    }));
    return launch_status() != GPTQ_OK ? GPTQ_EHIP : GPTQ_OK;
}

int fold32_make_u(char* ws, const FoldLayout& L, float* U, int64_t n, int64_t j0, int64_t j1,
                  hipStream_t st);
int64_t u_split(int64_t n, const FoldLayout& L);

// A bulk update's launch: 64 x 64 tiles when it has fewer than kSmallBulkTiles 128-tiles, about
// 1.8 rounds of the GPU's 512 bulk slots.  Replaying the bulk launches of the n = 17408 fold
// alone, the 64-tile wins from 820 tiles down (one 128-tile's latency sets such a launch's
// time) and loses from 990 up.
constexpr int kSmallBulkTiles = 900;
static GemmBatch bulk_batch(const GemmProblem& a, const GemmProblem* b) {
    GemmBatch g = gemm_batch(a, b);
    g.small = g.total < kSmallBulkTiles ? 1 : 0;
    return g;
}

// One f32 attempt at damping lam: the scales, the reversed equilibrated matrix, and the blocked
// Cholesky with the blocked inverse trailing it, for the ng groups of ht (the gang open on this
// thread, or one group); rows [u_split, n) of U are made on the inverse's stream once the rows of
// X they read are final (while the last panel's chain runs), and are made again by the next
// attempt if this one fails.  Pivots that are not above tau (or not finite) set the group's flag
// and make its remaining launches return at once.  Ends with the helper streams joined into st.
int fold32_attempt(const HTab& ht, int ng, int64_t n, bool build_vec, const float* hdiag,
                   const uint8_t* dead, FoldState* state, double lam, float tau, char* ws,
                   const FoldLayout& L, float* U, hipStream_t st, const Helper& hp, bool single) {
    float* dinv = (float*)(ws + L.off_dinv);
    float* MI = (float*)(ws + L.off_mi);
    float* A = (float*)(ws + L.off_a);
    float* X = (float*)(ws + L.off_x);
    float* Tb = (float*)(ws + L.off_t);
    float* Xt = (float*)(ws + L.off_xt);
    const int64_t np = L.np;
    const int64_t gs = gang_current().gs;
    const Span st_rw = wr(state, 1, 1, sizeof(FoldState), 1);
    hipStream_t ts = hp.stream;
    auto record = [single](hipEvent_t e, hipStream_t s) { return single ? GPTQ_OK : ev_record(e, s); };
    auto wait = [single](hipStream_t s, hipEvent_t e) { return single ? GPTQ_OK : stream_wait(s, e); };
    {
        ProfScope ps(FAM_FOLD_BUILD, st, 0.0, 4.0 * (double)n * n + 4.0 * (double)np * np / 2);
        GPTQ_LAUNCH(st, "fold_scale",
                    (fold_scale_kernel<<<gang_grid((unsigned)((np + 255) / 256)), 256, 0, st>>>(
                        hdiag, dead, state, lam, n, np, dinv, gs)),
                    rd(hdiag, n, 1, n), rd(dead, n, 1, n, 1), st_rw, wr(dinv, np, 1, np));
        const unsigned build_grid = (unsigned)((np / 64) * (np / 64 + 1) / 2);
        std::vector<Span> acc;
        push_hessians(acc, ht, ng, n);
        acc.push_back(rd(dinv, np, 1, np));
        acc.push_back(rd(dead, n, 1, n, 1));
        acc.push_back(rd(state, 1, 1, sizeof(FoldState), 1));
        acc.push_back(wr(A, np, np, np));
        FOLD_OK(launch_with(st, "fold_build", acc, [&] {
            if (build_vec)
                fold_build_kernel<true><<<gang_grid(build_grid), 256, 0, st>>>(ht, dinv, dead, state,
                                                                              lam, A, n, np, gs);
            else
                fold_build_kernel<false><<<gang_grid(build_grid), 256, 0, st>>>(ht, dinv, dead, state,
                                                                               lam, A, n, np, gs);
        }));
    }
    if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
    // Outer panels of width w (the K of the bulk updates); inside a panel, 128-wide steps
    // factor the diagonal block, solve the rows below and update the rest of the panel.
    // Three streams:
    //   st  the Cholesky's serial chain: the panel steps, then the next panel's columns
    //       (look-ahead of one panel);
    //   ts  the two bulk updates of panel k, one after the other, overlapping the next
    //       panel's chain: the Cholesky's trailing update beyond the next panel (ev_b, which
    //       the look-ahead after next waits for), then the inverse's update of every row of X
    //       below the panel (ev_d);
    //   tx  the inverse's small steps, once panel k of L is final (ev_a): the inverse of the
    //       panel's diagonal block and the panel's rows of X (ev_c; those rows need the
    //       previous panel's update of X, ev_d).  Nothing in the Cholesky waits for them.
    // One bulk update at a time gets the whole GPU beside the chain; two concurrent ones (the
    // inverse's update on tx) each ran at about 75% of the per-launch rate and no sooner.
    hipStream_t tx = hp.stream2;
    bool first_bulk = true;
    bool x_pending = false;  // ev_d holds an update of X that the next rows of X need
    for (int64_t kb = 0; kb < np; kb += L.nb2) {
        const int64_t w = std::min<int64_t>(L.nb2, np - kb);
        const int64_t R = w / NB;
        for (int64_t r = 0; r < R; ++r) {
            const int64_t cb = kb + r * NB;
            const int64_t rest_c = np - cb - NB;
            {
                ProfScope ps(FAM_FOLD_DIAG, st, 2.0 * NB * NB * NB / 3.0, 0.0);
                GPTQ_LAUNCH(st, "fold_diag",
                            (fold_diag_kernel<<<gang_grid(1), 256, 0, st>>>(A, MI, np, (int)(cb / NB),
                                                                           &state->flag, &state->minp32,
                                                                           tau, gs)),
                            rd(A + cb * np + cb, np, NB, NB), wr(MI + (cb / NB) * NB * NB, NB, NB, NB),
                            st_rw);
            }
            if (rest_c <= 0) continue;
            const float* mic = MI + (cb / NB) * NB * NB;
            // L_ic = A_ic MI_c^T for every row below (in place, whole tiles per workgroup).
            const GemmProblem pa = gemm_full(A + (cb + NB) * np + cb, np, mic, NB, nullptr,
                                             A + (cb + NB) * np + cb, np, (int)rest_c, NB, NB,
                                             1.0f, 0);
            {
                ProfScope ps(FAM_FOLD_PANEL, st, 2.0 * NB * NB * (double)rest_c, 0.0);
                FOLD_OK((launch_gemm<1, true, false, false>("fold_panel", st, gemm_batch(pa, nullptr),
                                                            &state->flag)));
            }
            // The rest of the panel's columns: A[cb+128:, cb+128:kb+w] -= L_ic L_jc^T.
            const int64_t ncol = kb + w - cb - NB;
            if (ncol > 0) {
                GemmProblem iu = gemm_full(A + (cb + NB) * np + cb, np, A + (cb + NB) * np + cb,
                                           np, A + (cb + NB) * np + cb + NB,
                                           A + (cb + NB) * np + cb + NB, np, (int)rest_c,
                                           (int)ncol, NB, -1.0f, 1);
                iu.mask_diag = 1;
                iu.skip_upper = 1;
                ProfScope ps(FAM_FOLD_NEXT, st, 2.0 * NB * (double)rest_c * ncol, 0.0);
                FOLD_OK((launch_gemm<4, true, true, false>("fold_in_panel", st, gemm_batch(iu, nullptr),
                                                           &state->flag)));
            }
            if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
        }
        // Panel k of L (and the inverses of its diagonal 128-blocks) is final.
        FOLD_OK(record(hp.ev_a, st));
        const int64_t rest = np - kb - w;
        const float* P = A + (kb + w) * np + kb;  // the panel's rows below its diagonal block

        // --- the inverse, on tx ---
        FOLD_OK(wait(tx, hp.ev_a));
        // Inverse of the panel's w x w diagonal block of L, into X[kb:kb+w, kb:kb+w]: the
        // 128-blocks on the diagonal are the MI_c written by the diagonal kernel; block row I
        // is -MI_I (L[I, <I] X[<I, <I]) (block forward substitution).
        GPTQ_LAUNCH(tx, "fold_x_diag",
                    (fold_x_diag_kernel<<<gang_grid((unsigned)((w + 255) / 256), (unsigned)w), 256, 0, tx>>>(
                        X, MI, np, kb, w, gs)),
                    rd(MI + (kb / NB) * NB * NB, NB, w, NB), wr(X + kb * np + kb, np, w, w));
        if (R > 1) {
            for (int64_t I = 1; I < R; ++I) {
                const int64_t ci = kb + I * NB;
                const GemmBatch t1 = gemm_batch(
                    gemm_full(A + ci * np + kb, np, X + kb * np + kb, np, nullptr, Tb, w, NB,
                              (int)(I * NB), (int)(I * NB), 1.0f, 0),
                    nullptr);
                const GemmBatch t2 = gemm_batch(
                    gemm_full(MI + (ci / NB) * NB * NB, NB, Tb, w, nullptr, X + ci * np + kb, np,
                              NB, (int)(I * NB), NB, -1.0f, 0),
                    nullptr);
                ProfScope ps(FAM_FOLD_PANEL, tx, 2.0 * NB * (double)(I * NB) * (I * NB + NB), 0.0);
                FOLD_OK((launch_gemm<5, false, false, false>("fold_inv_block_a", tx, t1, &state->flag)));
                FOLD_OK((launch_gemm<5, false, false, false>("fold_inv_block_b", tx, t2, &state->flag)));
            }
            if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
        }
        // Rows of X in this panel: X[kb:kb+w, 0:kb] = Minv_w X[kb:kb+w, 0:kb] (out of place,
        // then copied back: a workgroup tile spans only 128 of the w rows it reads).  They
        // need the previous panel's update of X (on ts, ev_d).
        if (kb > 0) {
            if (x_pending) FOLD_OK(wait(tx, hp.ev_d));
            const GemmBatch xb = gemm_batch(
                gemm_full(X + kb * np + kb, np, X + kb * np, np, nullptr, Xt, np, (int)w, (int)kb,
                          (int)w, 1.0f, 0),
                nullptr);
            {
                ProfScope ps(FAM_FOLD_PANEL, tx, 2.0 * (double)w * w * kb, 0.0);
                FOLD_OK((launch_gemm<9, false, false, false>("fold_x_rows", tx, xb, &state->flag)));
            }
            GPTQ_LAUNCH(tx, "fold_copy_rows",
                        (fold_copy_rows_kernel<<<gang_grid((unsigned)((kb + 1023) / 1024), (unsigned)w), 256, 0, tx>>>(
                            Xt, X + kb * np, np, kb, gs)),
                        rd(Xt, np, w, kb), wr(X + kb * np, np, w, kb));
            if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
        }
        if (rest <= 0) continue;
        FOLD_OK(record(hp.ev_c, tx));  // the panel's rows of X are final
        // Every panel but the last has made its rows of X: most of U now, beside the last
        // panel's chain (after ev_c, so that the inverse's update does not wait for it).
        if (kb + w + std::min<int64_t>(L.nb2, rest) >= np) FOLD_OK(fold32_make_u(ws, L, U, n, u_split(n, L), n, tx));

        // --- the Cholesky's trailing update ---
        const int64_t nw = std::min<int64_t>(L.nb2, rest);  // width of the next panel
        const int64_t rest2 = rest - nw;
        // Bulk, on ts: A_ij -= P_i P_j^T beyond the next panel.
        FOLD_OK(wait(ts, hp.ev_a));
        if (rest2 > 0) {
            const GemmProblem sy = gemm_syrk_lower(P + nw * np, np,
                                                   A + (kb + w + nw) * np + kb + w + nw,
                                                   A + (kb + w + nw) * np + kb + w + nw, np,
                                                   (int)rest2, (int)w, -1.0f, 1);
            const double fl = (double)w * rest2 * (rest2 + 1);
            {
                ProfScope ps(FAM_FOLD_UPDATE, ts, fl, 0.0);
                FOLD_OK((launch_gemm<0, true, false, false>("fold_bulk", ts, bulk_batch(sy, nullptr),
                                                            &state->flag)));
            }
            if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
        }
        // Look-ahead, on st: the next panel's columns (rows below kb+w, diagonal tiles lower
        // only); they need the previous panel's bulk update.
        if (!first_bulk) FOLD_OK(wait(st, hp.ev_b));
        GemmProblem strip = gemm_full(P, np, P, np, A + (kb + w) * np + kb + w,
                                      A + (kb + w) * np + kb + w, np, (int)rest, (int)nw,
                                      (int)w, -1.0f, 1);
        strip.mask_diag = 1;
        strip.skip_upper = 1;
        {
            ProfScope ps(FAM_FOLD_NEXT, st, 2.0 * w * (double)rest * nw, 0.0);
            FOLD_OK((launch_gemm<3, true, false, false>("fold_look_ahead", st, gemm_batch(strip, nullptr),
                                                        &state->flag)));
        }
        if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
        if (rest2 > 0) {
            FOLD_OK(record(hp.ev_b, ts));
            first_bulk = false;
        }
        // The inverse's update, on ts after the SYRK: every row below,
        // X_i,<kb+w -= L_i,k X[kb:kb+w, <kb+w] (X's columns kb..kb+w-1 are first written here,
        // so those tiles ignore C_in).
        {
            FOLD_OK(wait(ts, hp.ev_c));
            GemmProblem xu = gemm_full(P, np, X + kb * np, np, X + (kb + w) * np,
                                       X + (kb + w) * np, np, (int)rest, (int)(kb + w), (int)w,
                                       -1.0f, 1);
            xu.beta0_col = (int)kb;
            // Second slot of the bulk kernel (its B layout there is "N": rows of X).
            const GemmProblem none = gemm_none();
            ProfScope ps(FAM_FOLD_UPDATE, ts, 2.0 * w * (double)rest * (kb + w), 0.0);
            FOLD_OK((launch_gemm<0, true, false, false>("fold_x_update", ts, bulk_batch(none, &xu),
                                                        &state->flag)));
            if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
            FOLD_OK(record(hp.ev_d, ts));
            x_pending = true;
        }
    }
    // Join both helper streams.
    FOLD_OK(record(hp.ev_c, tx));
    FOLD_OK(wait(st, hp.ev_c));
    FOLD_OK(record(hp.ev_b, ts));
    FOLD_OK(wait(st, hp.ev_b));
    return GPTQ_OK;
}

// Rows j0 <= j < j1 of U = P X P D^-1 from an f32 attempt: they read rows n-1-j of X, which
// are final once the panel holding them has made its rows of X.
int fold32_make_u(char* ws, const FoldLayout& L, float* U, int64_t n, int64_t j0, int64_t j1,
                  hipStream_t st) {
    if (j1 <= j0) return GPTQ_OK;
    const float* X = (const float*)(ws + L.off_x);
    const float* dinv = (const float*)(ws + L.off_dinv);
    const int64_t np = L.np;
    const int64_t gs = gang_current().gs;
    ProfScope ps(FAM_FOLD_MAKEU, st, 0.0, 4.0 * (double)(j1 - j0) * n);
    const dim3 g64 = gang_grid((unsigned)((n + 63) / 64), (unsigned)((j1 - j0 + 63) / 64));
    const bool vec = n % 4 == 0 && ((uintptr_t)U & 15u) == 0 && gs % 16 == 0;
    GPTQ_LAUNCH(st, "fold_make_u",
                (vec ? fold_make_u_kernel<true><<<g64, 256, 0, st>>>(X, dinv, U, n, np, j0, j1, gs)
                     : fold_make_u_kernel<false><<<g64, 256, 0, st>>>(X, dinv, U, n, np, j0, j1, gs)),
                rd(X + (n - j1) * np, np, j1 - j0, n), rd(dinv, np, 1, np),
                wr(U + j0 * n, n, j1 - j0, n));
    return launch_status() != GPTQ_OK ? GPTQ_EHIP : GPTQ_OK;
}

// The rows of U that an f32 attempt makes before it ends (on the inverse's stream, once the
// rows of X of every panel but the last are final): [u_split(n, L), n).  The rest follows the
// attempt.
int64_t u_split(int64_t n, const FoldLayout& L) {
    const int64_t last = L.np - L.nb2 * ((L.np - 1) / L.nb2);  // width of the last panel
    const int64_t done = L.np - last;                          // rows of X final before it
    return std::max<int64_t>(0, n - done);
}

void fill_report(gptq_fold_report* report, double lam, const FoldState& host, int attempts,
                 bool degenerate, bool use64) {
    if (!report) return;
    report->lambda_used = lam;
    report->base = host.base;
    report->damp = lam * host.base;
    report->attempts = attempts;
    report->n_dead = host.n_dead;
    report->degenerate = degenerate ? 1 : 0;
    report->precision = use64 ? 64 : 32;
    double pm = 0.0;
    if (!degenerate) {
        if (use64) {
            memcpy(&pm, &host.minp64, sizeof(pm));
        } else {
            float p32;
            memcpy(&p32, &host.minp32, sizeof(p32));
            pm = p32;
        }
    }
    report->min_pivot = pm;
}

bool build_vec_ok(const float* H, int64_t n, int64_t ldh) {
    return ldh >= 0 && n % 4 == 0 && ldh % 4 == 0 && al16(H);
}

}  // namespace

int fold_run(const float* H, int64_t n, int64_t ldh, double lambda, int precision, float* U,
             float* hdiag, uint8_t* dead, void* workspace, size_t workspace_bytes, hipStream_t st,
             gptq_fold_report* report, bool single) {
    if (n <= 0 || !hessian_ld_ok(n, ldh) || !H || !U || !hdiag || !dead || !workspace)
        return GPTQ_EINVAL;
    if (n > (int64_t)1 << 20) return GPTQ_EINVAL;
    if (precision != GPTQ_FOLD_AUTO && precision != GPTQ_FOLD_F32 && precision != GPTQ_FOLD_F64)
        return GPTQ_EINVAL;
    if (!al16(workspace)) return GPTQ_EINVAL;  // its matrices are read as float4 / double2
    const FoldLayout L = fold_layout(n);
    if (workspace_bytes < (precision == GPTQ_FOLD_F32 ? L.total_f32 : L.total)) return GPTQ_EWORKSPACE;
    CheckScope check;
    check_buffer(H, sizeof(float) * (size_t)hessian_elems(n, ldh), "H");
    check_buffer(U, sizeof(float) * (size_t)(n * n), "U");
    check_buffer(hdiag, sizeof(float) * (size_t)n, "hdiag");
    check_buffer(dead, (size_t)n, "dead");
    check_buffer(workspace, workspace_bytes, "workspace");
    char* ws = (char*)workspace;
    FoldState* state = (FoldState*)(ws + L.off_state);
    const HTab ht = htab_one(H, ldh);
    const HLayout hl{n, ldh};

    FOLD_OK(fold_prep(ht, 1, n, hdiag, dead, state, st));

    // single: every launch on st, in program order (an order the helper streams' events allow,
    // so the same results bit for bit); no helper stream or event is taken.
    Helper hp{st, st, nullptr, nullptr, nullptr, nullptr, -1};
    if (!single && helper_acquire(&hp) != GPTQ_OK) return GPTQ_EHIP;
    struct Release {
        const Helper& h;
        ~Release() { helper_release(h); }
    } release{hp};

    double lam = (lambda > 0.0) ? lambda : 0.0;
    int attempts = 0;
    FoldState host{};
    bool degenerate = false;
    // f64 from the start, or once an f32 attempt of the "auto" precision met a pivot at or below
    // the floor (then for the rest of the damping schedule).
    bool use64 = precision == GPTQ_FOLD_F64;
    const float tau = precision == GPTQ_FOLD_AUTO ? kF32PivotFloor : 0.0f;
    for (;;) {
        ++attempts;
        if (use64)
            FOLD_OK(fold64_attempt(H, hl, hdiag, dead, state, lam, ws, L, st, hp, single));
        else
            FOLD_OK(fold32_attempt(ht, 1, n, build_vec_ok(H, n, ldh), hdiag, dead, state, lam, tau,
                                   ws, L, U, st, hp, single));
        if (dry_run()) {
            host_sync_record(st);
            host.flag = 0u;
            host.base = 1.0;
            host.n_dead = 0;
        } else {
            GPTQ_HIP(hipMemcpyAsync(&host, state, sizeof(FoldState), hipMemcpyDeviceToHost, st));
            GPTQ_HIP(hipStreamSynchronize(st));
        }
        if (host.flag == 0u) break;
        if (!use64 && precision == GPTQ_FOLD_AUTO) {
            use64 = true;  // the same damping again, in f64
            continue;
        }
        lam = (lam == 0.0) ? 1e-4 : lam * 10.0;
        if (lam > 10.0) {
            degenerate = true;
            break;
        }
    }
    const dim3 g((unsigned)((n + 31) / 32), (unsigned)((n + 31) / 32));
    if (degenerate) {
        GPTQ_LAUNCH(st, "fold_identity", (fold_identity_kernel<<<g, 256, 0, st>>>(U, n)), wr(U, n, n, n));
        if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
    } else if (use64) {
        FOLD_OK(fold64_make_u(U, n, ws, L, st));
    } else {
        FOLD_OK(fold32_make_u(ws, L, U, n, 0, u_split(n, L), st));
    }
    FOLD_OK(check.finish());
    fill_report(report, lam, host, attempts, degenerate, use64);
    return degenerate ? GPTQ_DEGENERATE : GPTQ_OK;
}

int fold_gang(const HTab& ht, int G, int64_t gs, int64_t n, double lambda, int precision,
              float* U, float* hdiag, uint8_t* dead, char* ws, size_t ws_bytes, hipStream_t st,
              FoldState* host, unsigned* failed, gptq_fold_report* reports) {
    if (G < 1 || G > kMaxGang || n <= 0 || n > ((int64_t)1 << 20)) return GPTQ_EINVAL;
    if (precision != GPTQ_FOLD_AUTO && precision != GPTQ_FOLD_F32) return GPTQ_EINVAL;
    if (gs % 256 != 0 || !al16(ws) || !al16(U)) return GPTQ_EINVAL;
    const FoldLayout L = fold_layout(n);
    if (ws_bytes < L.total_f32) return GPTQ_EWORKSPACE;
    bool vec = true;
    for (int g = 0; g < G; ++g) {
        if (!ht.H[g] || !hessian_ld_ok(n, ht.ldh[g])) return GPTQ_EINVAL;
        vec = vec && build_vec_ok(ht.H[g], n, ht.ldh[g]);
    }
    CheckScope check;
    for (int g = 0; g < G; ++g) {
        check_buffer(ht.H[g], sizeof(float) * (size_t)hessian_elems(n, ht.ldh[g]), "H");
        check_buffer((const char*)U + g * gs, sizeof(float) * (size_t)(n * n), "U");
        check_buffer((const char*)hdiag + g * gs, sizeof(float) * (size_t)n, "hdiag");
        check_buffer((const char*)dead + g * gs, (size_t)n, "dead");
        check_buffer(ws + g * gs, ws_bytes, "workspace");
    }
    FoldState* state = (FoldState*)(ws + L.off_state);
    const double lam = (lambda > 0.0) ? lambda : 0.0;
    const float tau = precision == GPTQ_FOLD_AUTO ? kF32PivotFloor : 0.0f;
    Helper hp{};
    if (helper_acquire(&hp) != GPTQ_OK) return GPTQ_EHIP;
    struct Release {
        const Helper& h;
        ~Release() { helper_release(h); }
    } release{hp};
    {
        GangScope gang(G, gs);
        FOLD_OK(fold_prep(ht, G, n, hdiag, dead, state, st));
        FOLD_OK(fold32_attempt(ht, G, n, vec, hdiag, dead, state, lam, tau, ws, L, U, st, hp, false));
        FOLD_OK(fold32_make_u(ws, L, U, n, 0, u_split(n, L), st));
    }
    if (dry_run()) {
        host_sync_record(st);
        for (int g = 0; g < G; ++g) {
            host[g] = FoldState{};
            host[g].base = 1.0;
        }
    } else {
        for (int g = 0; g < G; ++g)
            GPTQ_HIP(hipMemcpyAsync(&host[g], (const char*)state + g * gs, sizeof(FoldState),
                                    hipMemcpyDeviceToHost, st));
        GPTQ_HIP(hipStreamSynchronize(st));
    }
    FOLD_OK(check.finish());
    for (int g = 0; g < G; ++g) {
        failed[g] = host[g].flag;
        if (host[g].flag == 0u) fill_report(&reports[g], lam, host[g], 1, false, false);
    }
    return GPTQ_OK;
}

#undef FOLD_OK

}  // namespace gptq
