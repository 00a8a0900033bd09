// fold64.hip -- the damped, equilibrated GPTQ fold in f64 on gfx950.
//
// The same operator as the f32 fold (fold.hip): U = P L^-1 P D^-1, the upper Cholesky factor of
// H_d^-1, from the reversed equilibrated matrix A = P D^-1 H_d D^-1 P = L L^T.  The f32 factor
// of A is accurate to about u32 / (smallest pivot); where that pivot is small (rank-deficient
// Hessians at small damping) the fold runs here instead, in the precision of the pages' host
// fold (page "cortiq-cli 0.8.45 src/gptq.rs", gptq_fold_operator_par, f64; page "cortiq-engine
// 0.8.41 src/gpu_wgpu/gptq_dev.rs", module documentation steps 1-4, which state that the
// device operator equals the host's up to rounding).  The pivot rule is the host's: a pivot
// that is not positive or not finite fails the attempt (the caller raises the damping).
//
// Device layout (f64, padded to n_p, a multiple of 128, identity padding):
//   A64 [n_p][n_p]  the reversed equilibrated matrix, then L (lower) in place
//   X64 [n_p][n_p]  L^-1 (lower), block row by block row
//   MI  [n_p/64][64][64]  inverses of L's 64 x 64 diagonal blocks
//   dinv [n_p]      (H_ii + damp)^-1/2, dead: (1 + damp)^-1/2
//   Tb [64][256], Xt [256][n_p]   staging for the inverse's small steps
//
// Per outer panel of w = 256 columns (four 64-wide steps), all on the caller's stream:
//   step   : diag (L_cc, MI_c = L_cc^-1, one wave in registers), panel solve L_ic = A_ic MI_c^T
//            (in place),
//            the rest of the panel's columns A -= L_ic L_jc^T;
//   inverse: the panel's w x w diagonal block of X by block forward substitution from the MI,
//            its rows of X, X[kb:kb+w, <kb] = X_ww X[kb:kb+w, <kb] (staged, copied back);
//   bulk   : one launch with two problems, the trailing SYRK A[kb+w:, kb+w:] -= P P^T and the
//            inverse's update X[kb+w:, <kb+w] -= P X[kb:kb+w, <kb+w], P = L[kb+w:, kb:kb+w].
#include <math.h>

#include <utility>

#include "fold.hpp"
#include "gemm64.hpp"

namespace gptq {

// Per attempt: f64 inverse equilibration scales; the flag and the smallest-pivot record reset.
__global__ void fold64_scale_kernel(const float* __restrict__ hdiag, const uint8_t* __restrict__ dead,
                                    FoldState* st, double lam, int64_t n, int64_t np,
                                    double* __restrict__ dinv) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0) {
        __atomic_store_n(&st->flag, 0u, __ATOMIC_RELAXED);
        __atomic_store_n(&st->minp64, 0x7FF0000000000000ull, __ATOMIC_RELAXED);  // +inf
    }
    if (i >= np) return;
    if (i >= n) {
        dinv[i] = 1.0;
        return;
    }
    const double damp = lam * st->base;
    const double v = dead[i] ? 1.0 + damp : (double)hdiag[i] + damp;
    dinv[i] = 1.0 / sqrt(v);
}

// A[i][j] (i >= j) of the reversed, damped, equilibrated H read from its upper triangle, in
// f64; the padding block is the identity and the entries above the diagonal inside diagonal
// tiles are 0.  One workgroup per lower 64 x 64 tile; a wave covers one row of the tile, so the
// reads of H (its columns in reverse order) and the writes of A coalesce.
__global__ __launch_bounds__(256) void fold64_build_kernel(const float* __restrict__ H, HLayout hl,
                                                           const double* __restrict__ dinv,
                                                           const uint8_t* __restrict__ dead,
                                                           const FoldState* st, double lam,
                                                           double* __restrict__ A, int64_t n,
                                                           int64_t np) {
    int ti, tj;
    tri_of(blockIdx.x, ti, tj);
    const double damp = lam * st->base;
    const int64_t j = (int64_t)tj * 64 + (threadIdx.x & 63);
    const bool jin = j < n;
    const int64_t bc = n - 1 - j;  // column of H
    const bool dead_b = jin && dead[bc];
    const double db = jin ? dinv[bc] : 0.0;
#pragma unroll 4
    for (int q = 0; q < 16; ++q) {
        const int64_t i = (int64_t)ti * 64 + (threadIdx.x >> 6) + 4 * q;
        double v;
        if (j > i) {
            v = 0.0;
        } else if (i >= n || !jin) {
            v = (i == j) ? 1.0 : 0.0;
        } else {
            const int64_t a = n - 1 - i;  // a <= bc: the upper triangle of H
            if (dead[a] || dead_b) v = (a == bc) ? 1.0 : 0.0;
            else if (a == bc) v = ((double)H[hl.at(a, a)] + damp) * db * db;
            else v = (double)H[hl.at(a, bc)] * dinv[a] * db;
        }
        A[i * np + j] = v;
    }
}

// Diagonal block at cb: L_cc = chol(A_cc) and MI = L_cc^-1, 64 x 64, by one wave in registers.
// Lane i holds row i of the block (x[], becoming row i of L) and column i of the inverse (t[],
// starting as e_i).  Step c: the pivot x[c] of lane c is tested and turned into 1 / L_cc; x[c]
// scaled by it makes L_ic final on every lane (L_cc on lane c), t[c] scaled by it makes
// T_c,i final; then for every s > c the entry L_sc, broadcast from lane s, drives the same
// update in both halves: the Cholesky update x[s] -= L_ic L_sc of the later columns and the
// substitution step t[s] -= T_c,i L_sc.  Entries above the diagonal of x carry values nothing
// reads.  A pivot that is not positive and finite sets flag bit 0 and is replaced by 1 so the
// arithmetic stays finite; the smallest accepted pivot goes to minp64.
__device__ __forceinline__ double bcast_f64(double v, int src) {
    const int lo = __builtin_amdgcn_readlane(__double2loint(v), src);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(v), src);
    return __hiloint2double(hi, lo);
}

template <int C>
__device__ __forceinline__ void leaf64_step(double (&x)[NB64], double (&t)[NB64], bool& bad,
                                            double& pmin) {
    double p = bcast_f64(x[C], C);
    const bool b = !(p > 0.0) || !isfinite(p);
    bad = bad || b;
    pmin = b ? pmin : fmin(pmin, p);
    p = b ? 1.0 : p;
    const double rl = 1.0 / sqrt(p);
    x[C] *= rl;
    t[C] *= rl;
    // Four broadcasts at a time, each group fenced off from the next (an empty asm that
    // "rewrites" x[C]), so the scalar registers they occupy stay few instead of every broadcast
    // of the step being hoisted together and spilled.
#pragma unroll
    for (int s0 = (C + 1) & ~3; s0 < NB64; s0 += 4) {
        double ls[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (s0 + u > C) ls[u] = bcast_f64(x[C], s0 + u);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (s0 + u > C) {
                x[s0 + u] -= x[C] * ls[u];
                t[s0 + u] -= t[C] * ls[u];
            }
        asm volatile("" : "+v"(x[C]));
    }
#pragma unroll
    for (int s2 = C + 1; s2 < NB64; ++s2) asm volatile("" : "+v"(x[s2]), "+v"(t[s2]));
}

template <int... C>
__device__ __forceinline__ void leaf64_steps(double (&x)[NB64], double (&t)[NB64], bool& bad,
                                             double& pmin, std::integer_sequence<int, C...>) {
    (leaf64_step<C>(x, t, bad, pmin), ...);
}

__global__ __launch_bounds__(64) void fold64_diag_kernel(const double* __restrict__ A,
                                                         double* __restrict__ MI, int64_t np,
                                                         int64_t cb, FoldState* st) {
    if (__atomic_load_n(&st->flag, __ATOMIC_RELAXED)) return;
    __builtin_amdgcn_s_setprio(CHAIN_PRIO);
    const int lane = threadIdx.x;
    double x[NB64], t[NB64];
    const double* arow = A + (cb + lane) * np + cb;
#pragma unroll
    for (int k = 0; k < NB64; k += 2) {
        const f64x2 v = *reinterpret_cast<const f64x2*>(arow + k);
        x[k] = (k <= lane) ? v[0] : 0.0;
        x[k + 1] = (k + 1 <= lane) ? v[1] : 0.0;
        t[k] = (k == lane) ? 1.0 : 0.0;
        t[k + 1] = (k + 1 == lane) ? 1.0 : 0.0;
    }
    bool bad = false;
    double pmin = INFINITY;
    leaf64_steps(x, t, bad, pmin, std::make_integer_sequence<int, NB64>{});
    // MI[i][lane] = T_i,lane: row i of MI is written by the 64 lanes together.
    double* mi = MI + (cb / NB64) * NB64 * NB64;
#pragma unroll
    for (int i = 0; i < NB64; ++i) mi[i * NB64 + lane] = t[i];
    if (lane == 0) {
        if (bad) atomicOr(&st->flag, 1u);
        atomicMin(&st->minp64, (unsigned long long)__double_as_longlong(pmin));
    }
}

// The w x w diagonal block of X at kb before its block forward substitution: the diagonal
// 64-blocks are the MI, the blocks above are 0 (the blocks below are written by the
// substitution).
__global__ __launch_bounds__(256) void fold64_x_diag_kernel(double* __restrict__ X,
                                                            const double* __restrict__ MI,
                                                            int64_t np, int64_t kb, int64_t w,
                                                            const FoldState* st) {
    if (__atomic_load_n(&st->flag, __ATOMIC_RELAXED)) return;
    const int64_t r = blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= w) return;
    const int64_t I = r / NB64, J = c / NB64;
    if (J > I) X[(kb + r) * np + kb + c] = 0.0;
    else if (J == I) X[(kb + r) * np + kb + c] = MI[((kb / NB64 + I) * NB64 + (r % NB64)) * NB64 + (c % NB64)];
}

__global__ __launch_bounds__(256) void fold64_copy_rows_kernel(const double* __restrict__ src,
                                                               double* __restrict__ dst, int64_t ld,
                                                               int64_t cols, const FoldState* st) {
    if (__atomic_load_n(&st->flag, __ATOMIC_RELAXED)) return;
    const int64_t r = blockIdx.y;
    for (int64_t c = (int64_t)blockIdx.x * 512 + threadIdx.x * 2; c < cols; c += (int64_t)gridDim.x * 512)
        *reinterpret_cast<f64x2*>(dst + r * ld + c) = *reinterpret_cast<const f64x2*>(src + r * ld + c);
}

// U[j][c] = f32(X[n-1-j][n-1-c] * dinv[c]) for c >= j, 0 below the diagonal.  One workgroup
// per 64 x 64 tile of U; a wave covers one row of the tile.
__global__ __launch_bounds__(256) void fold64_make_u_kernel(const double* __restrict__ X,
                                                            const double* __restrict__ dinv,
                                                            float* __restrict__ U, int64_t n,
                                                            int64_t np) {
    const bool below = blockIdx.x < blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
    if (c >= n) return;
    const double dc = below ? 0.0 : dinv[c];
#pragma unroll 4
    for (int q = 0; q < 16; ++q) {
        const int64_t j = (int64_t)blockIdx.y * 64 + (threadIdx.x >> 6) + 4 * q;
        if (j >= n) continue;
        U[j * n + c] = (!below && c >= j) ? (float)(X[(n - 1 - j) * np + (n - 1 - c)] * dc) : 0.0f;
    }
}

#define F64_OK(call)                    \
    do {                                \
        const int rc_ = (call);         \
        if (rc_ != GPTQ_OK) return rc_; \
    } while (0)

int fold64_attempt(const float* H, HLayout hl, const float* hdiag, const uint8_t* dead,
                   FoldState* state, double lam, char* ws, const FoldLayout& L, hipStream_t st,
                   const Helper& hp, bool single) {
    const int64_t n = hl.n, np = L.np;
    double* A = (double*)(ws + L.off_a);
    double* X = (double*)(ws + L.off_x64);
    double* MI = (double*)(ws + L.off_mi64);
    double* dinv = (double*)(ws + L.off_dinv64);
    double* Tb = (double*)(ws + L.off_tb64);
    double* Xt = (double*)(ws + L.off_xt64);
    const unsigned* flag = &state->flag;
    const Span st_rw = wr(state, 1, 1, sizeof(FoldState), 1);
    // Streams as in the f32 fold: st the Cholesky's serial chain and the look-ahead of the next
    // panel's columns; ts the trailing update beyond the next panel, then the inverse's update
    // of the rows of X below the panel; tx the inverse's small steps (its diagonal block and
    // the panel's rows of X).  single: all of it on st, in program order.  The pivot flag, which
    // only goes from 0 to set and makes later launches return at once, is polled by launches on
    // every stream and left out of their recorded accesses, as the GEMMs leave it out.
    hipStream_t ts = single ? st : hp.stream, tx = single ? st : hp.stream2;
    auto record = [single](hipEvent_t e, hipStream_t s) { return single ? GPTQ_OK : ev_record(e, s); };
    auto wait = [single](hipStream_t s, hipEvent_t e) { return single ? GPTQ_OK : stream_wait(s, e); };
    {
        ProfScope ps(FAM_FOLD_BUILD, st, 0.0, 4.0 * (double)n * n + 8.0 * (double)np * np / 2);
        GPTQ_LAUNCH(st, "fold64_scale",
                    (fold64_scale_kernel<<<(unsigned)((np + 255) / 256), 256, 0, st>>>(hdiag, dead, state,
                                                                                      lam, n, np, dinv)),
                    rd(hdiag, n, 1, n), rd(dead, n, 1, n, 1), st_rw, wr(dinv, np, 1, np, 8));
        const unsigned grid = (unsigned)((np / 64) * (np / 64 + 1) / 2);
        GPTQ_LAUNCH(st, "fold64_build",
                    (fold64_build_kernel<<<grid, 256, 0, st>>>(H, hl, dinv, dead, state, lam, A, n, np)),
                    hessian_span(H, n, hl.ldh, false), rd(dinv, np, 1, np, 8), rd(dead, n, 1, n, 1),
                    rd(state, 1, 1, sizeof(FoldState), 1), wr(A, np, np, np, 8));
    }
    if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
    bool first_bulk = true;
    bool x_pending = false;  // ev_d holds an update of X that the next rows of X need
    for (int64_t kb = 0; kb < np; kb += W64) {
        const int64_t w = std::min<int64_t>(W64, np - kb);
        const int64_t R = w / NB64;
        for (int64_t r = 0; r < R; ++r) {
            const int64_t cb = kb + r * NB64;
            const int64_t rest_c = np - cb - NB64;
            {
                ProfScope ps(FAM_FOLD_DIAG, st, 2.0 * NB64 * NB64 * NB64 / 3.0, 0.0);
                GPTQ_LAUNCH(st, "fold64_diag",
                            (fold64_diag_kernel<<<1, 64, 0, st>>>(A, MI, np, cb, state)),
                            rd(A + cb * np + cb, np, NB64, NB64, 8),
                            wr(MI + (cb / NB64) * NB64 * NB64, NB64, NB64, NB64, 8), st_rw);
            }
            if (rest_c <= 0) continue;
            const double* mic = MI + (cb / NB64) * NB64 * NB64;
            {
                // L_ic = A_ic MI_c^T for every row below, in place: a 64 x 64 tile spans the
                // whole block column it reads before it writes.
                ProfScope ps(FAM_FOLD_PANEL, st, 2.0 * NB64 * NB64 * (double)rest_c, 0.0);
                F64_OK((launch_gemm64<64, 64, true, false, true>(
                    "fold64_panel", st,
                    gemm64_full(A + (cb + NB64) * np + cb, np, mic, NB64, nullptr,
                                A + (cb + NB64) * np + cb, np, (int)rest_c, NB64, NB64, 1.0, 0),
                    nullptr, flag)));
            }
            const int64_t ncol = kb + w - cb - NB64;
            if (ncol > 0) {
                GemmProblem64 iu = gemm64_full(A + (cb + NB64) * np + cb, np, A + (cb + NB64) * np + cb,
                                               np, A + (cb + NB64) * np + cb + NB64,
                                               A + (cb + NB64) * np + cb + NB64, np, (int)rest_c,
                                               (int)ncol, NB64, -1.0, 1);
                iu.mask_diag = 1;
                iu.skip_upper = 1;
                ProfScope ps(FAM_FOLD_NEXT, st, 2.0 * NB64 * (double)rest_c * ncol, 0.0);
                F64_OK((launch_gemm64<64, 64, true, false, true>("fold64_in_panel", st, iu, nullptr, flag)));
            }
            if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
        }
        // Panel k of L (and the inverses of its diagonal 64-blocks) is final.
        F64_OK(record(hp.ev_a, st));
        const int64_t rest = np - kb - w;
        const double* P = A + (kb + w) * np + kb;  // the panel's rows below its diagonal block

        // --- the inverse, on tx ---
        F64_OK(wait(tx, hp.ev_a));
        // The inverse of the panel's w x w diagonal block into X[kb:kb+w, kb:kb+w]: block row I
        // is -MI_I (L[I, <I] X[<I, <I]) below the diagonal block MI_I.
        GPTQ_LAUNCH(tx, "fold64_x_diag",
                    (fold64_x_diag_kernel<<<dim3((unsigned)((w + 255) / 256), (unsigned)w), 256, 0, tx>>>(
                        X, MI, np, kb, w, state)),
                    rd(MI + (kb / NB64) * NB64 * NB64, NB64, w, NB64, 8), wr(X + kb * np + kb, np, w, w, 8));
        for (int64_t I = 1; I < R; ++I) {
            const int64_t ci = kb + I * NB64;
            ProfScope ps(FAM_FOLD_PANEL, tx, 2.0 * NB64 * (double)(I * NB64) * (I * NB64 + NB64), 0.0);
            F64_OK((launch_gemm64<64, 64, false, false, true>(
                "fold64_inv_block_a", tx,
                gemm64_full(A + ci * np + kb, np, X + kb * np + kb, np, nullptr, Tb, W64, NB64,
                            (int)(I * NB64), (int)(I * NB64), 1.0, 0),
                nullptr, flag)));
            F64_OK((launch_gemm64<64, 64, false, false, true>(
                "fold64_inv_block_b", tx,
                gemm64_full(MI + (ci / NB64) * NB64 * NB64, NB64, Tb, W64, nullptr, X + ci * np + kb, np,
                            NB64, (int)(I * NB64), NB64, -1.0, 0),
                nullptr, flag)));
        }
        if (kb > 0) {
            // Rows of X in this panel, X[kb:kb+w, <kb] = X_ww X[kb:kb+w, <kb]: staged in Xt (a
            // tile reads all w rows of its columns) and copied back.  They need the previous
            // panel's update of X (on ts, ev_d).
            if (x_pending) F64_OK(wait(tx, hp.ev_d));
            {
                ProfScope ps(FAM_FOLD_PANEL, tx, 2.0 * (double)w * w * kb, 0.0);
                F64_OK((launch_gemm64<64, 64, false, false, true>(
                    "fold64_x_rows", tx,
                    gemm64_full(X + kb * np + kb, np, X + kb * np, np, nullptr, Xt, np, (int)w, (int)kb,
                                (int)w, 1.0, 0),
                    nullptr, flag)));
            }
            GPTQ_LAUNCH(tx, "fold64_copy_rows",
                        (fold64_copy_rows_kernel<<<dim3((unsigned)((kb + 511) / 512), (unsigned)w), 256, 0, tx>>>(
                            Xt, X + kb * np, np, kb, state)),
                        rd(Xt, np, w, kb, 8), wr(X + kb * np, np, w, kb, 8));
        }
        if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
        if (rest <= 0) continue;
        F64_OK(record(hp.ev_c, tx));  // the panel's rows of X are final

        // --- the Cholesky's trailing update ---
        const int64_t nw = std::min<int64_t>(W64, rest);  // width of the next panel
        const int64_t rest2 = rest - nw;
        // Bulk, on ts: A_ij -= P_i P_j^T beyond the next panel.
        F64_OK(wait(ts, hp.ev_a));
        if (rest2 > 0) {
            const GemmProblem64 sy = gemm64_syrk_lower(P + nw * np, np, A + (kb + w + nw) * np + kb + w + nw,
                                                       A + (kb + w + nw) * np + kb + w + nw, np,
                                                       (int)rest2, (int)w, -1.0, 1);
            ProfScope ps(FAM_FOLD_UPDATE, ts, (double)w * rest2 * (rest2 + 1), 0.0);
            F64_OK((launch_gemm64<64, 64, true, false>("fold64_bulk", ts, sy, nullptr, flag)));
        }
        // Look-ahead, on st: the next panel's columns (rows below kb+w, diagonal tiles lower
        // only); they need the previous panel's bulk update.
        if (!first_bulk) F64_OK(wait(st, hp.ev_b));
        {
            GemmProblem64 strip = gemm64_full(P, np, P, np, A + (kb + w) * np + kb + w,
                                              A + (kb + w) * np + kb + w, np, (int)rest, (int)nw,
                                              (int)w, -1.0, 1);
            strip.mask_diag = 1;
            strip.skip_upper = 1;
            ProfScope ps(FAM_FOLD_NEXT, st, 2.0 * w * (double)rest * nw, 0.0);
            F64_OK((launch_gemm64<64, 64, true, false, true>("fold64_look_ahead", st, strip, nullptr, flag)));
        }
        if (rest2 > 0) {
            F64_OK(record(hp.ev_b, ts));
            first_bulk = false;
        }
        // The inverse's update, on ts after the SYRK: every row below,
        // X_i,<kb+w -= L_i,k X[kb:kb+w, <kb+w] (X's columns kb..kb+w-1 are first written here,
        // so those tiles ignore C_in).
        {
            F64_OK(wait(ts, hp.ev_c));
            GemmProblem64 xu = gemm64_full(P, np, X + kb * np, np, X + (kb + w) * np, X + (kb + w) * np,
                                           np, (int)rest, (int)(kb + w), (int)w, -1.0, 1);
            xu.beta0_col = (int)kb;
            ProfScope ps(FAM_FOLD_UPDATE, ts, 2.0 * w * (double)rest * (kb + w), 0.0);
            F64_OK((launch_gemm64<64, 64, true, false>("fold64_x_update", ts, gemm64_none(), &xu, flag)));
            F64_OK(record(hp.ev_d, ts));
            x_pending = true;
        }
        if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
    }
    // Join both helper streams.
    F64_OK(record(hp.ev_c, tx));
    F64_OK(wait(st, hp.ev_c));
    F64_OK(record(hp.ev_b, ts));
    F64_OK(wait(st, hp.ev_b));
    return GPTQ_OK;
}

int fold64_make_u(float* U, int64_t n, char* ws, const FoldLayout& L, hipStream_t st) {
    const double* X = (const double*)(ws + L.off_x64);
    const double* dinv = (const double*)(ws + L.off_dinv64);
    const dim3 g64((unsigned)((n + 63) / 64), (unsigned)((n + 63) / 64));
    ProfScope ps(FAM_FOLD_MAKEU, st, 0.0, 4.0 * (double)n * n + 4.0 * (double)n * n);
    GPTQ_LAUNCH(st, "fold64_make_u", (fold64_make_u_kernel<<<g64, 256, 0, st>>>(X, dinv, U, n, L.np)),
                rd(X, L.np, L.np, L.np, 8), rd(dinv, L.np, 1, L.np, 8), wr(U, n, n, n));
    return launch_status() == GPTQ_OK ? GPTQ_OK : GPTQ_EHIP;
}

#undef F64_OK

}  // namespace gptq
