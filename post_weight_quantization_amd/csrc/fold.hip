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
//   update : A_ij -= L_ik L_jk^T (lower tiles);      X_i,<=k -= L_ik X_k,<=k   (one GEMM launch)
// The pages factor and invert in two separate passes; both are right-looking and the inverse
// of step k only needs L's column block k, so one pass does both.
#include <math.h>

#include "common.hpp"
#include "gemm_mfma.hpp"

namespace gptq {

constexpr int NB = 128;
constexpr int LDL = NB + 1;

struct FoldState {
    double base;
    unsigned flag;
    int n_dead;
    double pad[6];
};

// Diagonal, dead mask, mean of the diagonal with dead channels counted as 1 (f64, fixed
// reduction order).
__global__ __launch_bounds__(1024) void fold_prep_kernel(const float* __restrict__ H, int64_t n,
                                                          int64_t ldh, float* __restrict__ hdiag,
                                                          uint8_t* __restrict__ dead,
                                                          FoldState* st) {
    __shared__ double ssum[1024];
    __shared__ int scnt[1024];
    const int t = threadIdx.x;
    double s = 0.0;
    int cnt = 0;
    for (int64_t i = t; i < n; i += 1024) {
        const float d = H[i * ldh + i];
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
                                  float* __restrict__ dinv) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0) __atomic_store_n(&st->flag, 0u, __ATOMIC_RELAXED);
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
// padding block is the identity; entries above the diagonal inside diagonal 32x32 tiles are 0.
__global__ __launch_bounds__(256) void fold_build_kernel(const float* __restrict__ H, int64_t ldh,
                                                         const float* __restrict__ dinv,
                                                         const uint8_t* __restrict__ dead,
                                                         const FoldState* st, double lam,
                                                         float* __restrict__ A, int64_t n,
                                                         int64_t np) {
    const int tj = blockIdx.x, ti = blockIdx.y;
    if (tj > ti) return;
    const double damp = lam * st->base;
    for (int e = threadIdx.x; e < 32 * 32; e += 256) {
        const int64_t i = (int64_t)ti * 32 + (e >> 5);
        const int64_t j = (int64_t)tj * 32 + (e & 31);
        float v;
        if (j > i) {
            v = 0.0f;
        } else if (i >= n || j >= n) {
            v = (i == j) ? 1.0f : 0.0f;
        } else {
            const int64_t a = n - 1 - i, b = n - 1 - j;  // a <= b: upper triangle of H
            if (dead[a] || dead[b]) {
                v = (a == b) ? 1.0f : 0.0f;
            } else if (a == b) {
                const double di = (double)dinv[a];
                v = (float)(((double)H[a * ldh + a] + damp) * di * di);
            } else {
                v = H[a * ldh + b] * dinv[a] * dinv[b];
            }
        }
        A[i * np + j] = v;
    }
}

// L_kk = chol(A_kk) and MI_k = L_kk^-1 for the NB x NB diagonal block at k * NB.
// Cholesky: right-looking by columns with the column scaling deferred (the trailing update
// uses a_rc a_sc / p_c); a pivot that is not > 0 (or NaN) sets the flag and is replaced by 1.
// Inverse: column c of L^-1 by forward substitution, one thread per column.
__global__ __launch_bounds__(256) void fold_diag_kernel(float* __restrict__ A, float* __restrict__ X,
                                                        float* __restrict__ MI, int64_t np, int k,
                                                        unsigned* flag) {
    if (__atomic_load_n(flag, __ATOMIC_RELAXED)) return;
    __shared__ float Ls[NB * LDL];
    __shared__ float Ms[NB * LDL];
    __shared__ float piv[NB];
    const int tid = threadIdx.x;
    const int64_t kb = (int64_t)k * NB;
    for (int e = tid; e < NB * NB; e += 256) {
        const int r = e / NB, c = e % NB;
        Ls[r * LDL + c] = (c <= r) ? A[(kb + r) * np + kb + c] : 0.0f;
    }
    __syncthreads();
    const int s = tid & (NB - 1), par = tid >> 7;
    bool bad_any = false;
    for (int c = 0; c < NB; ++c) {
        const float p = Ls[c * LDL + c];
        const bool bad = !(p > 0.0f);
        const float pp = bad ? 1.0f : p;
        if (s > c) {
            const float lsc = Ls[s * LDL + c] / pp;
            for (int r = s + par; r < NB; r += 2) Ls[r * LDL + s] -= Ls[r * LDL + c] * lsc;
        }
        if (tid == 0) {
            piv[c] = pp;
            bad_any = bad_any || bad;
        }
        __syncthreads();
    }
    if (tid == 0 && bad_any) atomicOr(flag, 1u);
    for (int e = tid; e < NB * NB; e += 256) {
        const int r = e / NB, c = e % NB;
        if (c < r) Ls[r * LDL + c] = Ls[r * LDL + c] / sqrtf(piv[c]);
        else if (c == r) Ls[r * LDL + c] = sqrtf(piv[c]);
    }
    __syncthreads();
    if (tid < NB) {
        const int c = tid;
        for (int r = 0; r < NB; ++r) Ms[r * LDL + c] = (r == c) ? 1.0f : 0.0f;
        for (int q = 0; q < NB; ++q) {
            if (q >= c) {
                const float mq = Ms[q * LDL + c] / Ls[q * LDL + q];
                Ms[q * LDL + c] = mq;
                for (int r = q + 1; r < NB; ++r) Ms[r * LDL + c] -= Ls[r * LDL + q] * mq;
            }
        }
    }
    __syncthreads();
    float* mi = MI + (int64_t)k * NB * NB;
    for (int e = tid; e < NB * NB; e += 256) {
        const int r = e / NB, c = e % NB;
        const float m = (c <= r) ? Ms[r * LDL + c] : 0.0f;
        if (c <= r) A[(kb + r) * np + kb + c] = Ls[r * LDL + c];
        mi[e] = m;
        X[(kb + r) * np + kb + c] = m;
    }
}

// U[j][c] = X[n-1-j][n-1-c] * dinv[c] for c >= j, 0 below the diagonal.
__global__ __launch_bounds__(256) void fold_make_u_kernel(const float* __restrict__ X,
                                                          const float* __restrict__ dinv,
                                                          float* __restrict__ U, int64_t n,
                                                          int64_t np) {
    for (int e = threadIdx.x; e < 32 * 32; e += 256) {
        const int64_t j = (int64_t)blockIdx.y * 32 + (e >> 5);
        const int64_t c = (int64_t)blockIdx.x * 32 + (e & 31);
        if (j >= n || c >= n) continue;
        U[j * n + c] = (c >= j) ? X[(n - 1 - j) * np + (n - 1 - c)] * dinv[c] : 0.0f;
    }
}

__global__ __launch_bounds__(256) void fold_identity_kernel(float* __restrict__ U, int64_t n) {
    for (int e = threadIdx.x; e < 32 * 32; e += 256) {
        const int64_t j = (int64_t)blockIdx.y * 32 + (e >> 5);
        const int64_t c = (int64_t)blockIdx.x * 32 + (e & 31);
        if (j < n && c < n) U[j * n + c] = (j == c) ? 1.0f : 0.0f;
    }
}

struct FoldLayout {
    int64_t np, nbk;
    size_t off_state, off_dinv, off_mi, off_a, off_x, total;
};

static FoldLayout fold_layout(int64_t n) {
    FoldLayout L{};
    L.np = round_up(n, NB);
    L.nbk = L.np / NB;
    size_t o = 0;
    L.off_state = o; o += align256(sizeof(FoldState));
    L.off_dinv = o; o += align256(sizeof(float) * (size_t)L.np);
    L.off_mi = o; o += align256(sizeof(float) * (size_t)(L.nbk * NB * NB));
    L.off_a = o; o += align256(sizeof(float) * (size_t)(L.np * L.np));
    L.off_x = o; o += align256(sizeof(float) * (size_t)(L.np * L.np));
    L.total = o;
    return L;
}

}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_fold_workspace_size(int64_t n) {
    if (n <= 0) return 0;
    return fold_layout(n).total;
}

extern "C" int gptq_fold(const float* H, int64_t n, int64_t ldh, double lambda, float* U,
                         float* hdiag, uint8_t* dead, void* workspace, size_t workspace_bytes,
                         void* stream, gptq_fold_report* report) {
    if (n <= 0 || ldh < n || !H || !U || !hdiag || !dead || !workspace) return GPTQ_EINVAL;
    if (n > (int64_t)1 << 20) return GPTQ_EINVAL;
    const FoldLayout L = fold_layout(n);
    if (workspace_bytes < L.total) return GPTQ_EWORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    char* ws = (char*)workspace;
    FoldState* state = (FoldState*)(ws + L.off_state);
    float* dinv = (float*)(ws + L.off_dinv);
    float* MI = (float*)(ws + L.off_mi);
    float* A = (float*)(ws + L.off_a);
    float* X = (float*)(ws + L.off_x);
    const int64_t np = L.np;
    const double n3 = (double)n * n * n;

    {
        ProfScope ps(FAM_FOLD_BUILD, st, 0.0, 8.0 * n);
        fold_prep_kernel<<<1, 1024, 0, st>>>(H, n, ldh, hdiag, dead, state);
    }
    GPTQ_HIP(hipGetLastError());

    double lam = (lambda > 0.0) ? lambda : 0.0;
    int attempts = 0;
    FoldState host{};
    bool degenerate = false;
    for (;;) {
        ++attempts;
        {
            ProfScope ps(FAM_FOLD_BUILD, st, 0.0, 4.0 * (double)n * n + 4.0 * (double)np * np / 2);
            fold_scale_kernel<<<(unsigned)((np + 255) / 256), 256, 0, st>>>(hdiag, dead, state, lam,
                                                                            n, np, dinv);
            fold_build_kernel<<<dim3((unsigned)(np / 32), (unsigned)(np / 32)), 256, 0, st>>>(
                H, ldh, dinv, dead, state, lam, A, n, np);
        }
        GPTQ_HIP(hipGetLastError());
        for (int64_t k = 0; k < L.nbk; ++k) {
            const int64_t kb = k * NB;
            const int64_t rest = np - kb - NB;
            {
                ProfScope ps(FAM_FOLD_DIAG, st, 2.0 * NB * NB * NB / 3.0, 0.0);
                fold_diag_kernel<<<1, 256, 0, st>>>(A, X, MI, np, (int)k, &state->flag);
            }
            const float* mik = MI + k * NB * NB;
            GemmBatch pb{};
            pb.p[0] = gemm_full(A + (kb + NB) * np + kb, np, mik, NB, 1, nullptr,
                                A + (kb + NB) * np + kb, np, (int)rest, NB, NB, 1.0f, 0);
            pb.p[1] = gemm_full(mik, NB, X + kb * np, np, 0, nullptr, X + kb * np, np, NB,
                                (int)kb, NB, 1.0f, 0);
            pb.nprob = 2;
            const int pt = pb.p[0].ntiles + pb.p[1].ntiles;
            if (pt > 0) {
                ProfScope ps(FAM_FOLD_PANEL, st, 2.0 * NB * NB * ((double)rest + kb), 0.0);
                gemm_kernel<1><<<pt, G_THREADS, 0, st>>>(pb, &state->flag);
            }
            if (rest > 0) {
                const float* P = A + (kb + NB) * np + kb;
                GemmBatch ub{};
                ub.p[0] = gemm_syrk_lower(P, np, A + (kb + NB) * np + kb + NB,
                                          A + (kb + NB) * np + kb + NB, np, (int)rest, NB, -1.0f, 1);
                ub.p[1] = gemm_full(P, np, X + kb * np, np, 0, X + (kb + NB) * np,
                                    X + (kb + NB) * np, np, (int)rest, (int)(kb + NB), NB, -1.0f, 1);
                ub.p[1].beta0_from_tn = (int)k;
                ub.nprob = 2;
                const double fl = (double)NB * rest * (rest + 1) + 2.0 * NB * rest * (kb + NB);
                ProfScope ps(FAM_FOLD_UPDATE, st, fl, 0.0);
                gemm_kernel<0><<<ub.p[0].ntiles + ub.p[1].ntiles, G_THREADS, 0, st>>>(ub,
                                                                                     &state->flag);
            }
            GPTQ_HIP(hipGetLastError());
        }
        GPTQ_HIP(hipMemcpyAsync(&host, state, sizeof(FoldState), hipMemcpyDeviceToHost, st));
        GPTQ_HIP(hipStreamSynchronize(st));
        if (host.flag == 0u) break;
        lam = (lam == 0.0) ? 1e-4 : lam * 10.0;
        if (lam > 10.0) {
            degenerate = true;
            break;
        }
    }
    const dim3 g((unsigned)((n + 31) / 32), (unsigned)((n + 31) / 32));
    if (degenerate) {
        fold_identity_kernel<<<g, 256, 0, st>>>(U, n);
    } else {
        ProfScope ps(FAM_FOLD_MAKEU, st, 0.0, 4.0 * (double)n * n);
        fold_make_u_kernel<<<g, 256, 0, st>>>(X, dinv, U, n, np);
    }
    GPTQ_HIP(hipGetLastError());
    if (report) {
        report->lambda_used = lam;
        report->base = host.base;
        report->damp = lam * host.base;
        report->attempts = attempts;
        report->n_dead = host.n_dead;
        report->degenerate = degenerate ? 1 : 0;
        report->reserved = 0;
    }
    (void)n3;
    return degenerate ? GPTQ_DEGENERATE : GPTQ_OK;
}
