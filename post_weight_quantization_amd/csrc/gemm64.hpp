// gemm64.hpp -- f64 MFMA tile GEMM for gfx950: the dense contractions of the wide-precision
// fold (trailing Cholesky update, panel solve, triangular inverse).
//
//   C_out[i][j] = beta * C_in[i][j] + alpha * sum_k A[i][k] * B(k, j)
//
// The problem description follows the f32 GEMM (gemm_mfma.hpp): A row-major (k contiguous), B
// "T" (B(k, j) = Bm[j][k]) or "N" (B(k, j) = Bm[k][j]), lower (SYRK) grids, a diagonal mask,
// and a column cut-off for C_in.  The fold pads its matrices to whole tiles, so there are no
// bounds checks: the host rejects shapes that are not whole tiles.
//
// One workgroup of 256 threads (4 waves, 2 x 2) computes a TM x TN tile (128 x 128 for the bulk
// updates, 64 x 64 on the serial chain); each wave holds (TM/2) x (TN/2) as 16 x 16 accumulators
// of v_mfma_f64_16x16x4f64.  Lane l of that instruction feeds A(i = l % 16, k = l / 16) and
// B(k = l / 16, j = l % 16), and result slot v of lane l is D(l / 16 + 4 v, l % 16) (checked on
// the device).  K comes in chunks of 16 staged through LDS k-major (As[k][i], Bs[k][j]), so the
// 16 lanes that feed one MFMA row or column read 16 consecutive doubles; two buffers, one
// barrier per chunk.  An f64 MFMA takes many cycles per instruction, so the LDS traffic (two
// 8-byte reads per lane per MFMA group) is far from binding.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "check.hpp"
#include "common.hpp"
#include "gemm_mfma.hpp"

namespace gptq {

typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

constexpr int G64_K = 16;  // K chunk

struct GemmProblem64 {
    const double* A;
    const double* B;
    const double* Cin;
    double* Cout;
    int64_t lda, ldb, ldc;
    int M, N, K;       // whole tiles; K % 16 == 0
    int lower;         // 1: square tile grid, only tiles tn <= tm
    int mask_diag;     // 1: tiles with tm == tn store only i >= j
    int skip_upper;    // 1: tiles with tn > tm do nothing
    int tiles_n;       // tile columns (full grid) or tile rows = cols (lower)
    int ntiles;
    double alpha;
    int beta;          // 1: add C_in on tiles left of beta0_col
    int beta0_col;
};

struct GemmBatch64 {
    GemmProblem64 p[2];
    int nprob;
    int total;
};

// Global -> registers for one K chunk of a k-contiguous operand: R rows x 16 k as R/32 double2
// per thread (8 threads per 128-byte row segment).
template <int R>
__device__ __forceinline__ void g64_load_rows(const double* base, int64_t ld, int row0, int k0,
                                              int tid, f64x2 (&r)[R / 32]) {
    const int kk = (tid & 7) * 2;
#pragma unroll
    for (int p = 0; p < R / 32; ++p) {
        const int row = (tid >> 3) + 32 * p;
        r[p] = *reinterpret_cast<const f64x2*>(base + (int64_t)(row0 + row) * ld + k0 + kk);
    }
}

// ... stored k-major: lds[k][row], row stride LD.
template <int R, int LD>
__device__ __forceinline__ void g64_store_rows(double* lds, int tid, const f64x2 (&r)[R / 32]) {
    const int kk = (tid & 7) * 2;
#pragma unroll
    for (int p = 0; p < R / 32; ++p) {
        const int row = (tid >> 3) + 32 * p;
        lds[kk * LD + row] = r[p][0];
        lds[(kk + 1) * LD + row] = r[p][1];
    }
}

// An "N" operand: 16 k-rows x C columns (j contiguous) as C/32 double2 per thread.
template <int C>
__device__ __forceinline__ void g64_load_krows(const double* base, int64_t ld, int col0, int k0,
                                               int tid, f64x2 (&r)[C / 32]) {
    constexpr int TPR = C / 2;  // threads per k-row
    const int jq = (tid % TPR) * 2;
#pragma unroll
    for (int p = 0; p < C / 32; ++p) {
        const int kr = tid / TPR + (256 / TPR) * p;
        r[p] = *reinterpret_cast<const f64x2*>(base + (int64_t)(k0 + kr) * ld + col0 + jq);
    }
}

template <int C, int LD>
__device__ __forceinline__ void g64_store_krows(double* lds, int tid, const f64x2 (&r)[C / 32]) {
    constexpr int TPR = C / 2;
    const int jq = (tid % TPR) * 2;
#pragma unroll
    for (int p = 0; p < C / 32; ++p) {
        const int kr = tid / TPR + (256 / TPR) * p;
        *reinterpret_cast<f64x2*>(lds + kr * LD + jq) = r[p];
    }
}

template <int TM, int TN, bool TB>
__device__ __forceinline__ void gemm64_tile(const GemmProblem64& P, int tm, int tn, double* As,
                                            double* Bs) {
    constexpr int LDA_ = TM + 2, LDB_ = TN + 2;  // k-major row strides
    constexpr int WM = TM / 2, WN = TN / 2;     // one wave's sub-tile
    constexpr int BI = WM / 16, BJ = WN / 16;
    constexpr int SA = G64_K * LDA_, SB = G64_K * LDB_;  // doubles per buffer
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l16 = lane & 15, kq = lane >> 4;
    const int i0 = tm * TM, j0 = tn * TN;

    f64x4 acc[BI][BJ];
#pragma unroll
    for (int a = 0; a < BI; ++a)
#pragma unroll
        for (int b = 0; b < BJ; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};

    {
        f64x2 ra[TM / 32], rb[TN / 32];
        g64_load_rows<TM>(P.A, P.lda, i0, 0, tid, ra);
        if (TB) g64_load_rows<TN>(P.B, P.ldb, j0, 0, tid, rb);
        else g64_load_krows<TN>(P.B, P.ldb, j0, 0, tid, rb);
        g64_store_rows<TM, LDA_>(As, tid, ra);
        if (TB) g64_store_rows<TN, LDB_>(Bs, tid, rb);
        else g64_store_krows<TN, LDB_>(Bs, tid, rb);
    }
    __syncthreads();
    const int nchunk = P.K / G64_K;
    int buf = 0;
    for (int c = 0; c < nchunk; ++c) {
        const bool more = c + 1 < nchunk;
        f64x2 ra[TM / 32], rb[TN / 32];
        if (more) {
            const int k0 = (c + 1) * G64_K;
            g64_load_rows<TM>(P.A, P.lda, i0, k0, tid, ra);
            if (TB) g64_load_rows<TN>(P.B, P.ldb, j0, k0, tid, rb);
            else g64_load_krows<TN>(P.B, P.ldb, j0, k0, tid, rb);
        }
        __builtin_amdgcn_sched_barrier(0);
        const double* as = As + buf * SA;
        const double* bs = Bs + buf * SB;
#pragma unroll
        for (int s = 0; s < G64_K / 4; ++s) {
            const int k = 4 * s + kq;
            double a[BI], b[BJ];
#pragma unroll
            for (int bi = 0; bi < BI; ++bi) a[bi] = as[k * LDA_ + wm * WM + bi * 16 + l16];
#pragma unroll
            for (int bj = 0; bj < BJ; ++bj) b[bj] = bs[k * LDB_ + wn * WN + bj * 16 + l16];
#pragma unroll
            for (int bi = 0; bi < BI; ++bi)
#pragma unroll
                for (int bj = 0; bj < BJ; ++bj)
                    acc[bi][bj] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[bi], b[bj], acc[bi][bj], 0, 0, 0);
        }
        if (more) {
            const int nb = buf ^ 1;
            g64_store_rows<TM, LDA_>(As + nb * SA, tid, ra);
            if (TB) g64_store_rows<TN, LDB_>(Bs + nb * SB, tid, rb);
            else g64_store_krows<TN, LDB_>(Bs + nb * SB, tid, rb);
            __syncthreads();
            buf = nb;
        }
    }
    const bool use_c = P.beta && j0 < P.beta0_col;
    const bool diag_tile = P.mask_diag && tm == tn;
    const int64_t corner = (int64_t)i0 * P.ldc + j0;
#pragma unroll
    for (int bi = 0; bi < BI; ++bi)
#pragma unroll
        for (int bj = 0; bj < BJ; ++bj) {
            const int lj = wn * WN + bj * 16 + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int li = wm * WM + bi * 16 + kq + 4 * v;
                if (diag_tile && li < lj) continue;
                const int64_t off = corner + (int64_t)li * P.ldc + lj;
                const double base = use_c ? P.Cin[off] : 0.0;
                P.Cout[off] = base + P.alpha * acc[bi][bj][v];
            }
        }
}

// CHAIN: a product on the fold's serial chain, which raises its wave priority above the bulk
// updates' (CHAIN_PRIO).
template <int TM, int TN, bool TB0, bool TB1, bool CHAIN>
__global__ __launch_bounds__(256) void gemm64_kernel(GemmBatch64 batch, const unsigned* abort_flag) {
    if (abort_flag && __atomic_load_n(abort_flag, __ATOMIC_RELAXED)) return;
    if constexpr (CHAIN) __builtin_amdgcn_s_setprio(CHAIN_PRIO);
    __shared__ __attribute__((aligned(16))) double As[2 * G64_K * (TM + 2)];
    __shared__ __attribute__((aligned(16))) double Bs[2 * G64_K * (TN + 2)];
    int t = xcd_order(blockIdx.x, batch.total);
    int tm, tn;
    if (t < batch.p[0].ntiles) {
        tile_of(batch.p[0], t, tm, tn);
        if (batch.p[0].skip_upper && tn > tm) return;
        gemm64_tile<TM, TN, TB0>(batch.p[0], tm, tn, As, Bs);
    } else {
        t -= batch.p[0].ntiles;
        tile_of(batch.p[1], t, tm, tn);
        if (batch.p[1].skip_upper && tn > tm) return;
        gemm64_tile<TM, TN, TB1>(batch.p[1], tm, tn, As, Bs);
    }
}

// Host helpers ---------------------------------------------------------------------------------
inline GemmProblem64 gemm64_full(const double* A, int64_t lda, const double* B, int64_t ldb,
                                 const double* Cin, double* Cout, int64_t ldc, int M, int N, int K,
                                 double alpha, int beta) {
    GemmProblem64 p{};
    p.A = A; p.B = B; p.Cin = Cin; p.Cout = Cout;
    p.lda = lda; p.ldb = ldb; p.ldc = ldc;
    p.M = M; p.N = N; p.K = K;
    p.alpha = alpha; p.beta = beta; p.beta0_col = N;
    return p;  // tiles are counted by launch_gemm64 for the site's tile size
}

inline GemmProblem64 gemm64_syrk_lower(const double* A, int64_t lda, const double* Cin, double* Cout,
                                       int64_t ldc, int M, int K, double alpha, int beta) {
    GemmProblem64 p = gemm64_full(A, lda, A, lda, Cin, Cout, ldc, M, M, K, alpha, beta);
    p.lower = 1;
    p.mask_diag = 1;
    return p;
}

inline GemmProblem64 gemm64_none() {
    GemmProblem64 p{};
    p.tiles_n = 1;
    p.ntiles = 0;
    return p;
}

// Counts the tiles of p for TM x TN tiles; false when the shape is not whole tiles, K is not a
// multiple of 16, a lower grid or mask has non-square tiles, or ldc is out of range.
inline bool tile64(GemmProblem64& p, int TM, int TN) {
    if (p.M <= 0 || p.N <= 0) {
        p.tiles_n = 1;
        p.ntiles = 0;
        return true;
    }
    if (p.M % TM || p.N % TN || p.K <= 0 || p.K % G64_K || p.ldc <= 0) return false;
    if ((p.lower || p.mask_diag || p.skip_upper) && TM != TN) return false;
    if (p.lower) {
        const int T = p.M / TM;
        p.tiles_n = T;
        p.ntiles = T * (T + 1) / 2;
    } else {
        p.tiles_n = p.N / TN;
        p.ntiles = (p.M / TM) * p.tiles_n;
    }
    return true;
}

template <bool TB0, bool TB1>
inline int gemm64_spans(const GemmBatch64& b, Span* out) {
    int n = 0;
    for (int q = 0; q < b.nprob && q < 2; ++q) {
        const GemmProblem64& P = b.p[q];
        if (P.ntiles <= 0) continue;
        const bool TB = (q == 0) ? TB0 : TB1;
        out[n++] = rd(P.A, P.lda, P.M, P.K, 8);
        out[n++] = TB ? rd(P.B, P.ldb, P.N, P.K, 8) : rd(P.B, P.ldb, P.K, P.N, 8);
        if (P.beta && P.beta0_col > 0) out[n++] = rd(P.Cin, P.ldc, P.M, std::min(P.N, P.beta0_col), 8);
        out[n++] = wr(P.Cout, P.ldc, P.M, P.N, 8);
    }
    return n;
}

// Launch one batch of up to two problems with TM x TN tiles on stream s.
template <int TM, int TN, bool TB0, bool TB1, bool CHAIN = false>
inline int launch_gemm64(const char* name, hipStream_t s, GemmProblem64 p0, const GemmProblem64* p1,
                         const unsigned* flag) {
    GemmBatch64 b{};
    b.p[0] = p0;
    b.nprob = 1;
    if (p1) {
        b.p[1] = *p1;
        b.nprob = 2;
    }
    for (int q = 0; q < b.nprob; ++q)
        if (!tile64(b.p[q], TM, TN)) return GPTQ_EINVAL;
    b.total = b.p[0].ntiles + (b.nprob > 1 ? b.p[1].ntiles : 0);
    if (b.total <= 0) return GPTQ_OK;
    Span acc[8];
    const int na = gemm64_spans<TB0, TB1>(b, acc);
    const int rc = check_launch(name, s, acc, na);
    if (rc != GPTQ_OK) return rc;
    if (!dry_run()) gemm64_kernel<TM, TN, TB0, TB1, CHAIN><<<b.total, 256, 0, s>>>(b, flag);
    return GPTQ_OK;
}

}  // namespace gptq
