// gram.hip -- device Hessian accumulation H += X^T X on gfx950.
//
// Source of the method: page "cortiq-cli 0.8.45 src/gptq.rs" (calibration: every window's
// layer inputs are added to a device Hessian by gram_add_dev, read back by gram_take; the test
// device_fold_and_sweep_match_host accumulates h[i][j] += x[r][i] x[r][j] over the rows r of an
// activation matrix x [t, n]) and page "cortiq-engine 0.8.41 src/gpu_wgpu/gptq_dev.rs" (the fold
// reads the Hessian's upper triangle, packed by poff).
//
// X is [t, n] row-major (one row per token, one column per input channel), so both operands of
// the product come from rows of X: A(i, k) = X[k][i], B(k, j) = X[k][j].  Each workgroup owns a
// 128 x 128 tile of H on or above the diagonal (diagonal tiles store j >= i only); the token axis
// is the K of the product, consumed 32 rows of X at a time through LDS (double buffered), with
// the last chunk zero-filled past t.  MFMA v_mfma_f32_32x32x2_f32, 4 waves of 64 x 64 per
// tile, the same register and lane layout as the GEMM of the fold.  H is dense or packed
// (HLayout): only the addressing of its tile differs, so both layouts receive the same sums.
#include "check.hpp"
#include "common.hpp"
#include "gemm_mfma.hpp"

namespace gptq {

struct GramArgs {
    float* H;
    const float* X;
    HLayout hl;
    int64_t ldx;
    int n, t;
    int T;       // ceil(n / 128) tile rows
    int tiles;   // T (T + 1) / 2 upper tiles
};

// Rows k0 .. k0+31 of X, columns col0 .. col0+127, as 4 float4 per thread (32 threads per
// 128-float row segment); zero past t rows or past n columns (n % 4 == 0).
__device__ __forceinline__ void gram_load(const GramArgs& g, int col0, int k0, int tid,
                                          f32x4 (&r)[4]) {
    const int jq = (tid & 31) * 4;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int k = k0 + (tid >> 5) + 8 * p;
        if (k < g.t && col0 + jq < g.n)
            r[p] = *reinterpret_cast<const f32x4*>(g.X + (int64_t)k * g.ldx + col0 + jq);
        else
            r[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

__global__ __launch_bounds__(G_THREADS) void gram_kernel(GramArgs g) {
    __shared__ __attribute__((aligned(16))) float As[2 * LDS_TILE];
    __shared__ __attribute__((aligned(16))) float Bs[2 * LDS_TILE];
    // Upper tile (tm, tn), tn >= tm: the transpose of lower tile (r, c), r >= c, taken in the
    // GEMM's super-tile order (both operands are column blocks of X, shared in L2 by the
    // workgroups of one super-tile).
    GemmProblem lp{};
    lp.lower = 1;
    lp.tiles_n = g.T;
    lp.ntiles = g.tiles;
    int r, c;
    tile_of(lp, xcd_order(blockIdx.x, g.tiles), r, c);
    const int tm = c, tn = r;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int i0 = tm * GT_M, j0 = tn * GT_N;

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][c][v] = 0.0f;

    f32x4 ra[4], rb[4];
    gram_load(g, i0, 0, tid, ra);
    gram_load(g, j0, 0, tid, rb);
    // The H tile, fetched now and consumed after the K loop (clamped inside the matrix; values
    // outside it or below the diagonal are never stored).
    float cv[2][2][16];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int i = min(i0 + wm * 64 + bi * 32 + 8 * (v >> 2) + 4 * h + (v & 3), g.n - 1);
                const int j = min(j0 + wn * 64 + bj * 32 + l32, g.n - 1);
                cv[bi][bj][v] = g.H[g.hl.at(i, j)];
            }
    store_krows_n(As, tid, ra);
    store_krows_n(Bs, tid, rb);
    __syncthreads();

    const int nchunk = (g.t + GT_K - 1) / GT_K;
    for (int c = 0; c < nchunk; ++c) {
        const int buf = c & 1;
        const float* as = As + buf * LDS_TILE;
        const float* bs = Bs + buf * LDS_TILE;
        const bool more = c + 1 < nchunk;
        if (more) {
            gram_load(g, i0, (c + 1) * GT_K, tid, ra);
            gram_load(g, j0, (c + 1) * GT_K, tid, rb);
        }
        // Keep the loads ahead of the chunk's MFMAs (the scheduler would sink them to their use).
        __builtin_amdgcn_sched_barrier(0);
        // Both operands are k-rows in LDS: element (k, col) at k * LDS_NROW + col.  Lane l feeds
        // MFMA row / column l % 32 and k-half h = l / 32; step s uses k = 16 h + s.
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 a4[2], b4[2];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = 16 * h + 4 * m + q;
#pragma unroll
                for (int bi = 0; bi < 2; ++bi) a4[bi][q] = as[k * LDS_NROW + wm * 64 + bi * 32 + l32];
#pragma unroll
                for (int bj = 0; bj < 2; ++bj) b4[bj][q] = bs[k * LDS_NROW + wn * 64 + bj * 32 + l32];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                    for (int bj = 0; bj < 2; ++bj)
                        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[bi][q], b4[bj][q],
                                                                          acc[bi][bj], 0, 0, 0);
        }
        if (more) {
            store_krows_n(As + (buf ^ 1) * LDS_TILE, tid, ra);
            store_krows_n(Bs + (buf ^ 1) * LDS_TILE, tid, rb);
        }
        __syncthreads();
    }

    const bool diag = tm == tn;
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int li = wm * 64 + bi * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                const int lj = wn * 64 + bj * 32 + l32;
                const int i = i0 + li, j = j0 + lj;
                if (i < g.n && j < g.n && (!diag || lj >= li))
                    g.H[g.hl.at(i, j)] = cv[bi][bj][v] + acc[bi][bj][v];
            }
}

}  // namespace gptq

using namespace gptq;

extern "C" int gptq_gram_add(float* H, int64_t n, int64_t ldh, const float* X, int64_t t,
                             int64_t ldx, void* stream) {
    if (!H || n <= 0 || t < 0 || !hessian_ld_ok(n, ldh) || ldx < n || n % 4 != 0) return GPTQ_EINVAL;
    if (n > ((int64_t)1 << 20) || t > ((int64_t)1 << 30)) return GPTQ_EINVAL;
    if (t == 0) return GPTQ_OK;  // X may be NULL
    if (!X || ldx % 4 != 0 || ((uintptr_t)X & 15u) != 0) return GPTQ_EINVAL;
    CheckScope check;
    check_buffer(H, sizeof(float) * (size_t)hessian_elems(n, ldh), "H");
    check_buffer(X, sizeof(float) * (size_t)((t - 1) * ldx + n), "X");
    hipStream_t st = (hipStream_t)stream;
    const int T = (int)((n + GT_M - 1) / GT_M);
    GramArgs g{H, X, HLayout{n, ldh}, ldx, (int)n, (int)t, T, T * (T + 1) / 2};
    // Reads stay inside t x n of X and n x n of H (loads past the edge are skipped or clamped).
    {
        ProfScope ps(FAM_GRAM, st, (double)n * (n + 1) * (double)t, 0.0);
        GPTQ_LAUNCH(st, "gram_add", (gram_kernel<<<(unsigned)g.tiles, G_THREADS, 0, st>>>(g)),
                    rd(X, ldx, t, n), hessian_span(H, n, ldh, false), hessian_span(H, n, ldh, true));
    }
    if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
    return check.finish();
}
