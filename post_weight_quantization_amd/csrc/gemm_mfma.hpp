// gemm_mfma.hpp -- f32 MFMA tile GEMM for gfx950: the dense contractions of the fold
// (trailing Cholesky update, panel solve, triangular inverse) and of the sweep (E * U).
//
//   C_out[i][j] = beta * C_in[i][j] + alpha * sum_k A[i][k] * B(k, j)
//
// A is row-major (k contiguous).  B is either "T" (B(k, j) = Bm[j][k], rows of Bm contiguous in
// k) or "N" (B(k, j) = Bm[k][j]); the layout is a compile-time parameter, as is the bounds
// checking (the fold's matrices are padded to whole tiles and need none).  One workgroup of
// 256 threads (4 waves, 2 x 2) computes a 128 x 128 tile; each wave holds a 64 x 64 sub-tile as
// 2 x 2 accumulators of v_mfma_f32_32x32x2_f32.  K is consumed in chunks of 32 staged through
// LDS, double buffered (one barrier per chunk); the C tile is fetched into registers during the
// last chunk so its latency hides behind that chunk's MFMAs.  A launch carries up to two independent
// problems so that the fold can update the Cholesky trailing matrix and the inverse in one
// grid.  Workgroups are dealt to the 8 XCDs round-robin by the hardware; tiles are renumbered
// so that each XCD works on a contiguous range (neighbouring tiles share operand rows in the
// XCD's L2).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "check.hpp"
#include "common.hpp"

namespace gptq {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// The global address space view of a generic pointer.  The kernels receive their matrices as
// generic pointers, and a load through one compiles to a FLAT load, which counts against the
// LDS counter as well as the memory counter: the wait for a chunk's LDS operands would then
// also wait for the next chunk's global loads issued just before, exposing their whole
// latency in front of every chunk's MFMAs.  Through these views the loads and stores are
// global_load / global_store, counted by the memory counter alone.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gmem(const T* p) {
    return (const __attribute__((address_space(1))) T*)p;
}
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gmem(T* p) {
    return (__attribute__((address_space(1))) T*)p;
}

constexpr int GT_M = 128;        // tile rows
constexpr int GT_N = 128;        // tile cols
constexpr int GT_K = 32;         // K chunk
constexpr int G_THREADS = 256;
constexpr int LDS_KROW = GT_K + 4;   // row stride (floats) of k-contiguous LDS tiles
constexpr int LDS_NROW = GT_N + 4;   // row stride of the j-contiguous ("N") B tile
constexpr int LDS_TILE = GT_M * LDS_KROW;  // >= GT_K * LDS_NROW
constexpr int NUM_XCD = 8;

struct GemmProblem {
    const float* A;
    const float* B;
    const float* Cin;
    float* Cout;
    int64_t lda, ldb, ldc;
    int M, N, K;          // K % 32 == 0; N % 4 == 0 for the N layout
    int lower;            // 1: square tile grid, only tiles tn <= tm; diagonal tiles store i >= j
    int mask_diag;        // 1: tiles with tm == tn store only i >= j (set whenever lower is)
    int skip_upper;       // 1: tiles with tn > tm do nothing (full grid over a lower-triangular C)
    int tiles_n;          // tile columns (full grid) or tile rows = cols (lower)
    int ntiles;
    float alpha;
    int beta;             // 1: add C_in (tiles that start left of beta0_col), 0: never read C_in
    int beta0_col;        // tiles whose first column is at or right of this ignore C_in
};

struct GemmBatch {
    GemmProblem p[2];
    int nprob;
    int total;            // p[0].ntiles + p[1].ntiles
    int64_t gs;           // a gang's slot stride in bytes (grid z = group); 0 outside a gang
    int small;            // 1: 64 x 64 tiles at a 128-tile site that allows them (GemmCfg::small)
};

// The problem of group blockIdx.z of a gang: every matrix and the flag lie in its slot.
__device__ __forceinline__ GemmProblem gang_problem(const GemmProblem& P0, int64_t gs) {
    GemmProblem P = P0;
    P.A = gang_ptr(P.A, gs);
    P.B = gang_ptr(P.B, gs);
    P.Cin = gang_ptr(P.Cin, gs);
    P.Cout = gang_ptr(P.Cout, gs);
    return P;
}

// Tile order.  Consecutive tile numbers walk super-tiles of GT_S x GT_S tiles (1024 x 1024
// elements of C), row by row inside a super-tile, so that the workgroups resident on one XCD at
// a time share the A rows and B columns of one super-tile in that XCD's L2 (about 2 GT_S
// operand blocks for GT_S^2 tiles, instead of a fresh B block for every tile of a tile row).
// Full grids: super-rows of GT_S tile rows (the last one may be shorter), each cut into
// super-tiles of GT_S tile columns (the last one may be narrower).  Lower grids (tn <= tm):
// super-row R holds R full super-tiles left of the diagonal and the diagonal one, a triangle.
constexpr int GT_S = 8;

// Tiles in the lower grid's super-rows 0 .. R-1 when those are all GT_S tile rows high.
__host__ __device__ __forceinline__ int lower_prefix(int R) {
    return GT_S * GT_S * (R * (R - 1) / 2) + R * (GT_S * (GT_S + 1) / 2);
}

// Row r and column c of entry u of a lower triangle enumerated row by row (c <= r).
__host__ __device__ __forceinline__ void tri_of(int u, int& r, int& c) {
    r = (int)((sqrtf(8.0f * (float)u + 1.0f) - 1.0f) * 0.5f);
    while ((r + 1) * (r + 2) / 2 <= u) ++r;
    while (r * (r + 1) / 2 > u) --r;
    c = u - r * (r + 1) / 2;
}

// PROB is any problem type with the fields lower, tiles_n and ntiles (the f32 and f64 GEMMs).
template <class PROB>
__host__ __device__ __forceinline__ void tile_of(const PROB& P, int t, int& tm, int& tn) {
    if (P.lower) {
        const int T = P.tiles_n;
        const int RB = (T + GT_S - 1) / GT_S;
        int R = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) / (2.0f * GT_S));
        R = R < 0 ? 0 : (R > RB - 1 ? RB - 1 : R);
        while (R + 1 <= RB - 1 && lower_prefix(R + 1) <= t) ++R;
        while (R > 0 && lower_prefix(R) > t) --R;
        const int u = t - lower_prefix(R);
        const int m = (T - R * GT_S < GT_S) ? T - R * GT_S : GT_S;  // tile rows in super-row R
        if (u < R * m * GT_S) {
            const int C = u / (m * GT_S), v = u - C * m * GT_S;
            tm = R * GT_S + v / GT_S;
            tn = C * GT_S + v % GT_S;
        } else {
            int r, c;
            tri_of(u - R * m * GT_S, r, c);
            tm = R * GT_S + r;
            tn = R * GT_S + c;
        }
    } else {
        const int TN = P.tiles_n, TM = P.ntiles / P.tiles_n;
        const int R = t / (GT_S * TN), u = t - R * GT_S * TN;
        const int m = (TM - R * GT_S < GT_S) ? TM - R * GT_S : GT_S;
        const int C = u / (m * GT_S), v = u - C * m * GT_S;
        const int w = (TN - C * GT_S < GT_S) ? TN - C * GT_S : GT_S;
        tm = R * GT_S + v / w;
        tn = C * GT_S + v % w;
    }
}

// Workgroup b of group z of a gang (grid z): the hardware deals the workgroups of a launch to
// the XCDs in launch order, so group z's slice starts at XCD (total z) % 8.  Rotating the
// slice's numbering by that much keeps xcd_order's ranges on their XCDs; a rotation mod total
// is a bijection of [0, total) for every z.
__host__ __device__ __forceinline__ int gang_block(int b, int z, int total) {
    if (z == 0) return b;
    return (int)(((int64_t)b + ((int64_t)total * z) % NUM_XCD) % total);
}

// Bijective renumbering: the hardware sends workgroup b to XCD b % 8; give XCD x the
// contiguous tile range [o_x, o_x + c_x).
__host__ __device__ __forceinline__ int xcd_order(int b, int total) {
    const int q = total / NUM_XCD, r = total % NUM_XCD;
    const int x = b % NUM_XCD, i = b / NUM_XCD;
    return x * q + (x < r ? x : r) + i;
}

// Global -> registers for one K chunk.  A (and "T" B): 128 rows x 32 k as 4 float4 per thread,
// 8 threads per 128-byte row segment.  "N" B: 32 k-rows x 128 j as 4 float4 per thread.
template <bool CHK>
__device__ __forceinline__ void load_rows_k(const float* base, int64_t ld, int row0, int nrows,
                                            int k0, int tid, f32x4 (&r)[4]) {
    const int kq = (tid & 7) * 4;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int row = (tid >> 3) + 32 * p;
        const float* src = base + (int64_t)(row0 + row) * ld + k0 + kq;
        if (!CHK || row0 + row < nrows) r[p] = *gmem(reinterpret_cast<const f32x4*>(src));
        else r[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

__device__ __forceinline__ void store_rows_k(float* lds, int tid, const f32x4 (&r)[4]) {
    const int kq = (tid & 7) * 4;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int row = (tid >> 3) + 32 * p;
        *reinterpret_cast<f32x4*>(lds + row * LDS_KROW + kq) = r[p];
    }
}

template <bool CHK>
__device__ __forceinline__ void load_krows_n(const float* base, int64_t ld, int col0, int ncols,
                                             int k0, int tid, f32x4 (&r)[4]) {
    const int jq = (tid & 31) * 4;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int kr = (tid >> 5) + 8 * p;
        const float* src = base + (int64_t)(k0 + kr) * ld + col0 + jq;
        if (!CHK || col0 + jq < ncols) r[p] = *gmem(reinterpret_cast<const f32x4*>(src));
        else r[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

__device__ __forceinline__ void store_krows_n(float* lds, int tid, const f32x4 (&r)[4]) {
    const int jq = (tid & 31) * 4;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int kr = (tid >> 5) + 8 * p;
        *reinterpret_cast<f32x4*>(lds + kr * LDS_NROW + jq) = r[p];
    }
}

template <bool TB, bool CHK>
__device__ __forceinline__ void load_b(const GemmProblem& P, int j0, int k0, int tid,
                                       f32x4 (&r)[4]) {
    if (TB) load_rows_k<CHK>(P.B, P.ldb, j0, P.N, k0, tid, r);
    else load_krows_n<CHK>(P.B, P.ldb, j0, P.N, k0, tid, r);
}

template <bool TB>
__device__ __forceinline__ void store_b(float* lds, int tid, const f32x4 (&r)[4]) {
    if (TB) store_rows_k(lds, tid, r);
    else store_krows_n(lds, tid, r);
}

// The MFMAs of one K chunk staged in LDS (as, bs): lane l of a wave feeds MFMA row/col (l % 32)
// and k-half h = l / 32; in step s of the chunk the k index is 16 h + s for both operands, so
// the two lane halves together cover the chunk's 32 k values over 16 steps.
template <bool TB>
__device__ __forceinline__ void chunk_mfma(const float* as, const float* bs, int wm, int wn,
                                           int l32, int h, f32x16 (&acc)[2][2]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        f32x4 a4[2], b4[2];
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
            a4[bi] = *reinterpret_cast<const f32x4*>(
                as + (wm * 64 + bi * 32 + l32) * LDS_KROW + 16 * h + 4 * m);
        if (TB) {
#pragma unroll
            for (int bj = 0; bj < 2; ++bj)
                b4[bj] = *reinterpret_cast<const f32x4*>(
                    bs + (wn * 64 + bj * 32 + l32) * LDS_KROW + 16 * h + 4 * m);
        } else {
#pragma unroll
            for (int bj = 0; bj < 2; ++bj)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    b4[bj][q] = bs[(16 * h + 4 * m + q) * LDS_NROW + wn * 64 + bj * 32 + l32];
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
}

// One 128 x 128 tile of problem P.  K goes through LDS in chunks of 32, NBUF buffers deep: with
// two, the next chunk is stored into the other buffer while this one feeds the MFMAs (one
// barrier per chunk); with one, after a second barrier.  The next chunk's global loads are
// issued before this chunk's MFMAs either way.  The C tile is fetched during the last chunk, so
// its latency hides behind that chunk's MFMAs and its registers are not held through the loop.
// Output slot v of a 32 x 32 accumulator holds row 8 (v / 4) + 4 h + v % 4, column l % 32.
template <bool TB, bool CHK, int NBUF>
__device__ __forceinline__ void gemm_tile(const GemmProblem& P, int tm, int tn, float* As,
                                          float* Bs) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int i0 = tm * GT_M, j0 = tn * GT_N;

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
    const bool use_c = P.beta && tn * GT_N < P.beta0_col;
    const bool diag_tile = P.mask_diag && tm == tn;
    {
        f32x4 ra[4], rb[4];
        load_rows_k<CHK>(P.A, P.lda, i0, P.M, 0, tid, ra);
        load_b<TB, CHK>(P, j0, 0, tid, rb);
        store_rows_k(As, tid, ra);
        store_b<TB>(Bs, tid, rb);
    }
    __syncthreads();
    const int nchunk = P.K / GT_K;
    int buf = 0;
    for (int c = 0; c + 1 < nchunk; ++c) {
        f32x4 ra[4], rb[4];
        const int k0 = (c + 1) * GT_K;
        load_rows_k<CHK>(P.A, P.lda, i0, P.M, k0, tid, ra);
        load_b<TB, CHK>(P, j0, k0, tid, rb);
        // Keep the loads here, ahead of the chunk's MFMAs: left to itself the scheduler sinks
        // them to just before the LDS stores that use them, exposing their whole latency.
        __builtin_amdgcn_sched_barrier(0);
        chunk_mfma<TB>(As + buf * LDS_TILE, Bs + buf * LDS_TILE, wm, wn, l32, h, acc);
        if (NBUF == 1) __syncthreads();
        const int nb = NBUF == 2 ? (buf ^ 1) : 0;
        store_rows_k(As + nb * LDS_TILE, tid, ra);
        store_b<TB>(Bs + nb * LDS_TILE, tid, rb);
        __syncthreads();
        buf = nb;
    }
    // C addresses: the tile's corner as one 64-bit offset, each element as a 32-bit offset from
    // it (the host bounds ldc, so 128 rows of C fit), so no element needs a 64-bit multiply.
    const int64_t corner = (int64_t)i0 * P.ldc + j0;
    const int ldc = (int)P.ldc;
    float cv[2][2][16];
    if (use_c) {
        const float* cin = P.Cin + corner;
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < 2; ++bj) {
                const float* cp = cin + (wm * 64 + bi * 32 + 4 * h) * ldc + wn * 64 + bj * 32 + l32;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    if (CHK) {
                        // Unconditional load, clamped inside the matrix; masked values are
                        // never stored.
                        const int li = min(wm * 64 + bi * 32 + 8 * (v >> 2) + 4 * h + (v & 3),
                                           P.M - 1 - i0);
                        const int lj = min(wn * 64 + bj * 32 + l32, P.N - 1 - j0);
                        cv[bi][bj][v] = gmem(cin)[li * ldc + lj];
                    } else {
                        // Rows 0-3, 8-11, 16-19, 24-27 (+ 4h) of the block, by pointer steps.
                        cv[bi][bj][v] = *gmem(cp);
                        cp += ((v & 3) == 3) ? 5 * ldc : ldc;
                    }
                }
            }
    }
    chunk_mfma<TB>(As + buf * LDS_TILE, Bs + buf * LDS_TILE, wm, wn, l32, h, acc);
    float* cout = P.Cout + corner;
    if (!CHK && !diag_tile) {
        // Every element of the tile is stored (the common case): no per-element conditions.
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < 2; ++bj) {
                // Walk the block's rows 0-3, 8-11, 16-19, 24-27 (+ 4h) with a pointer.
                float* cp = cout + (wm * 64 + bi * 32 + 4 * h) * ldc + wn * 64 + bj * 32 + l32;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float base = use_c ? cv[bi][bj][v] : 0.0f;
                    *gmem(cp) = base + P.alpha * acc[bi][bj][v];
                    cp += ((v & 3) == 3) ? 5 * ldc : ldc;
                }
            }
        return;
    }
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
            const int lj = wn * 64 + bj * 32 + l32;
            float* cp = cout + (wm * 64 + bi * 32 + 4 * h) * ldc + lj;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int li = wm * 64 + bi * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                if ((!CHK || (i0 + li < P.M && j0 + lj < P.N)) && (!diag_tile || li >= lj)) {
                    const float base = use_c ? cv[bi][bj][v] : 0.0f;
                    *gmem(cp) = base + P.alpha * acc[bi][bj][v];
                }
                cp += ((v & 3) == 3) ? 5 * ldc : ldc;
            }
        }
}

// A 64 x 64 tile, for the small products on the serial chains: four times the workgroups of
// the 128 tile for the same product, each with a quarter of the MFMAs, so a launch that fills
// only part of the GPU finishes sooner.  Each of the 4 waves computes 32 x 32 with one
// accumulator; K chunks of 32 through LDS as in the 128 tile ("T" operands as k-contiguous rows
// of stride LDS_KROW, the "N" B as k-rows of stride LDS_NROW64).
constexpr int LDS_NROW64 = 64 + 4;
constexpr int LDS_TILE64 = 64 * LDS_KROW;  // >= GT_K * LDS_NROW64

template <bool CHK>
__device__ __forceinline__ void load_rows_k64(const float* base, int64_t ld, int row0, int nrows,
                                              int k0, int tid, f32x4 (&r)[2]) {
    const int kq = (tid & 7) * 4;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int row = (tid >> 3) + 32 * p;
        if (!CHK || row0 + row < nrows)
            r[p] = *gmem(reinterpret_cast<const f32x4*>(base + (int64_t)(row0 + row) * ld + k0 + kq));
        else
            r[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

__device__ __forceinline__ void store_rows_k64(float* lds, int tid, const f32x4 (&r)[2]) {
    const int kq = (tid & 7) * 4;
#pragma unroll
    for (int p = 0; p < 2; ++p)
        *reinterpret_cast<f32x4*>(lds + ((tid >> 3) + 32 * p) * LDS_KROW + kq) = r[p];
}

template <bool CHK>
__device__ __forceinline__ void load_krows_n64(const float* base, int64_t ld, int col0, int ncols,
                                               int k0, int tid, f32x4 (&r)[2]) {
    const int jq = (tid & 15) * 4;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int kr = (tid >> 4) + 16 * p;
        if (!CHK || col0 + jq < ncols)
            r[p] = *gmem(reinterpret_cast<const f32x4*>(base + (int64_t)(k0 + kr) * ld + col0 + jq));
        else
            r[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

__device__ __forceinline__ void store_krows_n64(float* lds, int tid, const f32x4 (&r)[2]) {
    const int jq = (tid & 15) * 4;
#pragma unroll
    for (int p = 0; p < 2; ++p)
        *reinterpret_cast<f32x4*>(lds + ((tid >> 4) + 16 * p) * LDS_NROW64 + jq) = r[p];
}

// B staging of the small tiles: TN = 64 uses the helpers above, TN = 128 those of the 128 tile.
template <bool TB, bool CHK, int TN>
__device__ __forceinline__ void load_b_small(const GemmProblem& P, int j0, int k0, int tid,
                                             f32x4 (&r)[TN / 32]) {
    if constexpr (TN == 64) {
        if (TB) load_rows_k64<CHK>(P.B, P.ldb, j0, P.N, k0, tid, r);
        else load_krows_n64<CHK>(P.B, P.ldb, j0, P.N, k0, tid, r);
    } else {
        if (TB) load_rows_k<CHK>(P.B, P.ldb, j0, P.N, k0, tid, r);
        else load_krows_n<CHK>(P.B, P.ldb, j0, P.N, k0, tid, r);
    }
}

template <bool TB, int TN>
__device__ __forceinline__ void store_b_small(float* lds, int tid, const f32x4 (&r)[TN / 32]) {
    if constexpr (TN == 64) {
        if (TB) store_rows_k64(lds, tid, r);
        else store_krows_n64(lds, tid, r);
    } else {
        if (TB) store_rows_k(lds, tid, r);
        else store_krows_n(lds, tid, r);
    }
}

// Wave (wm, wn) of a 64 x TN tile: rows wm*32 .. +32, columns wn*TN/2 .. +TN/2 as TN/64
// accumulators of 32 x 32.
template <bool TB, int TN>
__device__ __forceinline__ void chunk_mfma_small(const float* as, const float* bs, int wm, int wn,
                                                 int l32, int h, f32x16 (&acc)[TN / 64]) {
    constexpr int NA = TN / 64, NROW = TN + 4;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(as + (wm * 32 + l32) * LDS_KROW + 16 * h + 4 * m);
        f32x4 b4[NA];
#pragma unroll
        for (int bj = 0; bj < NA; ++bj) {
            const int col = wn * (TN / 2) + bj * 32 + l32;
            if (TB) {
                b4[bj] = *reinterpret_cast<const f32x4*>(bs + col * LDS_KROW + 16 * h + 4 * m);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) b4[bj][q] = bs[(16 * h + 4 * m + q) * NROW + col];
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int bj = 0; bj < NA; ++bj)
                acc[bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[q], b4[bj][q], acc[bj], 0, 0, 0);
    }
}

// A 64 x TN tile (TN = 64 or 128), the same K loop as the 128 tile.
template <bool TB, bool CHK, int TN>
__device__ __forceinline__ void gemm_tile_small(const GemmProblem& P, int tm, int tn, float* As,
                                                float* Bs) {
    constexpr int NA = TN / 64, NB_ = TN / 32;
    constexpr int BT = TN == 64 ? LDS_TILE64 : LDS_TILE;  // floats per B buffer
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int i0 = tm * 64, j0 = tn * TN;
    f32x16 acc[NA];
#pragma unroll
    for (int bj = 0; bj < NA; ++bj)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[bj][v] = 0.0f;
    const bool use_c = P.beta && j0 < P.beta0_col;
    const bool diag_tile = P.mask_diag && tm == tn;  // square tiles only (host-checked)
    {
        f32x4 ra[2], rb[NB_];
        load_rows_k64<CHK>(P.A, P.lda, i0, P.M, 0, tid, ra);
        load_b_small<TB, CHK, TN>(P, j0, 0, tid, rb);
        store_rows_k64(As, tid, ra);
        store_b_small<TB, TN>(Bs, tid, rb);
    }
    __syncthreads();
    const int nchunk = P.K / GT_K;
    int buf = 0;
    for (int c = 0; c + 1 < nchunk; ++c) {
        f32x4 ra[2], rb[NB_];
        const int k0 = (c + 1) * GT_K;
        load_rows_k64<CHK>(P.A, P.lda, i0, P.M, k0, tid, ra);
        load_b_small<TB, CHK, TN>(P, j0, k0, tid, rb);
        __builtin_amdgcn_sched_barrier(0);
        chunk_mfma_small<TB, TN>(As + buf * LDS_TILE64, Bs + buf * BT, wm, wn, l32, h, acc);
        const int nb = buf ^ 1;
        store_rows_k64(As + nb * LDS_TILE64, tid, ra);
        store_b_small<TB, TN>(Bs + nb * BT, tid, rb);
        __syncthreads();
        buf = nb;
    }
    // C addresses as in the 128 tile: a 64-bit corner and 32-bit element offsets.
    const int64_t corner = (int64_t)i0 * P.ldc + j0;
    const int ldc = (int)P.ldc;
    float cv[NA][16];
    if (use_c) {
        const float* cin = P.Cin + corner;
#pragma unroll
        for (int bj = 0; bj < NA; ++bj) {
            const float* cp = cin + (wm * 32 + 4 * h) * ldc + wn * (TN / 2) + bj * 32 + l32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                if (CHK) {
                    const int li = min(wm * 32 + 8 * (v >> 2) + 4 * h + (v & 3), P.M - 1 - i0);
                    const int lj = min(wn * (TN / 2) + bj * 32 + l32, P.N - 1 - j0);
                    cv[bj][v] = gmem(cin)[li * ldc + lj];
                } else {
                    cv[bj][v] = *gmem(cp);
                    cp += ((v & 3) == 3) ? 5 * ldc : ldc;
                }
            }
        }
    }
    chunk_mfma_small<TB, TN>(As + buf * LDS_TILE64, Bs + buf * BT, wm, wn, l32, h, acc);
    float* cout = P.Cout + corner;
    if (!CHK && !diag_tile) {
#pragma unroll
        for (int bj = 0; bj < NA; ++bj) {
            float* cp = cout + (wm * 32 + 4 * h) * ldc + wn * (TN / 2) + bj * 32 + l32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float base = use_c ? cv[bj][v] : 0.0f;
                *gmem(cp) = base + P.alpha * acc[bj][v];
                cp += ((v & 3) == 3) ? 5 * ldc : ldc;
            }
        }
        return;
    }
#pragma unroll
    for (int bj = 0; bj < NA; ++bj) {
        const int lj = wn * (TN / 2) + bj * 32 + l32;
        float* cp = cout + (wm * 32 + 4 * h) * ldc + lj;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int li = wm * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
            if ((!CHK || (i0 + li < P.M && j0 + lj < P.N)) && (!diag_tile || li >= lj)) {
                const float base = use_c ? cv[bj][v] : 0.0f;
                *gmem(cp) = base + P.alpha * acc[bj][v];
            }
            cp += ((v & 3) == 3) ? 5 * ldc : ldc;
        }
    }
}

// LDS buffers, waves per SIMD and tile size for a launch site.  The two bulk updates (the fold's,
// 0, and the sweep's, 2) stage K through one LDS buffer (a second barrier per chunk): their
// registers already hold them to two workgroups per CU, and the LDS this frees lets the serial
// chains' kernels run beside them instead of waiting for a workgroup to finish.  Every other
// site uses two buffers.
// The products on the serial chains that do not fill the GPU with 128 tiles take 64 x 64 tiles:
// the fold's look-ahead (3) and update inside a panel (4), the inverse's diagonal-block steps
// (5) and panel rows of X (9), the sweep's update inside a panel (6) and look-ahead (7).  The
// fold's panel solve (1) takes 64 x 128 tiles: it works in place on a 128-column block, and a
// tile row 128 columns wide is what makes that safe (each workgroup reads all the columns it
// overwrites before it writes).
// prio: the wave priority (s_setprio) of the site's waves.  The chains' products raise theirs
// above the bulk updates' (0), so that on a SIMD shared with bulk waves their instructions are
// issued first: the bulk updates hide behind the chains, not the other way round.
template <int TAG>
struct GemmCfg {
    static constexpr int nbuf = 2;
    static constexpr int waves = 2;
    static constexpr int tile = 128;    // tile rows
    static constexpr int tile_n = 128;  // tile columns
    static constexpr int prio = 0;
    static constexpr bool small = false;  // a launch may ask for 64 x 64 tiles (GemmBatch::small)
};
#define GPTQ_CHAIN_CFG(TAG, TN)                                                                     \
    template <> struct GemmCfg<TAG> {                                                               \
        static constexpr int nbuf = 2, waves = 4, tile = 64, tile_n = TN, prio = CHAIN_PRIO;       \
        static constexpr bool small = false;                                                        \
    }
GPTQ_CHAIN_CFG(1, 128);
GPTQ_CHAIN_CFG(3, 64);
GPTQ_CHAIN_CFG(4, 64);
GPTQ_CHAIN_CFG(5, 64);
GPTQ_CHAIN_CFG(6, 64);
GPTQ_CHAIN_CFG(7, 64);
GPTQ_CHAIN_CFG(9, 64);
#undef GPTQ_CHAIN_CFG
// The fold's bulk updates take 64 x 64 tiles for launches of less than about one and a half
// rounds of 128-tiles (the last SYRKs and the first and last inverse updates), where one
// 128-tile's latency sets the launch's time: four times the workgroups, a quarter of the work
// each, the same k order per element.
template <> struct GemmCfg<0> {
    static constexpr int nbuf = 1, waves = 2, tile = 128, tile_n = 128, prio = 0;
    static constexpr bool small = true;
};
template <> struct GemmCfg<2> {
    static constexpr int nbuf = 1, waves = 2, tile = 128, tile_n = 128, prio = 0;
    static constexpr bool small = true;
};

// TAG only separates the launch sites in profiles (one symbol per use).  TB0 / TB1: B layout
// of problems 0 and 1; CHK: bounds checks on M and N.
template <int TAG, bool TB0, bool TB1, bool CHK>
__global__ __launch_bounds__(G_THREADS) __attribute__((amdgpu_waves_per_eu(GemmCfg<TAG>::waves, GemmCfg<TAG>::waves)))
void gemm_kernel(GemmBatch batch, const unsigned* abort_flag) {
    if (abort_flag && __atomic_load_n(gang_ptr(abort_flag, batch.gs), __ATOMIC_RELAXED)) return;
    if constexpr (GemmCfg<TAG>::prio > 0) __builtin_amdgcn_s_setprio(GemmCfg<TAG>::prio);
    constexpr int NBUF = GemmCfg<TAG>::nbuf;
    constexpr int TILE = GemmCfg<TAG>::tile, TILE_N = GemmCfg<TAG>::tile_n;
    static_assert(TILE == 128 ? TILE_N == 128 : (TILE == 64 && (TILE_N == 64 || TILE_N == 128)),
                  "tile shapes: 128 x 128, 64 x 64, 64 x 128");
    constexpr int LA = TILE == 128 ? NBUF * LDS_TILE : 2 * LDS_TILE64;
    constexpr int LB = TILE == 128 ? NBUF * LDS_TILE : 2 * (TILE_N == 64 ? LDS_TILE64 : LDS_TILE);
    static_assert(!GemmCfg<TAG>::small || (LA >= 2 * LDS_TILE64 && LB >= 2 * LDS_TILE64),
                  "the 64-tile path stages two buffers of each operand");
    __shared__ __attribute__((aligned(16))) float As[LA];
    __shared__ __attribute__((aligned(16))) float Bs[LB];
    int t = xcd_order(gang_block((int)blockIdx.x, (int)blockIdx.z, batch.total), batch.total);
    int tm, tn;
    if (t < batch.p[0].ntiles) {
        tile_of(batch.p[0], t, tm, tn);
        if (batch.p[0].skip_upper && tn > tm) return;
        const GemmProblem P = gang_problem(batch.p[0], batch.gs);
        if constexpr (GemmCfg<TAG>::small) {
            if (batch.small) {
                gemm_tile_small<TB0, CHK, 64>(P, tm, tn, As, Bs);
                return;
            }
        }
        if (TILE == 128) gemm_tile<TB0, CHK, NBUF>(P, tm, tn, As, Bs);
        else gemm_tile_small<TB0, CHK, TILE_N>(P, tm, tn, As, Bs);
    } else {
        t -= batch.p[0].ntiles;
        tile_of(batch.p[1], t, tm, tn);
        if (batch.p[1].skip_upper && tn > tm) return;
        const GemmProblem P = gang_problem(batch.p[1], batch.gs);
        if constexpr (GemmCfg<TAG>::small) {
            if (batch.small) {
                gemm_tile_small<TB1, CHK, 64>(P, tm, tn, As, Bs);
                return;
            }
        }
        if (TILE == 128) gemm_tile<TB1, CHK, NBUF>(P, tm, tn, As, Bs);
        else gemm_tile_small<TB1, CHK, TILE_N>(P, tm, tn, As, Bs);
    }
}

// Host helpers ---------------------------------------------------------------------------------
inline GemmProblem gemm_full(const float* A, int64_t lda, const float* B, int64_t ldb,
                             const float* Cin, float* Cout, int64_t ldc, int M, int N, int K,
                             float alpha, int beta) {
    GemmProblem p{};
    p.A = A; p.B = B; p.Cin = Cin; p.Cout = Cout;
    p.lda = lda; p.ldb = ldb; p.ldc = ldc;
    p.M = M; p.N = N; p.K = K;
    p.lower = 0;
    p.mask_diag = 0;
    p.skip_upper = 0;
    p.tiles_n = (N + GT_N - 1) / GT_N;
    p.ntiles = ((M + GT_M - 1) / GT_M) * p.tiles_n;
    p.alpha = alpha; p.beta = beta; p.beta0_col = N;
    if (M <= 0 || N <= 0) p.ntiles = 0;
    return p;
}

// C (M x M, lower tiles) = beta*C + alpha * A A^T with A M x K (k contiguous): use TB = true.
inline GemmProblem gemm_syrk_lower(const float* A, int64_t lda, const float* Cin, float* Cout,
                                   int64_t ldc, int M, int K, float alpha, int beta) {
    GemmProblem p = gemm_full(A, lda, A, lda, Cin, Cout, ldc, M, M, K, alpha, beta);
    const int T = (M + GT_M - 1) / GT_M;
    p.lower = 1;
    p.mask_diag = 1;
    p.tiles_n = T;
    p.ntiles = M > 0 ? T * (T + 1) / 2 : 0;
    return p;
}

// The tile grid of a problem for tiles of tm x tn (the helpers above count 128-tiles).
// Returns false for a lower grid or a diagonal mask with non-square tiles.
inline bool retile(GemmProblem& p, int tm, int tn) {
    if (p.ntiles <= 0) return true;
    if ((p.lower || p.mask_diag || p.skip_upper) && tm != tn) return false;
    if (p.lower) {
        const int T = (p.M + tm - 1) / tm;
        p.tiles_n = T;
        p.ntiles = T * (T + 1) / 2;
    } else {
        p.tiles_n = (p.N + tn - 1) / tn;
        p.ntiles = ((p.M + tm - 1) / tm) * p.tiles_n;
    }
    return true;
}

// A problem with no tiles: fills the first slot of a batch whose only problem needs the
// second slot's B layout.
inline GemmProblem gemm_none() {
    GemmProblem p{};
    p.tiles_n = 1;
    p.ntiles = 0;
    return p;
}

inline GemmBatch gemm_batch(const GemmProblem& a, const GemmProblem* b) {
    GemmBatch g{};
    g.p[0] = a;
    g.nprob = 1;
    if (b) {
        g.p[1] = *b;
        g.nprob = 2;
    }
    g.total = g.p[0].ntiles + (b ? g.p[1].ntiles : 0);
    return g;
}

// Memory one batch touches, as spans for the schedule checker: per problem A, B, C_in (when
// read) and C_out, over whole tiles unless the launch checks bounds.  Returns the span count,
// or -1 when a problem breaks the kernel's shape rules (K a multiple of 32; with bounds checks
// and the "N" layout, N a multiple of 4; 0 < ldc <= 2^23).
template <bool TB0, bool TB1, bool CHK>
inline int gemm_spans(const GemmBatch& b, Span* out, int tile, int tile_n) {
    int n = 0;
    for (int q = 0; q < b.nprob && q < 2; ++q) {
        const GemmProblem& P = b.p[q];
        if (P.ntiles <= 0) continue;
        const bool TB = (q == 0) ? TB0 : TB1;
        // ldc is bounded so that an element's offset from its tile's corner fits in 32 bits.
        if (P.K <= 0 || P.K % GT_K != 0 || (CHK && !TB && P.N % 4 != 0) || P.tiles_n <= 0 ||
            P.ldc <= 0 || P.ldc > ((int64_t)1 << 23))
            return -1;
        const int64_t tm = P.lower ? P.tiles_n : P.ntiles / P.tiles_n;
        const int64_t rows = CHK ? P.M : tm * tile;
        const int64_t cols = CHK ? P.N : (int64_t)P.tiles_n * tile_n;
        out[n++] = rd(P.A, P.lda, rows, P.K);
        out[n++] = TB ? rd(P.B, P.ldb, cols, P.K) : rd(P.B, P.ldb, P.K, cols);
        if (P.beta && P.beta0_col > 0) {
            // Tiles starting left of beta0_col read C_in over their whole width.
            const int64_t c_in = ((int64_t)P.beta0_col + tile_n - 1) / tile_n * tile_n;
            out[n++] = rd(P.Cin, P.ldc, rows, cols < c_in ? cols : c_in);
        }
        out[n++] = wr(P.Cout, P.ldc, rows, cols);
    }
    return n;
}

// Launch one batch on stream s with `grid` workgroups (normally batch.total), after checking
// its shape rules (GPTQ_EINVAL) and recording its accesses (check mode).
template <int TAG, bool TB0, bool TB1, bool CHK>
inline int launch_gemm(const char* name, hipStream_t s, const GemmBatch& b0, const unsigned* flag) {
    GemmBatch b = b0;
    if (b.small && !GemmCfg<TAG>::small) return GPTQ_EINVAL;
    const int TILE = b.small ? 64 : GemmCfg<TAG>::tile, TILE_N = b.small ? 64 : GemmCfg<TAG>::tile_n;
    for (int q = 0; q < b.nprob && q < 2; ++q)
        if (!retile(b.p[q], TILE, TILE_N)) return GPTQ_EINVAL;
    b.total = b.p[0].ntiles + (b.nprob > 1 ? b.p[1].ntiles : 0);
    if (b.total <= 0) return GPTQ_OK;
    Span acc[8];
    const int na = gemm_spans<TB0, TB1, CHK>(b, acc, TILE, TILE_N);
    if (na < 0) return GPTQ_EINVAL;
    const int rc = check_launch(name, s, acc, na);
    if (rc != GPTQ_OK) return rc;
    b.gs = gang_current().gs;
    if (!dry_run()) gemm_kernel<TAG, TB0, TB1, CHK><<<gang_grid((unsigned)b.total), G_THREADS, 0, s>>>(b, flag);
    return GPTQ_OK;
}

// For sites whose shapes may be ragged: a batch whose problems all cover whole tiles of the
// site (M and N multiples of its tile) launches the kernel without bounds checks, which is
// the same computation with fewer instructions per load and store; any other batch launches
// the checked kernel.
template <int TAG, bool TB0, bool TB1>
inline int launch_gemm_fit(const char* name, hipStream_t s, const GemmBatch& b, const unsigned* flag) {
    const int TILE = b.small ? 64 : GemmCfg<TAG>::tile, TILE_N = b.small ? 64 : GemmCfg<TAG>::tile_n;
    bool whole = true;
    for (int q = 0; q < b.nprob && q < 2; ++q)
        whole = whole && b.p[q].M % TILE == 0 && b.p[q].N % TILE_N == 0;
    return whole ? launch_gemm<TAG, TB0, TB1, false>(name, s, b, flag)
                 : launch_gemm<TAG, TB0, TB1, true>(name, s, b, flag);
}

}  // namespace gptq
