// act_order.hip -- the channel order of act-order GPTQ and the permuted Hessian, on gfx950.
//
// Source of the method: page "cortiq-cli 0.8.45 src/gptq.rs": act_order_perm (channels by
// descending input energy H_ii, compared in the f32 total order, ties by ascending index),
// permute_sym (H[perm][perm]) and gptq_quantize_q4tp_act_order (the fold of the permuted
// Hessian; dead channels in the original order).
//
//   act_rank_kernel    the rank of every channel under that order, by counting (n^2 compares,
//                      keys staged through LDS, four threads per channel); perm[rank[i]] = i,
//                      dead[i] = !(H_ii > 0);
//   act_permute_kernel Hp[a][b] = H[min(pa, pb)][max(pa, pb)] (H read through its upper
//                      triangle): each upper 32 x 32 tile is gathered once and written twice
//                      (in place and transposed), so the full symmetric matrix is written.
#include <math.h>

#include "check.hpp"
#include "common.hpp"

namespace gptq {

// The f32 total order as a signed integer: -NaN < -inf < ... < -0 < +0 < ... < +inf < +NaN.
__device__ __forceinline__ int32_t total_key(float x) {
    const int32_t b = __float_as_int(x);
    return b >= 0 ? b : (b ^ 0x7fffffff);
}

// Four threads per channel i (64 channels per workgroup), each counting the channels j before
// i in one quarter of every 1024-key chunk; the four counts are summed with lane shuffles.
__global__ __launch_bounds__(256) void act_rank_kernel(const float* __restrict__ H, HLayout hl,
                                                       int64_t n, int32_t* __restrict__ perm,
                                                       uint8_t* __restrict__ dead) {
    __shared__ int32_t keys[1024];
    const int part = threadIdx.x & 3;
    const int64_t i = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
    const bool live = i < n;
    const float hi = live ? H[hl.at(i, i)] : 0.0f;
    const int32_t ki = total_key(hi);
    int rank = 0;
    for (int64_t j0 = 0; j0 < n; j0 += 1024) {
        __syncthreads();
        for (int t = threadIdx.x; t < 1024; t += 256) {
            const int64_t j = j0 + t;
            keys[t] = (j < n) ? total_key(H[hl.at(j, j)]) : INT32_MIN;
        }
        __syncthreads();
        const int m = (n - j0 < 1024) ? (int)(n - j0) : 1024;
        for (int t = part; t < m; t += 4) {
            const int32_t kj = keys[t];
            // j before i: a larger key, or the same key at a smaller index.
            rank += (kj > ki || (kj == ki && j0 + t < i)) ? 1 : 0;
        }
    }
    rank += __shfl_xor(rank, 1);
    rank += __shfl_xor(rank, 2);
    if (live && part == 0) {
        perm[rank] = (int32_t)i;
        dead[i] = (hi > 0.0f) ? 0 : 1;
    }
}

// One upper 32 x 32 tile (A, B), A <= B, of Hp per workgroup: its elements are gathered once
// (Hp[a][b] = H[min(pa, pb)][max(pa, pb)]) into LDS, stored in place and, off the diagonal,
// stored again transposed at (B, A); both stores coalesce.
__global__ __launch_bounds__(256) void act_permute_kernel(const float* __restrict__ H,
                                                          HLayout hl,
                                                          const int32_t* __restrict__ perm,
                                                          int64_t n, float* __restrict__ Hp) {
    __shared__ float tile[32][33];
    const int blk = blockIdx.x;
    int r = (int)((sqrtf(8.0f * (float)blk + 1.0f) - 1.0f) * 0.5f);
    while ((r + 1) * (r + 2) / 2 <= blk) ++r;
    while (r * (r + 1) / 2 > blk) --r;
    const int64_t a0 = (int64_t)(blk - r * (r + 1) / 2) * 32, b0 = (int64_t)r * 32;  // a0 <= b0
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    const int64_t b = b0 + tx;
    const int64_t pb = (b < n) ? perm[b] : -1;
    for (int rr = ty; rr < 32; rr += 8) {
        const int64_t a = a0 + rr;
        float v = 0.0f;
        if (a < n && b < n) {
            const int64_t pa = perm[a];
            if (pa >= 0 && pa < n && pb >= 0 && pb < n)
                v = (pa <= pb) ? H[hl.at(pa, pb)] : H[hl.at(pb, pa)];
            Hp[a * n + b] = v;
        }
        tile[rr][tx] = v;
    }
    if (a0 == b0) return;
    __syncthreads();
    for (int rr = ty; rr < 32; rr += 8) {
        const int64_t row = b0 + rr, col = a0 + tx;  // Hp[row][col] = tile[col - a0][row - b0]
        if (row < n && col < n) Hp[row * n + col] = tile[tx][rr];
    }
}

}  // namespace gptq

using namespace gptq;

extern "C" int gptq_act_order_perm(const float* H, int64_t n, int64_t ldh, int32_t* perm,
                                   uint8_t* dead, void* stream) {
    if (!H || !perm || !dead || n <= 0 || !hessian_ld_ok(n, ldh) || n > ((int64_t)1 << 24))
        return GPTQ_EINVAL;
    CheckScope check;
    check_buffer(H, sizeof(float) * (size_t)hessian_elems(n, ldh), "H");
    check_buffer(perm, sizeof(int32_t) * (size_t)n, "perm");
    check_buffer(dead, (size_t)n, "dead");
    hipStream_t st = (hipStream_t)stream;
    GPTQ_LAUNCH(st, "act_rank",
                (act_rank_kernel<<<(unsigned)((n + 63) / 64), 256, 0, st>>>(H, HLayout{n, ldh}, n, perm,
                                                                             dead)),
                hessian_span(H, n, ldh, false), wr(perm, n, 1, n), wr(dead, n, 1, n, 1));
    if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
    return check.finish();
}

extern "C" int gptq_permute_hessian(const float* H, int64_t n, int64_t ldh, const int32_t* perm,
                                    float* Hp, void* stream) {
    if (!H || !perm || !Hp || n <= 0 || !hessian_ld_ok(n, ldh) || n > ((int64_t)1 << 20))
        return GPTQ_EINVAL;
    CheckScope check;
    check_buffer(H, sizeof(float) * (size_t)hessian_elems(n, ldh), "H");
    check_buffer(perm, sizeof(int32_t) * (size_t)n, "perm");
    check_buffer(Hp, sizeof(float) * (size_t)(n * n), "Hp");
    hipStream_t st = (hipStream_t)stream;
    const unsigned nt = (unsigned)((n + 31) / 32);
    GPTQ_LAUNCH(st, "act_permute",
                (act_permute_kernel<<<nt * (nt + 1) / 2, 256, 0, st>>>(H, HLayout{n, ldh}, perm, n,
                                                                         Hp)),
                hessian_span(H, n, ldh, false), rd(perm, n, 1, n), wr(Hp, n, n, n));
    if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
    return check.finish();
}
