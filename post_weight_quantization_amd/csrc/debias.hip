// debias.hip -- output debias of a quantized layer on gfx950.
//
// Source of the method: page "cortiq-cli 0.8.45 src/gptq.rs", q4tp_debias_hessian /
// q2tp_debias_hessian and their GEMM form debias_gemm: per row r the regression slope
// b = (W^ H W^T)_rr / (W H W^T)_rr of the quantized row's outputs on the original row's outputs,
// in the calibration metric H, is removed through the row's f16 lo (every rung of the row is
// 2^(lo + c step), so lo - log2 b divides them all by b); codes, rungs and steps stay.  The
// GEMM form computes H w for every row with one f32 product W H and sums the two per-row dot
// products in f64.  The helper that applies b to lo is not printed on the pages; the reading
// here is lo <- f16(lo - log2 b), left unchanged unless num and den are positive and finite.
//
// The same for 2-bit codes (q2tp: "MSE-optimal 2-bit rounding shrinks every output"; the pages
// run it by default there and make the 4-bit form opt-in): gptq_debias_q2.
//
// Three kernels:
//   debias_sym_kernel   H_s = H read through its upper triangle (H_s[i][j] = H[min][max]) with
//                       dead channels' rows and columns zeroed, into the workspace (32 x 32
//                       tiles through LDS so both the read of H and the write of H_s coalesce);
//   gemm_kernel<8>      Y = W H_s (rows x n x n, MFMA f32; H_s is symmetric, so its rows serve
//                       as the k-contiguous "T" operand);
//   debias_row_kernel   one workgroup per row: num = sum_j W^_rj Y_rj and den = sum_j W_rj Y_rj
//                       in f64 (W^ decoded from the nibbles and the row's current scales), then
//                       the new lo, the row's TAB and its scales.
#include <math.h>

#include "check.hpp"
#include "common.hpp"
#include "gemm_mfma.hpp"

namespace gptq {

__global__ __launch_bounds__(256) void debias_sym_kernel(const float* __restrict__ H, HLayout hl,
                                                         const uint8_t* __restrict__ dead,
                                                         float* __restrict__ Hs, int64_t n) {
    __shared__ float tile[32][33];
    const int64_t bi = blockIdx.y, bj = blockIdx.x;  // output tile (bi, bj) of H_s
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
    if (bi <= bj) {
        // On or above the diagonal: rows of H as they are.
        for (int r = ty; r < 32; r += 8) {
            const int64_t i = bi * 32 + r, j = bj * 32 + tx;
            if (i < n && j < n) {
                float v = (j >= i) ? H[hl.at(i, j)] : H[hl.at(j, i)];
                if (dead[i] || dead[j]) v = 0.0f;
                Hs[i * n + j] = v;
            }
        }
    } else {
        // Below: the transpose of tile (bj, bi) of H's upper triangle, staged through LDS.
        for (int r = ty; r < 32; r += 8) {
            const int64_t i = bj * 32 + r, j = bi * 32 + tx;  // element of H, j > i
            tile[r][tx] = (i < n && j < n) ? H[hl.at(i, j)] : 0.0f;
        }
        __syncthreads();
        for (int r = ty; r < 32; r += 8) {
            const int64_t i = bi * 32 + r, j = bj * 32 + tx;  // element of H_s, i > j
            if (i < n && j < n) {
                float v = tile[tx][r];
                if (dead[i] || dead[j]) v = 0.0f;
                Hs[i * n + j] = v;
            }
        }
    }
}

// binary16 round to nearest, ties to even, of a finite double (the ladder's rounding of lo).
__device__ __forceinline__ double f16_round(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    const double a = fabs(x);
    if (a >= 65520.0) return copysign(INFINITY, x);
    const int e = ilogb(a);
    const int qe = (e < -14) ? -24 : e - 10;
    const double r = rint(ldexp(a, -qe));
    return copysign(ldexp(r, qe), x);
}

// TWO_BIT: the codes are q2tp levels (2-bit plane [rows, n/4], W^ = (q - 1.5) s) and the
// row's ladder is the q2tp one, TAB[0] = 0, TAB[c] = 2^(lo + (c - 1) step); otherwise 4-bit
// nibbles [rows, n/2], W^ = (q - 8) s, TAB[c] = 2^(lo + c step).
template <bool TWO_BIT>
__global__ __launch_bounds__(256) void debias_row_kernel(
    const float* __restrict__ W, const uint8_t* __restrict__ dead, const float* __restrict__ Y,
    const uint8_t* __restrict__ nib, const uint8_t* __restrict__ rung, float* __restrict__ lost,
    float* __restrict__ tab, float* __restrict__ scale, double* __restrict__ slope, int64_t n) {
    __shared__ double snum[256], sden[256];
    __shared__ double s_lo, s_st;
    const int64_t r = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t ng = n / 32;
    double num = 0.0, den = 0.0;
    // Thread t takes columns 4t .. 4t+3 of every block of 1024 (a fixed order).
    for (int64_t c = 4 * (int64_t)t; c < n; c += 1024) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(W + r * n + c);
        const f32x4 y = *reinterpret_cast<const f32x4*>(Y + r * n + c);
        const float s = scale[r * ng + c / 32];
        float q[4];
        if constexpr (TWO_BIT) {
            const uint8_t b = nib[r * (n / 4) + c / 4];
#pragma unroll
            for (int u = 0; u < 4; ++u) q[u] = (float)((b >> (2 * u)) & 3) - 1.5f;
        } else {
            const uint8_t b0 = nib[r * (n / 2) + c / 2], b1 = nib[r * (n / 2) + c / 2 + 1];
            q[0] = (float)(b0 & 15) - 8.0f;
            q[1] = (float)(b0 >> 4) - 8.0f;
            q[2] = (float)(b1 & 15) - 8.0f;
            q[3] = (float)(b1 >> 4) - 8.0f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float wq = q[u] * s;
            const float wv = dead[c + u] ? 0.0f : w[u];
            num += (double)wq * (double)y[u];
            den += (double)wv * (double)y[u];
        }
    }
    snum[t] = num;
    sden[t] = den;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (t < w) {
            snum[t] += snum[t + w];
            sden[t] += sden[t + w];
        }
        __syncthreads();
    }
    if (t == 0) {
        const double nm = snum[0], dn = sden[0];
        const double lo = (double)lost[r * 2], st = (double)lost[r * 2 + 1];
        double lo2 = lo;
        const double b = nm / dn;
        if (nm > 0.0 && dn > 0.0 && isfinite(b) && b > 0.0) lo2 = f16_round(lo - log2(b));
        if (!isfinite(lo2)) lo2 = lo;
        s_lo = lo2;
        s_st = st;
        lost[r * 2] = (float)lo2;
        if (slope) slope[r] = b;
    }
    __syncthreads();
    // The row's ladder with the new lo (an all-zero row keeps TAB = 1: step 0 and lo 0 there).
    __shared__ float stab[32];
    if (t < 32) {
        const float v = TWO_BIT ? (t == 0 ? 0.0f : (float)exp2(s_lo + (double)(t - 1) * s_st))
                                : (float)exp2(s_lo + (double)t * s_st);
        stab[t] = v;
        if (tab) tab[r * 32 + t] = v;
    }
    __syncthreads();
    for (int64_t g = t; g < ng; g += 256) scale[r * ng + g] = stab[rung[r * ng + g] & 31];
}

}  // namespace gptq

using namespace gptq;

static size_t debias_ws(int64_t rows, int64_t n, size_t* off_y) {
    const size_t hs = align256(sizeof(float) * (size_t)(n * n));
    if (off_y) *off_y = hs;
    return hs + align256(sizeof(float) * (size_t)(rows * n));
}

extern "C" size_t gptq_debias_workspace_size(int64_t rows, int64_t n) {
    if (rows <= 0 || n <= 0) return 0;
    return debias_ws(rows, n, nullptr);
}

static int debias_impl(const float* W, const float* H, int64_t ldh, const uint8_t* dead,
                       const uint8_t* nib, const uint8_t* rung, float* lost, float* tab,
                       float* scale, double* slope, int64_t rows, int64_t n, void* workspace,
                       size_t workspace_bytes, void* stream, bool two_bit) {
    if (rows <= 0 || n < 32 || n % 32 != 0 || !hessian_ld_ok(n, ldh) || !W || !H || !dead || !nib || !rung ||
        !lost || !scale || !workspace)
        return GPTQ_EINVAL;
    if (rows > ((int64_t)1 << 31) - 1 || n > ((int64_t)1 << 20)) return GPTQ_EINVAL;
    if (!al16(W) || !al16(workspace)) return GPTQ_EINVAL;  // W and the workspace are read as float4
    size_t off_y = 0;
    if (workspace_bytes < debias_ws(rows, n, &off_y)) return GPTQ_EWORKSPACE;
    CheckScope check;
    check_buffer(W, sizeof(float) * (size_t)(rows * n), "W");
    check_buffer(H, sizeof(float) * (size_t)hessian_elems(n, ldh), "H");
    check_buffer(dead, (size_t)n, "dead");
    const int64_t cb = two_bit ? n / 4 : n / 2;  // code bytes per row
    check_buffer(nib, (size_t)(rows * cb), "codes");
    check_buffer(rung, (size_t)(rows * (n / 32)), "rung");
    check_buffer(lost, sizeof(float) * (size_t)(rows * 2), "lost");
    if (tab) check_buffer(tab, sizeof(float) * (size_t)(rows * 32), "tab");
    check_buffer(scale, sizeof(float) * (size_t)(rows * (n / 32)), "scale");
    if (slope) check_buffer(slope, sizeof(double) * (size_t)rows, "slope");
    check_buffer(workspace, workspace_bytes, "workspace");
    hipStream_t st = (hipStream_t)stream;
    float* Hs = (float*)workspace;
    float* Y = (float*)((char*)workspace + off_y);
    {
        const unsigned nt = (unsigned)((n + 31) / 32);
        ProfScope ps(FAM_DEBIAS, st, 0.0, 4.0 * (double)n * n * 1.5);
        GPTQ_LAUNCH(st, "debias_sym", (debias_sym_kernel<<<dim3(nt, nt), 256, 0, st>>>(H, HLayout{n, ldh}, dead, Hs, n)),
                    hessian_span(H, n, ldh, false), rd(dead, n, 1, n, 1), wr(Hs, n, n, n));
    }
    if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
    {
        // Y = W H_s: B(k, j) = H_s[j][k] (H_s symmetric).
        const GemmBatch b = gemm_batch(
            gemm_full(W, n, Hs, n, nullptr, Y, n, (int)rows, (int)n, (int)n, 1.0f, 0), nullptr);
        ProfScope ps(FAM_DEBIAS, st, 2.0 * (double)rows * n * n, 0.0);
        const int rc = launch_gemm_fit<8, true, false>("debias_gemm", st, b, nullptr);
        if (rc != GPTQ_OK) return rc;
    }
    if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
    {
        ProfScope ps(FAM_DEBIAS, st, 0.0, 12.0 * (double)rows * n);
        GPTQ_LAUNCH(st, "debias_rows",
                    (two_bit ? debias_row_kernel<true><<<(unsigned)rows, 256, 0, st>>>(
                                   W, dead, Y, nib, rung, lost, tab, scale, slope, n)
                             : debias_row_kernel<false><<<(unsigned)rows, 256, 0, st>>>(
                                   W, dead, Y, nib, rung, lost, tab, scale, slope, n)),
                    rd(W, n, rows, n), rd(dead, n, 1, n, 1), rd(Y, n, rows, n),
                    rd(nib, cb, rows, cb, 1), rd(rung, n / 32, rows, n / 32, 1),
                    wr(lost, 2, rows, 2), wr(scale, n / 32, rows, n / 32),
                    wr(tab ? (const void*)tab : (const void*)lost, tab ? 32 : 2, tab ? rows : 0, tab ? 32 : 0),
                    wr(slope ? (const void*)slope : (const void*)lost, 1, slope ? 1 : 0, slope ? rows : 0, 8));
    }
    if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
    return check.finish();
}

extern "C" int gptq_debias(const float* W, const float* H, int64_t ldh, const uint8_t* dead,
                           const uint8_t* nib, const uint8_t* rung, float* lost, float* tab,
                           float* scale, double* slope, int64_t rows, int64_t n,
                           void* workspace, size_t workspace_bytes, void* stream) {
    return debias_impl(W, H, ldh, dead, nib, rung, lost, tab, scale, slope, rows, n, workspace,
                       workspace_bytes, stream, false);
}

extern "C" int gptq_debias_q2(const float* W, const float* H, int64_t ldh, const uint8_t* dead,
                              const uint8_t* plane, const uint8_t* rung, float* lost, float* tab,
                              float* scale, double* slope, int64_t rows, int64_t n,
                              void* workspace, size_t workspace_bytes, void* stream) {
    return debias_impl(W, H, ldh, dead, plane, rung, lost, tab, scale, slope, rows, n, workspace,
                       workspace_bytes, stream, true);
}
