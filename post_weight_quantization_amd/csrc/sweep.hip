// sweep.hip -- the per-row rung ladder and the q4tp GPTQ sweep on gfx950.
//
// Source of the method: page "cortiq-engine 0.8.41 src/gpu_wgpu/gptq_dev.rs" (module
// documentation step 5; kernels q4tp_group and q4tp_trail; driver sweep) and page
// "cortiq-cli 0.8.45 src/gptq.rs" (gptq_quantize_q4tp: rung rule, rounding, feedback;
// gptq_quantize_q4tp_dev: tab / lost layout).
//
// Per group of 32 columns (c0 = 32 g):
//   group kernel : one thread per row holds the corrected tile in registers, picks the rung,
//                  rounds the 32 columns in order with feedback inside the tile, and writes the
//                  nibbles, rung, scale and the scaled residuals E[:, c0:c0+32];
//   trail GEMM   : W[:, c0+32:] -= E[:, c0:c0+32] U[c0:c0+32, c0+32:]  (f32 MFMA, K = 32).
// W is never modified: the first trailing update reads the caller's W and writes the working
// copy, later ones update the copy in place.  Dead columns are zeroed whenever a tile is read
// (U has no off-diagonal entries in a dead row or column, so the GEMM leaves them alone).
#include <math.h>

#include "common.hpp"
#include "gemm_mfma.hpp"

namespace gptq {

// ---------------------------------------------------------------------------------------------
// binary16 rounding of an f64 value: nearest, ties to even, evaluated exactly in f64 by scaling
// with the quantum of the value's binade (2^-24 below the normal range).
__device__ double f16_nearest(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    const double a = fabs(x);
    if (a >= 65520.0) return copysign(INFINITY, x);
    const int e = ilogb(a);
    const int qe = (e < -14) ? -24 : e - 10;
    const double r = rint(ldexp(a, -qe));
    return copysign(ldexp(r, qe), x);
}

// One workgroup per row: group absmaxes of the dead-zeroed row, then lo / step / TAB.
__global__ __launch_bounds__(256) void ladder_kernel(const float* __restrict__ W,
                                                     const uint8_t* __restrict__ dead, int64_t n,
                                                     float* __restrict__ lost,
                                                     float* __restrict__ tab) {
    __shared__ float smin[256], smax[256];
    __shared__ double s_lo, s_st;
    __shared__ int s_any;
    const int64_t r = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t ng = n / 32;
    float amin = INFINITY, amax = 0.0f;
    for (int64_t g = t; g < ng; g += 256) {
        const float* w = W + r * n + g * 32;
        const uint8_t* d = dead + g * 32;
        float a = 0.0f;
        for (int q = 0; q < 32; q += 4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(w + q);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float x = d[q + u] ? 0.0f : fabsf(v[u]);
                a = fmaxf(a, x);
            }
        }
        if (a > 0.0f) {
            amin = fminf(amin, a);
            amax = fmaxf(amax, a);
        }
    }
    smin[t] = amin;
    smax[t] = amax;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (t < w) {
            smin[t] = fminf(smin[t], smin[t + w]);
            smax[t] = fmaxf(smax[t], smax[t + w]);
        }
        __syncthreads();
    }
    if (t == 0) {
        double lo = 0.0, st = 0.0;
        const int any = smax[0] > 0.0f;
        if (any) {
            lo = f16_nearest(log2((double)smin[0] / 7.0));
            const double hi = log2((double)smax[0] / 7.0);
            st = (hi > lo) ? f16_nearest((hi - lo) / 31.0) : 0.0;
            if (!(st > 0.0)) st = 0.0;
        }
        s_lo = lo;
        s_st = st;
        s_any = any;
        lost[r * 2] = (float)lo;
        lost[r * 2 + 1] = (float)st;
    }
    __syncthreads();
    if (t < 32) tab[r * 32 + t] = s_any ? (float)exp2(s_lo + (double)t * s_st) : 1.0f;
}

// ---------------------------------------------------------------------------------------------
// Rung choice inputs are the f32 corrected weights; the weighted error is summed in column
// order with every product and sum rounded separately (no contraction), the nominal rung is
// evaluated in f64, and codes come from correctly rounded f32 division, ties to even.
#pragma clang fp contract(off)
__device__ __forceinline__ float tile_err(const float (&w)[32], const float* hs, float s) {
    float err = 0.0f;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
        const float q = fminf(fmaxf(rintf(w[t] / s), -8.0f), 7.0f);
        const float qs = q * s;
        const float d = w[t] - qs;
        const float hd = hs[t] * d;
        const float hdd = hd * d;
        err = err + hdd;
    }
    return err;
}

__device__ __forceinline__ int nominal_rung(float amax, float lo, float st) {
    if (amax == 0.0f || st <= 0.0f) return 0;
    const double v = (log2((double)amax / 7.0) - (double)lo) / (double)st;
    double r = (v < 0.0) ? -floor(-v + 0.5) : floor(v + 0.5);
    r = fmin(fmax(r, 0.0), 31.0);
    return (int)r;
}
#pragma clang fp contract(on)

// One 32-column group: 64 rows per workgroup, one thread per row.
__global__ __launch_bounds__(64) void sweep_group_kernel(
    const float* __restrict__ src, int64_t n, int64_t c0, const float* __restrict__ U,
    const float* __restrict__ hdiag, const uint8_t* __restrict__ dead, const float* __restrict__ tab,
    const float* __restrict__ lost, int64_t rows, uint8_t* __restrict__ nib,
    uint8_t* __restrict__ rung, float* __restrict__ scale, float* __restrict__ E, int64_t ldE) {
    __shared__ float Us[32 * 33];
    __shared__ float hs[32];
    const int t = threadIdx.x;
    for (int e = t; e < 32 * 32; e += 64) {
        const int j = e >> 5, c = e & 31;
        Us[j * 33 + c] = (c >= j) ? U[(c0 + j) * n + c0 + c] : 0.0f;
    }
    if (t < 32) hs[t] = hdiag[c0 + t];
    __syncthreads();
    const int64_t r = (int64_t)blockIdx.x * 64 + t;
    if (r >= rows) return;

    float w[32];
    const float* srow = src + r * n + c0;
#pragma unroll
    for (int q = 0; q < 32; q += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(srow + q);
#pragma unroll
        for (int u = 0; u < 4; ++u) w[q + u] = dead[c0 + q + u] ? 0.0f : v[u];
    }
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 32; ++q) amax = fmaxf(amax, fabsf(w[q]));
    const float lo = lost[r * 2], st = lost[r * 2 + 1];
    const float* tb = tab + r * 32;
    const int nominal = nominal_rung(amax, lo, st);
    int best = nominal;
    if (amax > 0.0f) {
        float best_e = INFINITY;
        const int lo_c = nominal >= 2 ? nominal - 2 : 0;
        const int hi_c = nominal + 1 < 31 ? nominal + 1 : 31;
        for (int cand = lo_c; cand <= hi_c; ++cand) {
            const float s_c = tb[cand];
            if (s_c <= 0.0f) continue;
            const float err = tile_err(w, hs, s_c);
            if (err < best_e) {
                best_e = err;
                best = cand;
            }
        }
    }
    const float s = tb[best];
    const int64_t gi = r * (n / 32) + c0 / 32;
    rung[gi] = (uint8_t)best;
    scale[gi] = s;

    uint32_t words[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const float q = (s > 0.0f) ? fminf(fmaxf(rintf(w[j] / s), -8.0f), 7.0f) : 0.0f;
        words[j >> 3] |= ((uint32_t)((int)q + 8) & 15u) << (4 * (j & 7));
        const float ujj = Us[j * 33 + j];
        const float e = (ujj > 0.0f) ? (w[j] - q * s) / ujj : 0.0f;
        w[j] = e;  // the column is done: its slot now holds the residual
#pragma unroll
        for (int c = j + 1; c < 32; ++c) w[c] -= e * Us[j * 33 + c];
    }
    uint4* np4 = reinterpret_cast<uint4*>(nib + r * (n / 2) + c0 / 2);
    *np4 = make_uint4(words[0], words[1], words[2], words[3]);
    float* erow = E + r * ldE;
#pragma unroll
    for (int q = 0; q < 32; q += 4)
        *reinterpret_cast<f32x4*>(erow + q) = f32x4{w[q], w[q + 1], w[q + 2], w[q + 3]};
}

}  // namespace gptq

using namespace gptq;

extern "C" int gptq_ladder(const float* W, const uint8_t* dead, int64_t rows, int64_t n,
                           float* lost, float* tab, void* stream) {
    if (rows <= 0 || n < 32 || n % 32 != 0 || !W || !dead || !lost || !tab) return GPTQ_EINVAL;
    if (rows > ((int64_t)1 << 31) - 1) return GPTQ_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    ProfScope ps(FAM_LADDER, st, 0.0, 4.0 * (double)rows * n);
    ladder_kernel<<<(unsigned)rows, 256, 0, st>>>(W, dead, n, lost, tab);
    GPTQ_HIP(hipGetLastError());
    return GPTQ_OK;
}

static size_t sweep_ws(int64_t rows, int64_t n, size_t* off_e) {
    const size_t wc = align256(sizeof(float) * (size_t)(rows * n));
    if (off_e) *off_e = wc;
    return wc + align256(sizeof(float) * (size_t)(rows * 32));
}

extern "C" size_t gptq_sweep_workspace_size(int64_t rows, int64_t n) {
    if (rows <= 0 || n <= 0) return 0;
    return sweep_ws(rows, n, nullptr);
}

extern "C" int gptq_sweep(const float* W, const float* U, const float* hdiag, const uint8_t* dead,
                          const float* tab, const float* lost, int64_t rows, int64_t n,
                          uint8_t* nib, uint8_t* rung, float* scale, float* E, void* workspace,
                          size_t workspace_bytes, void* stream) {
    if (rows <= 0 || n < 32 || n % 32 != 0 || !W || !U || !hdiag || !dead || !tab || !lost ||
        !nib || !rung || !scale || !workspace)
        return GPTQ_EINVAL;
    if (rows > ((int64_t)1 << 31) - 64) return GPTQ_EINVAL;
    size_t off_e = 0;
    if (workspace_bytes < sweep_ws(rows, n, &off_e)) return GPTQ_EWORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    float* Wc = (float*)workspace;
    float* Eblk = (float*)((char*)workspace + off_e);
    const int64_t ng = n / 32;
    const unsigned nwg = (unsigned)((rows + 63) / 64);
    for (int64_t g = 0; g < ng; ++g) {
        const int64_t c0 = g * 32;
        const float* src = (g == 0) ? W : Wc;
        float* Eo = E ? E + c0 : Eblk;
        const int64_t ldE = E ? n : 32;
        {
            ProfScope ps(FAM_SWEEP_GROUP, st, 51.0 * 32.0 * rows, 4.0 * rows * 32 * 2 + 4.0 * 1024);
            sweep_group_kernel<<<nwg, 64, 0, st>>>(src, n, c0, U, hdiag, dead, tab, lost, rows, nib,
                                                   rung, scale, Eo, ldE);
        }
        const int64_t rest = n - c0 - 32;
        if (rest > 0) {
            GemmBatch b{};
            b.p[0] = gemm_full(Eo, ldE, U + c0 * n + c0 + 32, n, 0, src + c0 + 32, Wc + c0 + 32, n,
                               (int)rows, (int)rest, 32, -1.0f, 1);
            b.nprob = 1;
            ProfScope ps(FAM_SWEEP_TRAIL, st, 2.0 * 32.0 * rows * rest,
                         8.0 * rows * rest + 128.0 * rest + 128.0 * rows);
            gemm_kernel<2><<<b.p[0].ntiles, G_THREADS, 0, st>>>(b, nullptr);
        }
        GPTQ_HIP(hipGetLastError());
    }
    return GPTQ_OK;
}
