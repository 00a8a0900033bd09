// sweep.hip -- the per-row rung ladder and the q4tp GPTQ sweep on gfx950.
//
// Source of the method: page "cortiq-engine 0.8.41 src/gpu_wgpu/gptq_dev.rs" (module
// documentation step 5; kernels q4tp_group and q4tp_trail; driver sweep) and page
// "cortiq-cli 0.8.45 src/gptq.rs" (gptq_quantize_q4tp: rung rule, rounding, feedback;
// gptq_quantize_q4tp_dev: tab / lost layout).
//
// Blocks of 128 columns (4 groups of 32) inside outer panels of 512 columns:
//   block kernel : 16 lanes per row hold the row's corrected block in registers; per group the
//                  rung is chosen from the corrected tile, then the columns are rounded in order
//                  and each residual is fed into the rest of the block, column by column (the
//                  host sweep's full-row update restricted to the block);
//   inner update : the panel's columns right of the block, W[:, c0+128:P1] -= E_blk U_blk
//                  (f32 MFMA, K = 128);
//   panel update : every column right of the panel, W[:, P1:] -= E_pan U_pan (K = 512).
// Deferring the update of the columns right of a block (panel) to one product over its columns
// is the blocked ("lazy") form of the same elimination -- the pages' own q2tp host sweep is
// blocked the same way -- and a K = 512 product reads and writes the trailing W once per 16
// groups.  The panel update is split as in the fold: the next panel's 512 columns are updated
// first on the caller's stream, the rest on a helper stream, where it overlaps the next panel's
// blocks (look-ahead of one panel).
// W is never modified: the first update of a column reads the caller's W and writes the working
// copy, later ones update the copy in place.  Dead columns are zeroed whenever a tile is read
// (U has no off-diagonal entries in a dead row or column, so the GEMM leaves them alone).
#include <math.h>

#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "common.hpp"
#include "gemm_mfma.hpp"
#include "sweep.hpp"

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
// Q2: the q2tp ladder (outer level 1.5 s, 30 steps, TAB[0] = 0 for the all-zero group).
template <bool Q2>
__global__ __launch_bounds__(256) void ladder_kernel(const float* __restrict__ W,
                                                     const uint8_t* __restrict__ dead, int64_t n,
                                                     float* __restrict__ lost,
                                                     float* __restrict__ tab, int64_t gs) {
    W = gang_ptr(W, gs);
    dead = gang_ptr(dead, gs);
    lost = gang_ptr(lost, gs);
    tab = gang_ptr(tab, gs);
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
            const double top = Q2 ? 1.5 : 7.0;
            lo = f16_nearest(log2((double)smin[0] / top));
            const double hi = log2((double)smax[0] / top);
            st = (hi > lo) ? f16_nearest((hi - lo) / (Q2 ? 30.0 : 31.0)) : 0.0;
            if (!(st > 0.0)) st = 0.0;
        }
        s_lo = lo;
        s_st = st;
        s_any = any;
        lost[r * 2] = (float)lo;
        lost[r * 2 + 1] = (float)st;
    }
    __syncthreads();
    if (t < 32) {
        if (Q2)
            tab[r * 32 + t] = (t == 0) ? 0.0f : (s_any ? (float)exp2(s_lo + (double)(t - 1) * s_st) : 1.0f);
        else
            tab[r * 32 + t] = s_any ? (float)exp2(s_lo + (double)t * s_st) : 1.0f;
    }
}

// ---------------------------------------------------------------------------------------------
// Rung choice inputs are the f32 corrected weights; the weighted error is summed in column
// order with every product and sum rounded separately (no contraction), the nominal rung is
// evaluated in f64, and codes come from correctly rounded f32 division, ties to even.
// The nominal rung is evaluated in f64 from the f32 absmax of the corrected tile.
#pragma clang fp contract(off)
__device__ __forceinline__ int nominal_rung(float amax, float lo, float st) {
    if (amax == 0.0f || st <= 0.0f) return 0;
    const double v = (log2((double)amax / 7.0) - (double)lo) / (double)st;
    double r = (v < 0.0) ? -floor(-v + 0.5) : floor(v + 0.5);
    r = fmin(fmax(r, 0.0), 31.0);
    return (int)r;
}

// nominal_rung without its f64 log2 on the common path.  v = (log2(amax / 7) - lo) / st is
// estimated in f32 from the hardware log2; the rung is its rounding clamped to 0..31, which
// only a value within about 0.5 of 0.5 .. 30.5 can change, so the estimate decides unless it
// lies within its error bound of such a boundary (or amax is subnormal): then, rarely and
// behind a wave-uniform branch, nominal_rung itself decides.  The bound is generous: log2(amax)
// to 2^-16 max(1, |log2 amax|) (the hardware is accurate to about 2^-22 of that), the f32
// rounding of log2 7, of L - lo, of the division and of the estimate itself.  Every rung
// equals nominal_rung's.
__device__ __forceinline__ int nominal_rung_fast(float amax, float lo, float st) {
    if (amax == 0.0f || st <= 0.0f) return 0;
    const float la = __builtin_amdgcn_logf(amax);  // log2
    const float L = la - 2.80735492f;              // log2(amax / 7)
    const float v = (L - lo) / st;
    const float bound = (1.52587890625e-5f * fmaxf(fabsf(la), 1.0f) + 2e-7f + 1e-7f * fabsf(L - lo)) / st +
                        2e-7f * fabsf(v) + 1e-6f;
    const bool near = !(amax >= 1.17549435e-38f) ||
                      (!(fabsf(v - floorf(v) - 0.5f) > bound) && !(v < -1.0f) && !(v > 32.0f));
    int r = (int)fminf(fmaxf(floorf(v + 0.5f), 0.0f), 31.0f);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(near) != 0, 0)) {
        if (near) r = nominal_rung(amax, lo, st);
    }
    return r;
}
#pragma clang fp contract(fast)

// Cross-lane moves inside the 16-lane rows of a wave, as DPP operand modifiers (a VALU move,
// no LDS round trip).  C is the DPP control: quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_mirror = 0x140, row_half_mirror = 0x141, row_newbcast:L = 0x150 + L (lane L of each row
// to the whole row).
// Every control used here writes all lanes, so the move has no old value to keep (no register
// to clear first).
template <int C>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), C, 0xf, 0xf, false));
}
// Lane L of each 16-lane row group, broadcast to the whole group; L folds to a constant once
// the column loop is unrolled.
__device__ __forceinline__ float row_bcast(float v, int L) {
    switch (L) {
        case 0: return dpp_mov<0x150>(v);
        case 1: return dpp_mov<0x151>(v);
        case 2: return dpp_mov<0x152>(v);
        case 3: return dpp_mov<0x153>(v);
        case 4: return dpp_mov<0x154>(v);
        case 5: return dpp_mov<0x155>(v);
        case 6: return dpp_mov<0x156>(v);
        case 7: return dpp_mov<0x157>(v);
        case 8: return dpp_mov<0x158>(v);
        case 9: return dpp_mov<0x159>(v);
        case 10: return dpp_mov<0x15a>(v);
        case 11: return dpp_mov<0x15b>(v);
        case 12: return dpp_mov<0x15c>(v);
        case 13: return dpp_mov<0x15d>(v);
        case 14: return dpp_mov<0x15e>(v);
        default: return dpp_mov<0x15f>(v);
    }
}

// Sum / max over the 16 lanes of a row group: pairs within quads, quads within halves
// (half mirror), halves within the row (mirror).  A fixed tree; every lane gets the same value.
__device__ __forceinline__ float group16_sum(float v) {
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    v += dpp_mov<0x141>(v);
    v += dpp_mov<0x140>(v);
    return v;
}
__device__ __forceinline__ float group16_max(float v) {
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    v = fmaxf(v, dpp_mov<0x140>(v));
    return v;
}

#pragma clang fp contract(off)
// rint(fl(w / s)) -- the code decision on the correctly rounded quotient -- from w * fl(1/s):
// that product is within 3u|w/s| (u = 2^-24) of the quotient, so both round to the same integer
// unless the product lies within 4e-7 max(|w/s|, 1) of a half-integer; then divide.  The
// division sits behind a wave-uniform branch that is almost never taken, so the common path
// does not wait for it.
// Whether the code decision on w * fl(1/s) may differ from the one on fl(w / s) (rint_quot).
__device__ __forceinline__ bool near_half(float r) {
    return !(fabsf(r - floorf(r) - 0.5f) > 4e-7f * fmaxf(fabsf(r), 1.0f));
}

// fl(w / s), the correctly rounded f32 quotient, without a division: inv64 = RN64(1 / s) (0 for
// s <= 0).  The f64 product w * inv64 is within 2^-52 (relative) of w / s, while a quotient of
// two f32 numbers is never an f32 rounding boundary (a midpoint) and lies at least 2^-49
// (relative) from every one: its numerator and the midpoint times the divisor differ by at
// least one unit of their common grid.  So the product rounds to f32 exactly as w / s does,
// subnormal and overflowing quotients included.
__device__ __forceinline__ float quot_f32(float w, double inv64) { return (float)((double)w * inv64); }

__device__ __forceinline__ double bcast_f64_row(double v, int L) {
    const float lo = row_bcast(__int_as_float(__double2loint(v)), L);
    const float hi = row_bcast(__int_as_float(__double2hiint(v)), L);
    return __hiloint2double(__float_as_int(hi), __float_as_int(lo));
}

__device__ __forceinline__ float rint_quot(float w, float s, float inv_s) {
    const float r = w * inv_s;
    const float f = r - floorf(r);
    const bool near = !(fabsf(f - 0.5f) > 4e-7f * fmaxf(fabsf(r), 1.0f));
    float q = rintf(r);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(near) != 0, 0)) {
        if (near) q = rintf(w / s);
    }
    return q;
}

// Partial H_ii-weighted rounding error of two columns at scale s (each product and sum rounded);
// rint_quot for both columns behind one wave-uniform branch.
__device__ __forceinline__ float pair_err(float w0, float w1, float h0, float h1, float s,
                                          float inv_s) {
    const float r0 = w0 * inv_s, r1 = w1 * inv_s;
    const bool n0 = near_half(r0), n1 = near_half(r1);
    float qa = rintf(r0), qb = rintf(r1);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(n0 || n1) != 0, 0)) {
        if (n0) qa = rintf(w0 / s);
        if (n1) qb = rintf(w1 / s);
    }
    const float q0 = fminf(fmaxf(qa, -8.0f), 7.0f);
    const float q1 = fminf(fmaxf(qb, -8.0f), 7.0f);
    const float qs0 = q0 * s, qs1 = q1 * s;
    const float d0 = w0 - qs0, d1 = w1 - qs1;
    const float e0 = h0 * d0, e1 = h1 * d1;
    const float f0 = e0 * d0, f1 = e1 * d1;
    return f0 + f1;
}

// Unit-weight rounding error of a 32-column tile at scale s, summed in column order with every
// product and sum rounded separately (the static groups' rung choice).
__device__ __forceinline__ float unit_tile_err(const float (&w)[32], float s, float inv_s) {
    float err = 0.0f;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
        const float q = fminf(fmaxf(rint_quot(w[t], s, inv_s), -8.0f), 7.0f);
        const float qs = q * s;
        const float d = w[t] - qs;
        const float dd = d * d;
        err = err + dd;
    }
    return err;
}

// q2tp level q2_level(fl(w / s) + 1.5) = clamp(rne(clamp(x, -1, 4)), 0, 3), decided on the
// correctly rounded quotient as rint_quot does: x = w * fl(1/s) + 1.5 lands on the same level
// unless w * fl(1/s) lies within 4e-7 max(|.|, 1) of an integer (x near a half-integer); then
// (rarely, behind a wave-uniform branch) divide.
// The q2tp level clamp(rne(clamp(x, -1, 4)), 0, 3) of x = fl(w / s) + 1.5.
__device__ __forceinline__ float q2_level(float x) {
    return fminf(fmaxf(rintf(fminf(fmaxf(x, -1.0f), 4.0f)), 0.0f), 3.0f);
}

__device__ __forceinline__ float q2_level_quot(float w, float s, float inv_s) {
    const float r = w * inv_s;
    const bool near = !(fabsf(r - rintf(r)) > 4e-7f * fmaxf(fabsf(r), 1.0f));
    float x = r + 1.5f;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(near) != 0, 0)) {
        if (near) x = w / s + 1.5f;
    }
    return q2_level(x);
}

// Clipped-H_ii-weighted q2tp rounding error of two columns at scale s.
__device__ __forceinline__ float pair_err_q2(float w0, float w1, float h0, float h1, float s,
                                             float inv_s) {
    const float q0 = q2_level_quot(w0, s, inv_s), q1 = q2_level_quot(w1, s, inv_s);
    const float l0 = q0 - 1.5f, l1 = q1 - 1.5f;
    const float qs0 = l0 * s, qs1 = l1 * s;
    const float d0 = w0 - qs0, d1 = w1 - qs1;
    const float e0 = h0 * d0, e1 = h1 * d1;
    const float f0 = e0 * d0, f1 = e1 * d1;
    return f0 + f1;
}

// Clipped-H_ii-weighted q2tp rounding error of a 32-column tile at scale s, summed in column
// order with every product and sum rounded separately (the static q2 groups' rung choice).
__device__ __forceinline__ float q2_tile_err(const float (&w)[32], const float (&h)[32], float s,
                                             float inv_s) {
    float err = 0.0f;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
        const float q = q2_level_quot(w[t], s, inv_s);
        const float l = q - 1.5f;
        const float qs = l * s;
        const float d = w[t] - qs;
        const float e = h[t] * d;
        const float f = e * d;
        err = err + f;
    }
    return err;
}
#pragma clang fp contract(fast)

constexpr int SB = 128;          // columns per block (4 groups)
constexpr int RPW = 32;          // rows per workgroup of the block kernel (16 lanes each)
constexpr int BT = 16 * RPW;     // its threads
constexpr int ULD = SB + 4;      // LDS row stride of the block's U

struct BlockCtx {
    float* Us;           // U[c0 + j][c0 + t] in LDS, row stride ULD (SLIM: one group's rows)
    const float* uinv;   // 1 / U_jj (0 where U_jj <= 0), LDS
    const float* hs;     // H_ii of the block's columns, LDS
    const float* tb;     // the row's 32 rung scales
    const float* ti;     // their reciprocals (0 where the scale is not positive)
    const float* sp;     // static groups: this row's per-column scales from column c0
    uint8_t* codes;      // static groups: this row's codes (one byte each) from column c0
    float lo, st;
    int k;
    bool live;           // the row exists (SLIM: every thread runs the groups, for the barriers)
    const float* Ug;     // U in global memory (SLIM restages it group by group)
    int nc;              // the block's columns
};

// Rows [j0, j0 + 32) of the block's U (columns 0 .. nc - 1 of the block) into Us rows 0 .. 31,
// entries below the diagonal set to 0.
__device__ __forceinline__ void stage_u_rows(float* Us, const float* U, int64_t n, int64_t c0,
                                             int j0, int nc, int tid) {
    const int q4 = nc / 4;
    for (int e = tid; e < 32 * q4; e += BT) {
        const int j = e / q4, t4 = (e % q4) * 4;
        f32x4 v = *reinterpret_cast<const f32x4*>(U + (c0 + j0 + j) * n + c0 + t4);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = (t4 + q < j0 + j) ? 0.0f : v[q];
        *reinterpret_cast<f32x4*>(&Us[j * ULD + t4]) = v;
    }
}

// Group g of the block, with every register index a compile-time constant (the groups are
// unrolled by template recursion).
// MODE 0: q4tp.  MODE 1 (static groups, act order): no rung search; every column carries its
// own scale, read from cx.sp and broadcast from its owner like the weight, and the codes go to
// cx.codes as bytes.  MODE 2: q2tp ("placed"): the full search over rungs 1..31 (rung 0 for an
// all-zero group), 2-bit levels (q - 1.5) s, codes packed four to a byte.  MODE 3: static groups
// with 2-bit levels (q2tp act order): the scales of MODE 1, the levels of MODE 2, the level q
// (0..3) to cx.codes.
// SLIM: LDS holds only this group's 32 rows of U, restaged between groups behind barriers (a
// quarter of the LDS, so that four workgroups share a CU instead of two: for launches of many
// workgroups, as a gang's are); every thread then runs the groups, and only live rows store.
template <int G, int g, int MODE, bool SLIM>
__device__ __forceinline__ void block_group(float (&w)[G][2], const BlockCtx& cx, int64_t r,
                                            int64_t n, int64_t c0, uint8_t* __restrict__ nib,
                                            uint8_t* __restrict__ rung, float* __restrict__ scale,
                                            float* __restrict__ E, int64_t ldE) {
    constexpr bool ST = MODE == 1 || MODE == 3, Q2 = MODE == 2 || MODE == 3;
    const int k = cx.k;
    if constexpr (SLIM) {
        __syncthreads();  // every wave is done with the previous group's rows
        stage_u_rows(cx.Us, cx.Ug, n, c0, 32 * g, cx.nc, (int)threadIdx.x);
        __syncthreads();
    }
    float s = 0.0f, inv_s = 0.0f;
    float s_own[2] = {0.0f, 0.0f};
    double inv_own64[2] = {0.0, 0.0};
    if constexpr (Q2 && !ST) {
        const float amax = group16_max(fmaxf(fabsf(w[g][0]), fabsf(w[g][1])));
        int best = 0;
        if (amax > 0.0f) {
            best = 1;
            float best_e = INFINITY;
            const float h0 = cx.hs[32 * g + 2 * k], h1 = cx.hs[32 * g + 2 * k + 1];
            // Unrolled so that the candidates' 16-lane reductions overlap.
#pragma unroll 4
            for (int cand = 1; cand < 32; ++cand) {
                const float s_c = cx.tb[cand];
                if (!(s_c > 0.0f)) continue;
                const float err = group16_sum(pair_err_q2(w[g][0], w[g][1], h0, h1, s_c, cx.ti[cand]));
                if (err < best_e) {
                    best_e = err;
                    best = cand;
                }
            }
        }
        s = cx.tb[best];
        inv_s = cx.ti[best];
        if (k == 0 && cx.live) {
            const int64_t gi = r * (n / 32) + (c0 / 32) + g;
            rung[gi] = (uint8_t)best;
            scale[gi] = s;
        }
    } else if constexpr (ST) {
        const float2 sv = *reinterpret_cast<const float2*>(cx.sp + 32 * g + 2 * k);
        s_own[0] = sv.x;
        s_own[1] = sv.y;
        inv_own64[0] = (sv.x > 0.0f) ? 1.0 / (double)sv.x : 0.0;
        inv_own64[1] = (sv.y > 0.0f) ? 1.0 / (double)sv.y : 0.0;
    } else {
    const float amax = group16_max(fmaxf(fabsf(w[g][0]), fabsf(w[g][1])));
    const int nominal = nominal_rung_fast(amax, cx.lo, cx.st);
    int best = nominal;
    if (amax > 0.0f) {
        float best_e = INFINITY;
        const int lo_c = nominal >= 2 ? nominal - 2 : 0;
        const int hi_c = nominal + 1 < 31 ? nominal + 1 : 31;
        const float h0 = cx.hs[32 * g + 2 * k], h1 = cx.hs[32 * g + 2 * k + 1];
        // The window's (at most) four candidates, always four slots so that the loop unrolls
        // and their 16-lane reductions overlap; a slot past the window or at a scale that is
        // not positive is computed on a clamped rung and never chosen.  Ascending order and
        // strict improvement, as a loop over the window would take them.
        float err[4];
        bool ok[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cand = min(lo_c + i, 31);
            const float s_c = cx.tb[cand];
            ok[i] = lo_c + i <= hi_c && s_c > 0.0f;
            err[i] = group16_sum(pair_err(w[g][0], w[g][1], h0, h1, ok[i] ? s_c : 1.0f,
                                          ok[i] ? cx.ti[cand] : 1.0f));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (ok[i] && err[i] < best_e) {
                best_e = err[i];
                best = lo_c + i;
            }
    }
    s = cx.tb[best];
    inv_s = cx.ti[best];
    if (k == 0 && cx.live) {
        const int64_t gi = r * (n / 32) + (c0 / 32) + g;
        rung[gi] = (uint8_t)best;
        scale[gi] = s;
    }
    }
    const double inv_s64 = (s > 0.0f) ? 1.0 / (double)s : 0.0;  // RN64(1 / s) for quot_f32
    // The codes of this lane's two columns, kept as the owner computes them (a select per column;
    // they are packed once the group is done).
    float qo[2] = {0.0f, 0.0f};
    // This lane's entries of row j of U (own group and later groups) and 1 / U_jj are read one
    // column step ahead, so the serial chain -- broadcast, code, residual, the owner's next
    // column -- never waits on LDS; a scheduling barrier closes each step (otherwise the reads
    // of every step are hoisted together and the registers run out).
    float2 uo, ul[G];
    float ui;
    auto load_u = [&](int col, float2& o, float2 (&l)[G], float& iv) {
        iv = cx.uinv[col];
        const int row = SLIM ? col - 32 * g : col;
        o = *reinterpret_cast<const float2*>(&cx.Us[row * ULD + 32 * g + 2 * k]);
#pragma unroll
        for (int g2 = g + 1; g2 < G; ++g2)
            l[g2] = *reinterpret_cast<const float2*>(&cx.Us[row * ULD + 32 * g2 + 2 * k]);
    };
    load_u(32 * g, uo, ul, ui);
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) {
        const int owner = jj >> 1, slot = jj & 1;
        float2 uo_n = uo, ul_n[G];
        float ui_n = ui;
#pragma unroll
        for (int g2 = g + 1; g2 < G; ++g2) ul_n[g2] = ul[g2];
        if (jj + 1 < 32) load_u(32 * g + jj + 1, uo_n, ul_n, ui_n);
        float sj = s;
        double inv64 = inv_s64;
        if constexpr (ST) {
            sj = row_bcast(s_own[slot], owner);
            inv64 = bcast_f64_row(inv_own64[slot], owner);
        }
        const float wj = row_bcast(w[g][slot], owner);
        // The code from fl(w / s) itself (quot_f32): no division and no branch on the chain.
        const float qt = quot_f32(wj, inv64);
        float q, lev;  // the code and its level (q for q4tp, q - 1.5 for q2tp)
        if constexpr (Q2) {
            q = (sj > 0.0f) ? q2_level(qt + 1.5f) : 0.0f;
            lev = q - 1.5f;
        } else {
            q = (sj > 0.0f) ? fminf(fmaxf(rintf(qt), -8.0f), 7.0f) : 0.0f;
            lev = q;
        }
        const float e = (wj - lev * sj) * ui;
        // This lane's columns of the same group: U_jt is 0 for t < j, so the update touches
        // only the later ones; the owner's column j then takes the residual.
        w[g][0] -= e * uo.x;
        w[g][1] -= e * uo.y;
        const bool mine = k == owner;
        qo[slot] = mine ? q : qo[slot];
        w[g][slot] = mine ? e : w[g][slot];
        // ... and all of its columns of the later groups of the block.
#pragma unroll
        for (int g2 = g + 1; g2 < G; ++g2) {
            w[g2][0] -= e * ul[g2].x;
            w[g2][1] -= e * ul[g2].y;
        }
        // Pinned in this step: with no branch left in the step, the compiler would otherwise
        // sink the later groups' updates and the selects to their first use and hold every
        // step's residual, U entries and code in registers until then.
        asm volatile("" : "+v"(qo[slot]));
#pragma unroll
        for (int g2 = g + 1; g2 < G; ++g2) asm volatile("" : "+v"(w[g2][0]), "+v"(w[g2][1]));
        uo = uo_n;
        ui = ui_n;
#pragma unroll
        for (int g2 = g + 1; g2 < G; ++g2) ul[g2] = ul_n[g2];
        __builtin_amdgcn_sched_barrier(0);
    }
    const int q0 = (int)qo[0], q1 = (int)qo[1];
    uint32_t byte;
    if constexpr (ST) {
        byte = ((uint32_t)(q0 + (Q2 ? 0 : 8)) & 255u) | (((uint32_t)(q1 + (Q2 ? 0 : 8)) & 255u) << 8);
        if (cx.live) *reinterpret_cast<uint16_t*>(cx.codes + 32 * g + 2 * k) = (uint16_t)byte;
    } else if constexpr (Q2) {
        byte = ((uint32_t)q0 & 3u) | (((uint32_t)q1 & 3u) << 2);
        // Lanes 2m and 2m+1 hold columns 4m .. 4m+3: the even lane writes their byte.
        const uint32_t nb = (uint32_t)__float_as_int(dpp_mov<0xB1>(__int_as_float((int)byte)));
        if ((k & 1) == 0 && cx.live) nib[r * (n / 4) + (c0 + 32 * g) / 4 + k / 2] = (uint8_t)(byte | (nb << 4));
    } else {
        byte = ((uint32_t)(q0 + 8) & 15u) | (((uint32_t)(q1 + 8) & 15u) << 4);
        if (cx.live) nib[r * (n / 2) + (c0 + 32 * g) / 2 + k] = (uint8_t)byte;
    }
    if (cx.live) *reinterpret_cast<float2*>(E + r * ldE + 32 * g + 2 * k) = make_float2(w[g][0], w[g][1]);
    if constexpr (g + 1 < G) block_group<G, g + 1, MODE, SLIM>(w, cx, r, n, c0, nib, rung, scale, E, ldE);
}

// One block of up to 4 groups for RPW rows per workgroup, 16 lanes per row.  RPW = 32 (512
// threads) stages the block's U once for twice the rows of 16, and the 5120 rows of a down_proj
// layer make 160 workgroups, which find room beside the bulk update's sooner than 320 do; 20,
// 48 and 64 rows measured slower.  Lane k of a row
// owns columns 2k and 2k+1 of every group in the block (8 values in registers).  For each group:
// rung from the group's absmax and the 16-lane sums of the weighted error of each candidate;
// then the group's 32 columns in order: the column's corrected value is broadcast from its
// owner, every lane of the row computes the same code and residual, and each lane feeds the
// residual into its own later columns of the block through row j of U (held in LDS).
template <int G, int MODE, bool SLIM>
__global__ __launch_bounds__(BT) void sweep_block_kernel(
    const float* __restrict__ src, int64_t n, int64_t c0, const float* __restrict__ U,
    const float* __restrict__ hdiag, const uint8_t* __restrict__ dead,
    const float* __restrict__ tab, const float* __restrict__ lost, int64_t rows,
    uint8_t* __restrict__ nib, uint8_t* __restrict__ rung, float* __restrict__ scale,
    float* __restrict__ E, int64_t ldE, const float* __restrict__ sp,
    uint8_t* __restrict__ codes, int64_t gs) {
    __builtin_amdgcn_s_setprio(CHAIN_PRIO);
    constexpr int NC = 32 * G;
    constexpr bool ST = MODE == 1 || MODE == 3;
    src = gang_ptr(src, gs);
    U = gang_ptr(U, gs);
    hdiag = gang_ptr(hdiag, gs);
    dead = gang_ptr(dead, gs);
    tab = gang_ptr(tab, gs);
    lost = gang_ptr(lost, gs);
    nib = gang_ptr(nib, gs);
    rung = gang_ptr(rung, gs);
    scale = gang_ptr(scale, gs);
    E = gang_ptr(E, gs);
    if constexpr (ST) {
        sp = gang_ptr(sp, gs);
        codes = gang_ptr(codes, gs);
    }
    __shared__ __attribute__((aligned(16))) float Us[(SLIM ? 32 : SB) * ULD];
    __shared__ float hs[SB];
    __shared__ float uinv[SB];
    __shared__ float tabs[RPW * 32];
    __shared__ float tinv[RPW * 32];
    const int tid = threadIdx.x;
    // The block's U with its entries below the diagonal set to 0 (only the upper triangle of U
    // is read): the feedback of column j then runs unconditionally over every column.  SLIM
    // stages one group's rows at a time, in the groups.
    if constexpr (!SLIM)
        for (int j0 = 0; j0 < NC; j0 += 32) stage_u_rows(Us + j0 * ULD, U, n, c0, j0, NC, tid);
    if (tid < NC) {
        // q4tp weighs by H_ii, q2tp by max(H_ii, 0); static groups do not search.
        hs[tid] = ST ? 1.0f : (MODE == 2 ? fmaxf(hdiag[c0 + tid], 0.0f) : hdiag[c0 + tid]);
        const float d = U[(c0 + tid) * n + c0 + tid];
        uinv[tid] = (d > 0.0f) ? 1.0f / d : 0.0f;
    }
    const int64_t r0 = (int64_t)blockIdx.x * RPW;
    // The rows' rung scales and their reciprocals (the same IEEE division the search would do
    // per candidate, done once).
    for (int e = tid; e < RPW * 32; e += BT) {
        const float t = (r0 + e / 32 < rows) ? tab[(r0 + e / 32) * 32 + (e & 31)] : 1.0f;
        tabs[e] = t;
        tinv[e] = (t > 0.0f) ? 1.0f / t : 0.0f;
    }
    __syncthreads();
    const int k = tid & 15;
    const bool live = r0 + (tid >> 4) < rows;
    if (!SLIM && !live) return;
    // A row that does not exist (SLIM only) runs as row r0 with zero weights, storing nothing.
    const int64_t r = live ? r0 + (tid >> 4) : r0;

    float w[G][2];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int64_t c = c0 + 32 * g + 2 * k;
        const float2 v = live ? *reinterpret_cast<const float2*>(src + r * n + c) : make_float2(0.0f, 0.0f);
        // Static groups sweep a gathered, already dead-zeroed copy.
        w[g][0] = (!ST && dead[c]) ? 0.0f : v.x;
        w[g][1] = (!ST && dead[c + 1]) ? 0.0f : v.y;
    }
    BlockCtx cx;
    cx.Us = Us;
    cx.uinv = uinv;
    cx.hs = hs;
    cx.tb = &tabs[(tid >> 4) * 32];
    cx.ti = &tinv[(tid >> 4) * 32];
    cx.lo = (MODE == 0) ? lost[r * 2] : 0.0f;  // only q4tp's nominal rung reads the ladder's lo / step
    cx.st = (MODE == 0) ? lost[r * 2 + 1] : 0.0f;
    cx.k = k;
    cx.sp = ST ? sp + r * n + c0 : nullptr;
    cx.codes = ST ? codes + r * n + c0 : nullptr;
    cx.live = live;
    cx.Ug = U;
    cx.nc = NC;
    block_group<G, 0, MODE, SLIM>(w, cx, r, n, c0, nib, rung, scale, E, ldE);
}

// Static groups, step 1: the rung of every (row, group) chosen up front from the dead-zeroed
// original tile -- the sweep's rung rule with unit weights: nominal from the absmax, then the
// candidates nominal-2 .. nominal+1 by the f32 squared rounding error summed in column order.
// One thread per (row, group).
__global__ __launch_bounds__(256) void static_rung_kernel(const float* __restrict__ W,
                                                          const uint8_t* __restrict__ dead,
                                                          const float* __restrict__ tab,
                                                          const float* __restrict__ lost,
                                                          int64_t rows, int64_t n,
                                                          uint8_t* __restrict__ rung,
                                                          float* __restrict__ scale) {
    const int64_t ng = n / 32;
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= rows * ng) return;
    const int64_t r = id / ng, g = id % ng;
    float w[32];
    float amax = 0.0f;
#pragma unroll
    for (int t = 0; t < 32; t += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(W + r * n + 32 * g + t);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            w[t + u] = dead[32 * g + t + u] ? 0.0f : v[u];
            amax = fmaxf(amax, fabsf(w[t + u]));
        }
    }
    const float* tb = tab + r * 32;
    const int nominal = nominal_rung(amax, lost[r * 2], lost[r * 2 + 1]);
    int best = nominal;
    if (amax > 0.0f) {
        float best_e = INFINITY;
        const int lo_c = nominal >= 2 ? nominal - 2 : 0;
        const int hi_c = nominal + 1 < 31 ? nominal + 1 : 31;
        for (int cand = lo_c; cand <= hi_c; ++cand) {
            const float s_c = tb[cand];
            if (s_c <= 0.0f) continue;
            const float err = unit_tile_err(w, s_c, 1.0f / s_c);
            if (err < best_e) {
                best_e = err;
                best = cand;
            }
        }
    }
    rung[r * ng + g] = (uint8_t)best;
    scale[r * ng + g] = tb[best];
}

// Static groups of q2tp, step 1: the rung of every (row, group) chosen up front from the
// dead-zeroed original tile by the q2tp sweep's own search: rung 0 for an all-zero tile, else
// the best of rungs 1..31 (TAB > 0) by the max(H_ii, 0)-weighted f32 error summed in column
// order, a strictly smaller error replacing the current best.  One thread per (row, group).
// hdiag_p holds H_ii in elimination order (the fold of H[perm][perm]); channel c's weight is
// hdiag_p[inv[c]] (0 for a channel perm does not name).
__global__ __launch_bounds__(256) void static_rung_q2_kernel(const float* __restrict__ W,
                                                             const uint8_t* __restrict__ dead,
                                                             const float* __restrict__ hdiag_p,
                                                             const int32_t* __restrict__ inv,
                                                             const float* __restrict__ tab,
                                                             int64_t rows, int64_t n,
                                                             uint8_t* __restrict__ rung,
                                                             float* __restrict__ scale) {
    const int64_t ng = n / 32;
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= rows * ng) return;
    const int64_t r = id / ng, g = id % ng;
    float w[32], h[32];
    float amax = 0.0f;
#pragma unroll
    for (int t = 0; t < 32; t += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(W + r * n + 32 * g + t);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t c = 32 * g + t + u;
            const int32_t a = inv[c];
            w[t + u] = dead[c] ? 0.0f : v[u];
            h[t + u] = (a >= 0 && a < n) ? fmaxf(hdiag_p[a], 0.0f) : 0.0f;
            amax = fmaxf(amax, fabsf(w[t + u]));
        }
    }
    const float* tb = tab + r * 32;
    int best = 0;
    if (amax > 0.0f) {
        best = 1;
        float best_e = INFINITY;
        for (int cand = 1; cand < 32; ++cand) {
            const float s_c = tb[cand];
            if (!(s_c > 0.0f)) continue;
            const float err = q2_tile_err(w, h, s_c, 1.0f / s_c);
            if (err < best_e) {
                best_e = err;
                best = cand;
            }
        }
    }
    rung[r * ng + g] = (uint8_t)best;
    scale[r * ng + g] = tb[best];
}

// The ladder of every row (q4tp, or q2tp when Q2), for the gang open on this thread or one
// matrix.
static int ladder_launch(bool q2, const float* W, const uint8_t* dead, int64_t rows, int64_t n,
                         float* lost, float* tab, hipStream_t st) {
    const int64_t gs = gang_current().gs;
    ProfScope ps(FAM_LADDER, st, 0.0, 4.0 * (double)rows * n);
    GPTQ_LAUNCH(st, q2 ? "ladder_q2" : "ladder",
                (q2 ? ladder_kernel<true><<<gang_grid((unsigned)rows), 256, 0, st>>>(W, dead, n, lost, tab, gs)
                    : ladder_kernel<false><<<gang_grid((unsigned)rows), 256, 0, st>>>(W, dead, n, lost, tab, gs)),
                rd(W, n, rows, n), rd(dead, n, 1, n, 1), wr(lost, 2, rows, 2), wr(tab, 32, rows, 32));
    return launch_status() != GPTQ_OK ? GPTQ_EHIP : GPTQ_OK;
}

}  // namespace gptq

using namespace gptq;

extern "C" int gptq_ladder(const float* W, const uint8_t* dead, int64_t rows, int64_t n,
                           float* lost, float* tab, void* stream) {
    if (rows <= 0 || n < 32 || n % 32 != 0 || !W || !dead || !lost || !tab) return GPTQ_EINVAL;
    if (rows > ((int64_t)1 << 31) - 1 || !al16(W)) return GPTQ_EINVAL;  // rows read as float4
    CheckScope check;
    check_buffer(W, sizeof(float) * (size_t)(rows * n), "W");
    check_buffer(dead, (size_t)n, "dead");
    check_buffer(lost, sizeof(float) * (size_t)(rows * 2), "lost");
    check_buffer(tab, sizeof(float) * (size_t)(rows * 32), "tab");
    const int rc = ladder_launch(false, W, dead, rows, n, lost, tab, (hipStream_t)stream);
    if (rc != GPTQ_OK) return rc;
    return check.finish();
}

constexpr int SOB = 512;         // columns per outer panel

// Workspace: the working copy of W (rows x n) and two panel buffers of residuals (rows x 512,
// alternating between panels so that a panel's update can still read them while the next
// panel's blocks write the other one).
static size_t sweep_ws(int64_t rows, int64_t n, size_t* off_e) {
    const size_t wc = align256(sizeof(float) * (size_t)(rows * n));
    if (off_e) *off_e = wc;
    return wc + 2 * align256(sizeof(float) * (size_t)(rows * SOB));
}

extern "C" size_t gptq_sweep_workspace_size(int64_t rows, int64_t n) {
    if (rows <= 0 || n <= 0) return 0;
    return sweep_ws(rows, n, nullptr);
}

// A gang's launch (many workgroups) takes the SLIM form; q4tp and q2tp only.
template <int G, int MODE>
static void launch_block(unsigned nwg, hipStream_t st, const float* src, int64_t n, int64_t c0,
                         const float* U, const float* hdiag, const uint8_t* dead, const float* tab,
                         const float* lost, int64_t rows, uint8_t* nib, uint8_t* rung, float* scale,
                         float* E, int64_t ldE, const float* sp, uint8_t* codes) {
    const Gang gg = gang_current();
    if constexpr (MODE == 0 || MODE == 2) {
        if (gg.G > 1) {
            sweep_block_kernel<G, MODE, true><<<gang_grid(nwg), BT, 0, st>>>(
                src, n, c0, U, hdiag, dead, tab, lost, rows, nib, rung, scale, E, ldE, sp, codes, gg.gs);
            return;
        }
    }
    sweep_block_kernel<G, MODE, false><<<gang_grid(nwg), BT, 0, st>>>(
        src, n, c0, U, hdiag, dead, tab, lost, rows, nib, rung, scale, E, ldE, sp, codes, gg.gs);
}

// One sweep over the columns in their storage order (the channel order for the plain sweep,
// the elimination order for act order).
struct SweepRun {
    const float* first;  // what the first panel reads: the caller's W, or the gathered copy Wc
    const float* U;
    const float* hdiag;
    const uint8_t* dead;
    const float* tab;
    const float* lost;
    int64_t rows, n;
    uint8_t* nib;
    uint8_t* rung;
    float* scale;
    float* E;
    float* Wc;
    float* Epan[2];
    const float* sp;     // static groups: per-column scales [rows, n] (elimination order)
    uint8_t* codes;      // static groups: codes [rows, n] (elimination order)
};

// single: every launch on the caller's stream, in the order the two-stream pipeline's events
// impose (so each column receives the same updates in the same order: the same results, bit
// for bit); no helper stream or event is taken.
template <int MODE>
static int sweep_pipeline(const SweepRun& c, hipStream_t st, bool single = false) {
    const int64_t rows = c.rows, n = c.n;
    const float* U = c.U;
    float* Wc = c.Wc;
    const unsigned nwg = (unsigned)((rows + RPW - 1) / RPW);

    Helper hp{};
    if (!single && helper_acquire(&hp) != GPTQ_OK) return GPTQ_EHIP;
    hipStream_t ts = single ? st : hp.stream;
    struct Release {
        const Helper& h;
        bool on;
        ~Release() {
            if (on) helper_release(h);
        }
    } release{hp, !single};
#define SWEEP_OK(call)                          \
    do {                                        \
        const int rc_ = (call);                 \
        if (rc_ != GPTQ_OK) return rc_;         \
    } while (0)

    bool first_bulk = true;
    int pan = 0;
    for (int64_t P0 = 0; P0 < n; P0 += SOB, pan ^= 1) {
        const int64_t w = std::min<int64_t>(SOB, n - P0);
        float* Ep = c.E ? c.E + P0 : c.Epan[pan];
        const int64_t ldE = c.E ? n : SOB;
        for (int64_t c0 = P0; c0 < P0 + w; c0 += SB) {
            const int G = (int)((P0 + w - c0 >= SB) ? 4 : (P0 + w - c0) / 32);
            const int64_t nc = 32 * G;
            const float* src = (c0 == 0) ? c.first : Wc;
            float* Eo = Ep + (c0 - P0);
            {
                ProfScope ps(FAM_SWEEP_GROUP, st, 51.0 * nc * rows + (double)rows * nc * nc,
                             4.0 * rows * nc * 2 + 4.0 * nc * nc);
#define BLOCK_ARGS nwg, st, src, n, c0, U, c.hdiag, c.dead, c.tab, c.lost, rows, c.nib, c.rung, c.scale, Eo, ldE, c.sp, c.codes
                if constexpr (MODE == 1 || MODE == 3) {
                    GPTQ_LAUNCH(st, "sweep_block_static",
                                (G == 4   ? launch_block<4, MODE>(BLOCK_ARGS)
                                 : G == 3 ? launch_block<3, MODE>(BLOCK_ARGS)
                                 : G == 2 ? launch_block<2, MODE>(BLOCK_ARGS)
                                          : launch_block<1, MODE>(BLOCK_ARGS)),
                                rd(src + c0, n, rows, nc), rd(U + c0 * n + c0, n, nc, nc),
                                rd(c.sp + c0, n, rows, nc), wr(c.codes + c0, n, rows, nc, 1),
                                wr(Eo, ldE, rows, nc));
                } else if constexpr (MODE == 2) {
                    GPTQ_LAUNCH(st, "sweep_block_q2",
                                (G == 4   ? launch_block<4, 2>(BLOCK_ARGS)
                                 : G == 3 ? launch_block<3, 2>(BLOCK_ARGS)
                                 : G == 2 ? launch_block<2, 2>(BLOCK_ARGS)
                                          : launch_block<1, 2>(BLOCK_ARGS)),
                                rd(src + c0, n, rows, nc), rd(U + c0 * n + c0, n, nc, nc),
                                rd(c.hdiag + c0, n, 1, nc), rd(c.dead + c0, n, 1, nc, 1),
                                rd(c.tab, 32, rows, 32),
                                wr(c.nib + c0 / 4, n / 4, rows, nc / 4, 1),
                                wr(c.rung + c0 / 32, n / 32, rows, G, 1),
                                wr(c.scale + c0 / 32, n / 32, rows, G), wr(Eo, ldE, rows, nc));
                } else {
                    GPTQ_LAUNCH(st, "sweep_block",
                                (G == 4   ? launch_block<4, 0>(BLOCK_ARGS)
                                 : G == 3 ? launch_block<3, 0>(BLOCK_ARGS)
                                 : G == 2 ? launch_block<2, 0>(BLOCK_ARGS)
                                          : launch_block<1, 0>(BLOCK_ARGS)),
                                rd(src + c0, n, rows, nc), rd(U + c0 * n + c0, n, nc, nc),
                                rd(c.hdiag + c0, n, 1, nc), rd(c.dead + c0, n, 1, nc, 1),
                                rd(c.tab, 32, rows, 32), rd(c.lost, 2, rows, 2),
                                wr(c.nib + c0 / 2, n / 2, rows, nc / 2, 1),
                                wr(c.rung + c0 / 32, n / 32, rows, G, 1),
                                wr(c.scale + c0 / 32, n / 32, rows, G), wr(Eo, ldE, rows, nc));
                }
#undef BLOCK_ARGS
            }
            // The rest of the panel: columns c0 + nc .. P0 + w (last read at the same source).
            const int64_t rest_in = P0 + w - c0 - nc;
            if (rest_in > 0) {
                const GemmBatch b = gemm_batch(
                    gemm_full(Eo, ldE, U + c0 * n + c0 + nc, n, src + c0 + nc, Wc + c0 + nc, n,
                              (int)rows, (int)rest_in, (int)nc, -1.0f, 1),
                    nullptr);
                ProfScope ps(FAM_SWEEP_NEXT, st, 2.0 * nc * rows * rest_in,
                             8.0 * rows * rest_in + 4.0 * nc * rest_in + 4.0 * rows * nc);
                SWEEP_OK((launch_gemm_fit<6, false, false>("sweep_in_panel", st, b, nullptr)));
            }
            if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
        }
        const int64_t rest = n - P0 - w;
        if (rest <= 0) continue;
        // Columns right of the panel still hold the first source when this is the first panel.
        const float* src = (P0 == 0) ? c.first : Wc;
        const float* Up = U + P0 * n;  // the panel's rows of U
        const int64_t nw = std::min<int64_t>(SOB, rest);
        const int64_t rest2 = rest - nw;
        // Look-ahead: the next panel's columns, on the chain, after the previous panel's bulk
        // update (which wrote them, and read the residual buffer the next panel's blocks
        // overwrite).  Bulk: every column beyond the next panel, on the helper stream.  Both
        // become ready together; started together, the bulk update takes most of the GPU and
        // the look-ahead, which the next panel's blocks wait for, crawls (about 140 us instead
        // of 30).  So the look-ahead goes first and the bulk update waits for it.
        if (!first_bulk && !single) SWEEP_OK(stream_wait(st, hp.ev_b));
        {
            const int64_t j0 = P0 + w;
            const GemmBatch b = gemm_batch(
                gemm_full(Ep, ldE, Up + j0, n, src + j0, Wc + j0, n, (int)rows, (int)nw, (int)w,
                          -1.0f, 1),
                nullptr);
            ProfScope ps(FAM_SWEEP_NEXT, st, 2.0 * w * rows * nw,
                         8.0 * rows * nw + 4.0 * w * nw + 4.0 * rows * w);
            SWEEP_OK((launch_gemm_fit<7, false, false>("sweep_look_ahead", st, b, nullptr)));
            if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
        }
        if (rest2 > 0) {
            if (!single) {
                SWEEP_OK(ev_record(hp.ev_a, st));
                SWEEP_OK(stream_wait(ts, hp.ev_a));
            }
            const int64_t j0 = P0 + w + nw;
            GemmBatch b = gemm_batch(
                gemm_full(Ep, ldE, Up + j0, n, src + j0, Wc + j0, n, (int)rows, (int)rest2, (int)w,
                          -1.0f, 1),
                nullptr);
            // 64 x 64 tiles for a launch of fewer than 900 128-tiles across the gang's groups (as
            // the fold's small bulk launches); a gang's launches are larger by its group count.
            b.small = (int64_t)b.total * gang_current().G < 900 ? 1 : 0;
            ProfScope ps(FAM_SWEEP_TRAIL, ts, 2.0 * w * rows * rest2,
                         8.0 * rows * rest2 + 4.0 * w * rest2 + 4.0 * rows * w);
            SWEEP_OK((launch_gemm_fit<2, false, false>("sweep_bulk", ts, b, nullptr)));
            if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
            if (!single) SWEEP_OK(ev_record(hp.ev_b, ts));
            first_bulk = false;
        }
    }
    // Join the helper stream.
    if (!single) {
        SWEEP_OK(ev_record(hp.ev_b, ts));
        SWEEP_OK(stream_wait(st, hp.ev_b));
    }
#undef SWEEP_OK
    return GPTQ_OK;
}

// Argument rules shared by the q4tp sweep entry points (GPTQ_EINVAL otherwise): sizes, the
// required pointers, and 16-byte alignment of W, U and E (read and written as float4 / float2
// rows; n % 32 == 0 keeps every row aligned).
static bool sweep_args_ok(const float* W, const float* U, const float* hdiag, const uint8_t* dead,
                          const float* tab, const float* lost, int64_t rows, int64_t n,
                          const uint8_t* nib, const uint8_t* rung, const float* scale,
                          const float* E) {
    if (rows <= 0 || n < 32 || n % 32 != 0 || !W || !U || !hdiag || !dead || !tab || !lost ||
        !nib || !rung || !scale)
        return false;
    if (rows > ((int64_t)1 << 31) - 64 || n > ((int64_t)1 << 24)) return false;
    return al16(W) && al16(U) && al16(E);
}

static void sweep_check_buffers(const float* W, const float* U, const float* hdiag,
                                const uint8_t* dead, const float* tab, const float* lost,
                                int64_t rows, int64_t n, const uint8_t* nib, const uint8_t* rung,
                                const float* scale, const float* E) {
    check_buffer(W, sizeof(float) * (size_t)(rows * n), "W");
    check_buffer(U, sizeof(float) * (size_t)(n * n), "U");
    check_buffer(hdiag, sizeof(float) * (size_t)n, "hdiag");
    check_buffer(dead, (size_t)n, "dead");
    check_buffer(tab, sizeof(float) * (size_t)(rows * 32), "tab");
    check_buffer(lost, sizeof(float) * (size_t)(rows * 2), "lost");
    check_buffer(nib, (size_t)(rows * (n / 2)), "nib");
    check_buffer(rung, (size_t)(rows * (n / 32)), "rung");
    check_buffer(scale, sizeof(float) * (size_t)(rows * (n / 32)), "scale");
    if (E) check_buffer(E, sizeof(float) * (size_t)(rows * n), "E");
}

static SweepRun q4_run(const float* first, float* Wc, const float* U, const float* hdiag,
                       const uint8_t* dead, const float* tab, const float* lost, int64_t rows,
                       int64_t n, uint8_t* nib, uint8_t* rung, float* scale, float* E,
                       float* pan0, float* pan1) {
    SweepRun c{};
    c.first = first;
    c.U = U;
    c.hdiag = hdiag;
    c.dead = dead;
    c.tab = tab;
    c.lost = lost;
    c.rows = rows;
    c.n = n;
    c.nib = nib;
    c.rung = rung;
    c.scale = scale;
    c.E = E;
    c.Wc = Wc;
    c.Epan[0] = pan0;
    c.Epan[1] = pan1;
    return c;
}

namespace gptq {

int sweep_run(const float* W, const float* U, const float* hdiag, const uint8_t* dead,
              const float* tab, const float* lost, int64_t rows, int64_t n, uint8_t* nib,
              uint8_t* rung, float* scale, float* E, void* workspace, size_t workspace_bytes,
              hipStream_t st, bool single) {
    if (!sweep_args_ok(W, U, hdiag, dead, tab, lost, rows, n, nib, rung, scale, E) || !workspace ||
        !al16(workspace))
        return GPTQ_EINVAL;
    size_t off_e = 0;
    if (workspace_bytes < sweep_ws(rows, n, &off_e)) return GPTQ_EWORKSPACE;
    CheckScope check;
    sweep_check_buffers(W, U, hdiag, dead, tab, lost, rows, n, nib, rung, scale, E);
    check_buffer(workspace, workspace_bytes, "workspace");
    char* ws = (char*)workspace;
    const SweepRun c = q4_run(W, (float*)ws, U, hdiag, dead, tab, lost, rows, n, nib, rung, scale,
                              E, (float*)(ws + off_e),
                              (float*)(ws + off_e + align256(sizeof(float) * (size_t)(rows * SOB))));
    const int rc = sweep_pipeline<0>(c, st, single);
    if (rc != GPTQ_OK) return rc;
    return check.finish();
}

}  // namespace gptq

namespace gptq {

size_t sweep_panel_bytes(int64_t rows) { return align256(sizeof(float) * (size_t)(rows * SOB)); }

int sweep_gang(int G, int64_t gs, bool q2, float* Wc, const float* U, const float* hdiag,
               const uint8_t* dead, float* lost, float* tab, int64_t rows, int64_t n, uint8_t* nib,
               uint8_t* rung, float* scale, float* pan0, float* pan1, hipStream_t st) {
    if (G < 1 || G > kMaxGang || gs % 256 != 0) return GPTQ_EINVAL;
    if (!sweep_args_ok(Wc, U, hdiag, dead, tab, lost, rows, n, nib, rung, scale, nullptr) ||
        !al16(pan0) || !al16(pan1))
        return GPTQ_EINVAL;
    CheckScope check;
    const size_t pb = sweep_panel_bytes(rows);
    for (int g = 0; g < G; ++g) {
        const int64_t o = g * gs;
        check_buffer((const char*)Wc + o, sizeof(float) * (size_t)(rows * n), "Wc");
        check_buffer((const char*)U + o, sizeof(float) * (size_t)(n * n), "U");
        check_buffer((const char*)hdiag + o, sizeof(float) * (size_t)n, "hdiag");
        check_buffer((const char*)dead + o, (size_t)n, "dead");
        check_buffer((const char*)lost + o, sizeof(float) * (size_t)(rows * 2), "lost");
        check_buffer((const char*)tab + o, sizeof(float) * (size_t)(rows * 32), "tab");
        check_buffer((const char*)nib + o, (size_t)(rows * (n / (q2 ? 4 : 2))), "codes");
        check_buffer((const char*)rung + o, (size_t)(rows * (n / 32)), "rung");
        check_buffer((const char*)scale + o, sizeof(float) * (size_t)(rows * (n / 32)), "scale");
        check_buffer((const char*)pan0 + o, pb, "panel 0");
        check_buffer((const char*)pan1 + o, pb, "panel 1");
    }
    {
        GangScope gang(G, gs);
        int rc = ladder_launch(q2, Wc, dead, rows, n, lost, tab, st);
        if (rc != GPTQ_OK) return rc;
        // In place: the working copy is the matrix itself (the same results as a separate copy,
        // bit for bit).
        SweepRun c = q4_run(Wc, Wc, U, hdiag, dead, tab, lost, rows, n, nib, rung, scale, nullptr,
                            pan0, pan1);
        if (q2) {
            c.lost = nullptr;
            rc = sweep_pipeline<2>(c, st);
        } else {
            rc = sweep_pipeline<0>(c, st);
        }
        if (rc != GPTQ_OK) return rc;
    }
    return check.finish();
}

}  // namespace gptq

extern "C" int gptq_sweep(const float* W, const float* U, const float* hdiag, const uint8_t* dead,
                          const float* tab, const float* lost, int64_t rows, int64_t n,
                          uint8_t* nib, uint8_t* rung, float* scale, float* E, void* workspace,
                          size_t workspace_bytes, void* stream) {
    return sweep_run(W, U, hdiag, dead, tab, lost, rows, n, nib, rung, scale, E, workspace,
                     workspace_bytes, (hipStream_t)stream, false);
}

// In place: W is its own working copy, so the workspace holds only the two residual panels, and
// nothing at all when the residuals go to E.
static size_t sweep_panels_ws(int64_t rows) {
    return 2 * align256(sizeof(float) * (size_t)(rows * SOB));
}

extern "C" size_t gptq_sweep_inplace_workspace_size(int64_t rows, int64_t n) {
    if (rows <= 0 || n <= 0) return 0;
    return sweep_panels_ws(rows);
}

extern "C" int gptq_sweep_inplace(float* W, const float* U, const float* hdiag,
                                  const uint8_t* dead, const float* tab, const float* lost,
                                  int64_t rows, int64_t n, uint8_t* nib, uint8_t* rung,
                                  float* scale, float* E, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    if (!sweep_args_ok(W, U, hdiag, dead, tab, lost, rows, n, nib, rung, scale, E) ||
        !al16(workspace) || (!E && !workspace))
        return GPTQ_EINVAL;
    if (!E && workspace_bytes < sweep_panels_ws(rows)) return GPTQ_EWORKSPACE;
    CheckScope check;
    sweep_check_buffers(W, U, hdiag, dead, tab, lost, rows, n, nib, rung, scale, E);
    float* pan0 = nullptr;
    float* pan1 = nullptr;
    if (!E) {
        check_buffer(workspace, workspace_bytes, "workspace");
        pan0 = (float*)workspace;
        pan1 = (float*)((char*)workspace + align256(sizeof(float) * (size_t)(rows * SOB)));
    }
    const SweepRun c = q4_run(W, W, U, hdiag, dead, tab, lost, rows, n, nib, rung, scale, E, pan0, pan1);
    const int rc = sweep_pipeline<0>(c, (hipStream_t)stream);
    if (rc != GPTQ_OK) return rc;
    return check.finish();
}

// ---------------------------------------------------------------------------------------------
// For callers that cannot allocate device memory: the residual panels of the in-place sweep in
// a static device buffer of the library, 2 x kScratchRows x 512 f32 = 32 MiB on each GPU it
// runs on, held until the process ends.  Host code never passes the array's name to a kernel
// (on the host it is only a stand-in): each device's copy is located once, with that device
// current, by hipGetSymbolAddress, and that address is what the kernels get.
constexpr int64_t kScratchRows = 8192;
static __device__ __align__(256) float scratch[2 * kScratchRows * SOB];

static int scratch_address(float** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GPTQ_EHIP;
    static std::mutex mu;
    static std::vector<std::pair<int, float*>> known;  // (device, its copy of scratch)
    std::lock_guard<std::mutex> lk(mu);
    for (const auto& k : known)
        if (k.first == dev) {
            *out = k.second;
            return GPTQ_OK;
        }
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GPTQ_EHIP;
    known.emplace_back(dev, (float*)p);
    *out = (float*)p;
    return GPTQ_OK;
}

extern "C" int gptq_sweep_inplace_noalloc(float* W, const float* U, const float* hdiag,
                                          const uint8_t* dead, const float* tab, const float* lost,
                                          int64_t rows, int64_t n, uint8_t* nib, uint8_t* rung,
                                          float* scale, float* E, void* stream) {
    if (!sweep_args_ok(W, U, hdiag, dead, tab, lost, rows, n, nib, rung, scale, E))
        return GPTQ_EINVAL;
    if (!E && rows > kScratchRows) return GPTQ_ETOOBIG;
    CheckScope check;
    float* pan = nullptr;
    if (!E) {
        if (dry_run()) {
            pan = reinterpret_cast<float*>((uintptr_t)1 << 46);  // a stand-in for the schedule check
        } else {
            const int rc = scratch_address(&pan);
            if (rc != GPTQ_OK) return rc;
        }
    }
    sweep_check_buffers(W, U, hdiag, dead, tab, lost, rows, n, nib, rung, scale, E);
    if (pan) check_buffer(pan, sizeof(float) * (size_t)(2 * kScratchRows * SOB), "scratch");
    const SweepRun c = q4_run(W, W, U, hdiag, dead, tab, lost, rows, n, nib, rung, scale, E, pan,
                              pan ? pan + kScratchRows * SOB : nullptr);
    const int rc = sweep_pipeline<0>(c, (hipStream_t)stream, /*single=*/true);
    if (rc != GPTQ_OK) return rc;
    return check.finish();
}

extern "C" int gptq_ladder_q2(const float* W, const uint8_t* dead, int64_t rows, int64_t n,
                              float* lost, float* tab, void* stream) {
    if (rows <= 0 || n < 32 || n % 32 != 0 || !W || !dead || !lost || !tab) return GPTQ_EINVAL;
    if (rows > ((int64_t)1 << 31) - 1 || !al16(W)) return GPTQ_EINVAL;  // rows read as float4
    CheckScope check;
    check_buffer(W, sizeof(float) * (size_t)(rows * n), "W");
    check_buffer(dead, (size_t)n, "dead");
    check_buffer(lost, sizeof(float) * (size_t)(rows * 2), "lost");
    check_buffer(tab, sizeof(float) * (size_t)(rows * 32), "tab");
    const int rc = ladder_launch(true, W, dead, rows, n, lost, tab, (hipStream_t)stream);
    if (rc != GPTQ_OK) return rc;
    return check.finish();
}

namespace gptq {

int sweep_q2_run(const float* W, const float* U, const float* hdiag, const uint8_t* dead,
                 const float* tab, int64_t rows, int64_t n, uint8_t* plane, uint8_t* rung,
                 float* scale, float* E, void* workspace, size_t workspace_bytes, hipStream_t st,
                 bool single) {
    if (rows <= 0 || n < 32 || n % 32 != 0 || !W || !U || !hdiag || !dead || !tab || !plane ||
        !rung || !scale || !workspace)
        return GPTQ_EINVAL;
    if (rows > ((int64_t)1 << 31) - 64 || n > ((int64_t)1 << 24)) return GPTQ_EINVAL;
    if (!al16(W) || !al16(U) || !al16(E) || !al16(workspace)) return GPTQ_EINVAL;
    size_t off_e = 0;
    if (workspace_bytes < sweep_ws(rows, n, &off_e)) return GPTQ_EWORKSPACE;
    CheckScope check;
    check_buffer(W, sizeof(float) * (size_t)(rows * n), "W");
    check_buffer(U, sizeof(float) * (size_t)(n * n), "U");
    check_buffer(hdiag, sizeof(float) * (size_t)n, "hdiag");
    check_buffer(dead, (size_t)n, "dead");
    check_buffer(tab, sizeof(float) * (size_t)(rows * 32), "tab");
    check_buffer(plane, (size_t)(rows * (n / 4)), "plane");
    check_buffer(rung, (size_t)(rows * (n / 32)), "rung");
    check_buffer(scale, sizeof(float) * (size_t)(rows * (n / 32)), "scale");
    if (E) check_buffer(E, sizeof(float) * (size_t)(rows * n), "E");
    check_buffer(workspace, workspace_bytes, "workspace");
    SweepRun c{};
    c.first = W;
    c.U = U;
    c.hdiag = hdiag;
    c.dead = dead;
    c.tab = tab;
    c.lost = nullptr;  // the q2tp rule searches every rung: no nominal rung, no lo / step
    c.rows = rows;
    c.n = n;
    c.nib = plane;
    c.rung = rung;
    c.scale = scale;
    c.E = E;
    c.Wc = (float*)workspace;
    c.Epan[0] = (float*)((char*)workspace + off_e);
    c.Epan[1] = (float*)((char*)workspace + off_e + align256(sizeof(float) * (size_t)(rows * SOB)));
    const int rc = sweep_pipeline<2>(c, st, single);
    if (rc != GPTQ_OK) return rc;
    return check.finish();
}

}  // namespace gptq

extern "C" int gptq_sweep_q2(const float* W, const float* U, const float* hdiag,
                             const uint8_t* dead, const float* tab, int64_t rows, int64_t n,
                             uint8_t* plane, uint8_t* rung, float* scale, float* E,
                             void* workspace, size_t workspace_bytes, void* stream) {
    return sweep_q2_run(W, U, hdiag, dead, tab, rows, n, plane, rung, scale, E, workspace,
                        workspace_bytes, (hipStream_t)stream, false);
}

// --- act order (static groups) -------------------------------------------------------------

// Wc[r][a] = W[r][perm[a]] (0 for a dead channel) and sp[r][a] = scale[r][perm[a] / 32]; an
// index outside 0..n-1 reads as a dead channel, so a malformed perm cannot reach outside W.
__global__ __launch_bounds__(256) void act_gather_kernel(const float* __restrict__ W,
                                                         const uint8_t* __restrict__ dead,
                                                         const int32_t* __restrict__ perm,
                                                         const float* __restrict__ scale,
                                                         int64_t n, float* __restrict__ Wc,
                                                         float* __restrict__ sp) {
    const int64_t r = blockIdx.y;
    const int64_t a = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (a >= n) return;
    const int64_t pa = perm[a];
    const bool ok = pa >= 0 && pa < n;
    Wc[r * n + a] = (ok && !dead[pa]) ? W[r * n + pa] : 0.0f;
    sp[r * n + a] = ok ? scale[r * (n / 32) + pa / 32] : 0.0f;
}

// inv[perm[a]] = a, after inv is set to -1 (so that a channel no entry of perm names stays -1).
__global__ void act_inverse_kernel(const int32_t* __restrict__ perm, int64_t n,
                                   int32_t* __restrict__ inv, int phase) {
    const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (a >= n) return;
    if (phase == 0) {
        inv[a] = -1;
    } else {
        const int64_t pa = perm[a];
        if (pa >= 0 && pa < n) inv[pa] = (int32_t)a;
    }
}

// Nibble plane from the codes in elimination order: column 2m in the low nibble.
__global__ __launch_bounds__(256) void act_pack_kernel(const uint8_t* __restrict__ codes,
                                                       const int32_t* __restrict__ inv, int64_t n,
                                                       uint8_t* __restrict__ nib) {
    const int64_t r = blockIdx.y;
    const int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (m >= n / 2) return;
    const int32_t i0 = inv[2 * m], i1 = inv[2 * m + 1];
    const uint8_t c0 = (i0 >= 0 && i0 < n) ? codes[r * n + i0] : 8;
    const uint8_t c1 = (i1 >= 0 && i1 < n) ? codes[r * n + i1] : 8;
    nib[r * (n / 2) + m] = (uint8_t)((c0 & 15u) | ((c1 & 15u) << 4));
}

// The 2-bit plane from the levels in elimination order: column 4m + i in bits 2i of byte m (a
// channel no entry of perm names gets level 0).
__global__ __launch_bounds__(256) void act_pack_q2_kernel(const uint8_t* __restrict__ codes,
                                                          const int32_t* __restrict__ inv,
                                                          int64_t n, uint8_t* __restrict__ plane) {
    const int64_t r = blockIdx.y;
    const int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (m >= n / 4) return;
    uint32_t b = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int32_t a = inv[4 * m + i];
        const uint32_t q = (a >= 0 && a < n) ? (codes[r * n + a] & 3u) : 0u;
        b |= q << (2 * i);
    }
    plane[r * (n / 4) + m] = (uint8_t)b;
}

static size_t act_ws(int64_t rows, int64_t n, size_t* off_e, size_t* off_sp, size_t* off_codes,
                     size_t* off_inv) {
    size_t o = sweep_ws(rows, n, off_e);
    if (off_sp) *off_sp = o;
    o += align256(sizeof(float) * (size_t)(rows * n));
    if (off_codes) *off_codes = o;
    o += align256((size_t)(rows * n));
    if (off_inv) *off_inv = o;
    o += align256(sizeof(int32_t) * (size_t)n);
    return o;
}

extern "C" size_t gptq_sweep_act_order_workspace_size(int64_t rows, int64_t n) {
    if (rows <= 0 || n <= 0) return 0;
    return act_ws(rows, n, nullptr, nullptr, nullptr, nullptr);
}

// The act-order sweep with static groups, 4-bit (q4tp: the static rung from the ladder's nominal
// window with unit weights; lost is read) or 2-bit (q2tp: the static rung from the full search
// with max(H_ii, 0) weights; hdiag, in elimination order, is read).  out is the nibble plane or
// the 2-bit plane.
static int act_order_impl(const float* W, const float* U, const uint8_t* dead, const int32_t* perm,
                          const float* tab, const float* lost, const float* hdiag, bool two_bit,
                          int64_t rows, int64_t n, uint8_t* out, uint8_t* rung, float* scale,
                          float* E, void* workspace, size_t workspace_bytes, void* stream) {
    if (rows <= 0 || n < 32 || n % 32 != 0 || !W || !U || !dead || !perm || !tab ||
        (two_bit ? !hdiag : !lost) || !out || !rung || !scale || !workspace)
        return GPTQ_EINVAL;
    if (rows > 65535 || n > ((int64_t)1 << 24)) return GPTQ_EINVAL;  // rows index grid.y
    if (!al16(W) || !al16(U) || !al16(E) || !al16(workspace)) return GPTQ_EINVAL;
    size_t off_e = 0, off_sp = 0, off_codes = 0, off_inv = 0;
    if (workspace_bytes < act_ws(rows, n, &off_e, &off_sp, &off_codes, &off_inv))
        return GPTQ_EWORKSPACE;
    CheckScope check;
    const int64_t obytes = two_bit ? n / 4 : n / 2;  // output plane bytes per row
    check_buffer(W, sizeof(float) * (size_t)(rows * n), "W");
    check_buffer(U, sizeof(float) * (size_t)(n * n), "U");
    check_buffer(dead, (size_t)n, "dead");
    check_buffer(perm, sizeof(int32_t) * (size_t)n, "perm");
    check_buffer(tab, sizeof(float) * (size_t)(rows * 32), "tab");
    if (two_bit) check_buffer(hdiag, sizeof(float) * (size_t)n, "hdiag");
    else check_buffer(lost, sizeof(float) * (size_t)(rows * 2), "lost");
    check_buffer(out, (size_t)(rows * obytes), "plane");
    check_buffer(rung, (size_t)(rows * (n / 32)), "rung");
    check_buffer(scale, sizeof(float) * (size_t)(rows * (n / 32)), "scale");
    if (E) check_buffer(E, sizeof(float) * (size_t)(rows * n), "E");
    check_buffer(workspace, workspace_bytes, "workspace");
    hipStream_t st = (hipStream_t)stream;
    char* ws = (char*)workspace;
    float* Wc = (float*)ws;
    float* sp = (float*)(ws + off_sp);
    uint8_t* codes = (uint8_t*)(ws + off_codes);
    int32_t* inv = (int32_t*)(ws + off_inv);
    const int64_t ng = n / 32;
    {
        ProfScope ps(FAM_SWEEP_GROUP, st, 0.0, 4.0 * (double)rows * n);
        const unsigned grid = (unsigned)((rows * ng + 255) / 256);
        GPTQ_LAUNCH(st, "act_inverse_clear",
                    (act_inverse_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(perm, n, inv, 0)),
                    wr(inv, n, 1, n));
        GPTQ_LAUNCH(st, "act_inverse",
                    (act_inverse_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(perm, n, inv, 1)),
                    rd(perm, n, 1, n), wr(inv, n, 1, n));
        if (two_bit) {
            GPTQ_LAUNCH(st, "static_rungs_q2",
                        (static_rung_q2_kernel<<<grid, 256, 0, st>>>(W, dead, hdiag, inv, tab, rows, n,
                                                                     rung, scale)),
                        rd(W, n, rows, n), rd(dead, n, 1, n, 1), rd(hdiag, n, 1, n), rd(inv, n, 1, n),
                        rd(tab, 32, rows, 32), wr(rung, ng, rows, ng, 1), wr(scale, ng, rows, ng));
        } else {
            GPTQ_LAUNCH(st, "static_rungs",
                        (static_rung_kernel<<<grid, 256, 0, st>>>(W, dead, tab, lost, rows, n, rung, scale)),
                        rd(W, n, rows, n), rd(dead, n, 1, n, 1), rd(tab, 32, rows, 32),
                        rd(lost, 2, rows, 2), wr(rung, ng, rows, ng, 1), wr(scale, ng, rows, ng));
        }
        GPTQ_LAUNCH(st, "act_gather",
                    (act_gather_kernel<<<dim3((unsigned)((n + 255) / 256), (unsigned)rows), 256, 0, st>>>(
                        W, dead, perm, scale, n, Wc, sp)),
                    rd(W, n, rows, n), rd(dead, n, 1, n, 1), rd(perm, n, 1, n),
                    rd(scale, ng, rows, ng), wr(Wc, n, rows, n), wr(sp, n, rows, n));
    }
    if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
    SweepRun c{};
    c.first = Wc;
    c.U = U;
    c.hdiag = nullptr;
    c.dead = dead;
    c.tab = tab;
    c.lost = lost;
    c.rows = rows;
    c.n = n;
    c.nib = out;
    c.rung = rung;
    c.scale = scale;
    c.E = E;
    c.Wc = Wc;
    c.Epan[0] = (float*)(ws + off_e);
    c.Epan[1] = (float*)(ws + off_e + align256(sizeof(float) * (size_t)(rows * SOB)));
    c.sp = sp;
    c.codes = codes;
    int rc = two_bit ? sweep_pipeline<3>(c, st) : sweep_pipeline<1>(c, st);
    if (rc != GPTQ_OK) return rc;
    {
        ProfScope ps(FAM_SWEEP_GROUP, st, 0.0, 1.5 * (double)rows * n);
        if (two_bit) {
            GPTQ_LAUNCH(st, "act_pack_q2",
                        (act_pack_q2_kernel<<<dim3((unsigned)((n / 4 + 255) / 256), (unsigned)rows), 256, 0, st>>>(
                            codes, inv, n, out)),
                        rd(codes, n, rows, n, 1), rd(inv, n, 1, n), wr(out, n / 4, rows, n / 4, 1));
        } else {
            GPTQ_LAUNCH(st, "act_pack",
                        (act_pack_kernel<<<dim3((unsigned)((n / 2 + 255) / 256), (unsigned)rows), 256, 0, st>>>(
                            codes, inv, n, out)),
                        rd(codes, n, rows, n, 1), rd(inv, n, 1, n), wr(out, n / 2, rows, n / 2, 1));
        }
    }
    if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
    return check.finish();
}

extern "C" int gptq_sweep_act_order(const float* W, const float* U, const uint8_t* dead,
                                    const int32_t* perm, const float* tab, const float* lost,
                                    int64_t rows, int64_t n, uint8_t* nib, uint8_t* rung,
                                    float* scale, float* E, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    return act_order_impl(W, U, dead, perm, tab, lost, nullptr, false, rows, n, nib, rung, scale,
                          E, workspace, workspace_bytes, stream);
}

extern "C" int gptq_sweep_act_order_q2(const float* W, const float* U, const uint8_t* dead,
                                       const float* hdiag, const int32_t* perm, const float* tab,
                                       int64_t rows, int64_t n, uint8_t* plane, uint8_t* rung,
                                       float* scale, float* E, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    return act_order_impl(W, U, dead, perm, tab, nullptr, hdiag, true, rows, n, plane, rung, scale,
                          E, workspace, workspace_bytes, stream);
}
