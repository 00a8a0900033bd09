/*
 * gptq.h -- C ABI of the MI355X (gfx950) GPTQ fold-and-quantize library, libgptq_mi355x.so.
 *
 * Two calls make the method, plus the per-row ladder that the sweep consumes:
 *
 *   gptq_fold   : H (Hessian of one layer's inputs)  ->  U, the upper Cholesky factor of
 *                 H_d^-1 with H_d = H' + lambda*mean(diag)*I (dead channels zeroed, unit
 *                 diagonal).  Source: page "cortiq-engine 0.8.41 src/gpu_wgpu/gptq_dev.rs",
 *                 module documentation steps 1-4 and the driver `fold`; page "cortiq-cli 0.8.45
 *                 src/gptq.rs", `gptq_fold_operator_par` (same operator on the host).
 *   gptq_ladder : W -> per-row (lo, step) and the 32 rung scales TAB[c] = 2^(lo + c*step).
 *                 The pages take this from a converter whose rule is not printed; the rule
 *                 implemented is stated at the declaration below.
 *   gptq_sweep  : W, U -> 4-bit codes, one f32 scale per (row, 32-column group), and the scaled
 *                 residuals E.  Source: page "cortiq-engine 0.8.41 src/gpu_wgpu/gptq_dev.rs",
 *                 module documentation step 5, kernels `q4tp_group` / `q4tp_trail`; page
 *                 "cortiq-cli 0.8.45 src/gptq.rs", `gptq_quantize_q4tp`.
 *
 * Conventions shared by every call:
 *   - Matrices are row-major f32.  Every pointer argument except `report` is DEVICE memory
 *     owned by the caller; the library allocates nothing and keeps no per-call state.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued on it.
 *     gptq_fold and gptq_sweep also run parts of it on helper streams of the library's own
 *     (default priority, two per concurrent call) that wait on `stream` and are joined back
 *     into it before the call returns, so `stream` orders everything the call does.
 *   - Return value: a GPTQ_* status.  On GPTQ_EINVAL or GPTQ_EWORKSPACE nothing is written.
 *   - Workspaces and the matrices a call reads or writes in rows (W, U, E) must be 16-byte
 *     aligned (GPTQ_EINVAL otherwise); device allocations are.
 *   - Calls on different streams may run concurrently if their buffers are disjoint.
 *   - A Hessian H comes with a leading dimension ldh.  ldh >= n: a dense row-major [n, ldh]
 *     matrix of which only the upper triangle (with the diagonal) is read or written.
 *     ldh = GPTQ_PACKED_UPPER: the upper triangle packed row by row, as the pages' device
 *     Hessian (page "cortiq-engine 0.8.41 src/gpu_wgpu/gptq_dev.rs", poff): element (i, j >= i)
 *     at i (2n - i + 1) / 2 + (j - i), n (n + 1) / 2 floats in all, half the dense bytes.
 *     Both layouts give the same results bit for bit.
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    GPTQ_OK = 0,
    GPTQ_EINVAL = 1,      /* bad size or null required pointer */
    GPTQ_EWORKSPACE = 2,  /* workspace smaller than the matching *_workspace_size() */
    GPTQ_EHIP = 3,        /* a HIP runtime call failed */
    GPTQ_DEGENERATE = 4,  /* the damping passed 10 without a factor: U = I was written */
    GPTQ_ECHECK = 5,      /* check mode only (gptq_check.h): the schedule failed its check */
    GPTQ_ETOOBIG = 6      /* larger than the static scratch of gptq_sweep_inplace_noalloc */
};

/* ldh of a Hessian stored as its packed upper triangle (conventions above). */
#define GPTQ_PACKED_UPPER ((int64_t)-1)

/* Host-side record of one fold. */
typedef struct {
    double lambda_used; /* damping factor of the attempt that factored; on GPTQ_DEGENERATE the
                           first schedule value past 10 */
    double base;        /* max(mean of the diagonal with dead entries counted as 1, 1e-12) */
    double damp;        /* lambda_used * base, added to the diagonal */
    int32_t attempts;   /* factorizations tried, f32 and f64 (1 when the first one factors) */
    int32_t n_dead;     /* channels with !(H_ii > 0) */
    int32_t degenerate; /* 1 when U = I was written */
    int32_t precision;  /* 32 or 64: the arithmetic of the factorization U comes from */
    double min_pivot;   /* smallest pivot of that factorization (of the unit-diagonal
                           equilibrated matrix, so in (0, 1]); 0 on GPTQ_DEGENERATE */
} gptq_fold_report;

/* Arithmetic of the fold (gptq_fold_ex).
 *   GPTQ_FOLD_AUTO  each damping value is factored in f32 first; if a pivot of the equilibrated
 *                   matrix is at or below 1e-3 (the f32 factor's error in U D grows as 6e-8 /
 *                   smallest pivot) or fails, that damping value is factored again in f64, and
 *                   every later one too.  The pivot rule is then the f64 host's, so the damping
 *                   reached equals the f64 host fold's.
 *   GPTQ_FOLD_F32   f32 only, the pages' device rule (a pivot that is not > 0, or NaN, raises
 *                   lambda).  Accurate to about 6e-8 / min_pivot.
 *   GPTQ_FOLD_F64   f64 only (f64 MFMA), the host's rule (not > 0 or not finite). */
enum { GPTQ_FOLD_AUTO = 0, GPTQ_FOLD_F32 = 1, GPTQ_FOLD_F64 = 2 };

/* Bytes of device workspace gptq_fold_ex needs for size n and a precision, with
 * n_p = n rounded up to 128: GPTQ_FOLD_F32 two n_p x n_p f32 matrices plus O(n_p * 512);
 * GPTQ_FOLD_AUTO and GPTQ_FOLD_F64 two n_p x n_p f64 matrices plus O(n_p * 512).
 * 0 for n <= 0, n > 2^20 or an unknown precision. */
size_t gptq_fold_workspace_size_ex(int64_t n, int precision);
/* gptq_fold_workspace_size_ex(n, GPTQ_FOLD_AUTO): what gptq_fold needs. */
size_t gptq_fold_workspace_size(int64_t n);

/*
 * gptq_fold_ex -- the damped, equilibrated fold of one Hessian.
 *
 *   H        [n, ldh] f32, device, or packed (ldh = GPTQ_PACKED_UPPER).  Only the UPPER
 *            triangle (j >= i) is read; a dense lower one may hold anything.  Non-finite
 *            entries are allowed: a non-finite or non-positive diagonal marks the channel dead,
 *            anything else fails pivots and raises lambda.
 *   n        channels, 1 <= n <= 2^20.  ldh >= n or GPTQ_PACKED_UPPER.
 *   lambda   starting relative damping (negative or NaN is treated as 0).  A pivot that fails
 *            (see the precisions above) restarts the factorization with lambda -> 1e-4 (from
 *            0) or lambda * 10; past 10 the call writes U = I and returns GPTQ_DEGENERATE (the
 *            round-to-nearest operator of the host fold).
 *   precision  GPTQ_FOLD_AUTO, GPTQ_FOLD_F32 or GPTQ_FOLD_F64.
 *   U        [n, n] f32 out, device: U[j][k] for k >= j, zeros below the diagonal.
 *   hdiag    [n] f32 out, device: the raw H_ii (the sweep's rung-search weights).
 *   dead     [n] u8 out, device: 1 where !(H_ii > 0).
 *   workspace / workspace_bytes: device scratch of at least
 *            gptq_fold_workspace_size_ex(n, precision).
 *   stream   hipStream_t.
 *   report   host pointer (may be NULL).
 *
 * Steps on the device: diagonal, dead mask and mean (f64) -> per attempt: D_i^-1 =
 * (H_ii + damp)^-1/2 (dead: (1 + damp)^-1/2), the reversed equilibrated matrix
 * A = P D^-1 H_d D^-1 P, blocked Cholesky A = L L^T and the blocked right-looking inverse
 * X = L^-1 (in f32 pipelined on the helper streams one 512-column panel behind; in f64
 * trailing each 256-column panel) -> U = P X P D^-1.  The host reads the pivot flag once per
 * attempt (one stream synchronisation); U is still being written when the call returns.
 * Sources: page "cortiq-engine 0.8.41 src/gpu_wgpu/gptq_dev.rs", module documentation steps
 * 1-4 and the driver `fold`; page "cortiq-cli 0.8.45 src/gptq.rs", gptq_fold_operator_par.
 */
int gptq_fold_ex(const float* H, int64_t n, int64_t ldh, double lambda, int precision, float* U,
                 float* hdiag, uint8_t* dead, void* workspace, size_t workspace_bytes,
                 void* stream, gptq_fold_report* report);

/* gptq_fold_ex with precision GPTQ_FOLD_AUTO. */
int gptq_fold(const float* H, int64_t n, int64_t ldh, double lambda, float* U, float* hdiag,
              uint8_t* dead, void* workspace, size_t workspace_bytes, void* stream,
              gptq_fold_report* report);

/*
 * gptq_ladder -- per-row rung ladder from the dead-zeroed weights, groups of 32 columns.
 *
 *   W      [rows, n] f32, device (n % 32 == 0).   dead [n] u8, device (dead columns ignored).
 *   lost   [rows, 2] f32 out: (lo, step), both binary16 values.
 *   tab    [rows, 32] f32 out: TAB[c] = f32(2^(lo + c*step)), evaluated in f64.
 *
 * Rule (a stated reading; the pages' converter is not printed): with a_g the absmax of group g
 * and only a_g > 0 counted, lo = f16(log2(min a_g / 7)), hi = log2(max a_g / 7),
 * step = f16((hi - lo) / 31) when hi > lo else 0 (a non-positive rounded step is 0); a row with
 * no nonzero group gets lo = 0, step = 0, TAB = 1.  f16 rounding is to nearest, ties to even.
 * Asynchronous.
 */
int gptq_ladder(const float* W, const uint8_t* dead, int64_t rows, int64_t n, float* lost,
                float* tab, void* stream);

/* Bytes of device workspace gptq_sweep needs: the corrected working copy of W (rows x n f32)
 * plus two panel buffers of residuals (rows x 512 f32 each). */
size_t gptq_sweep_workspace_size(int64_t rows, int64_t n);

/*
 * gptq_sweep -- the q4tp GPTQ sweep of W against a fold.
 *
 *   W      [rows, n] f32, device, read only (dead columns are treated as zero).  Finite.
 *   U      [n, n] f32, device: the fold's output.   hdiag [n] f32, dead [n] u8: the fold's.
 *   tab    [rows, 32] f32, lost [rows, 2] f32: the ladder (gptq_ladder's layout).
 *   rows >= 1; n >= 32 with n % 32 == 0.
 *   nib    [rows, n/2] u8 out: 4-bit codes q + 8 (q in -8..7); column 2m in the low nibble of
 *          byte m, 2m+1 in the high nibble (each (row, group) is one 16-byte tile).
 *   rung   [rows, n/32] u8 out: the chosen rung c.   scale [rows, n/32] f32 out: TAB[row][c].
 *   E      [rows, n] f32 out or NULL: scaled residuals e_j = (w_j - q_j s) / U_jj.
 *   workspace / workspace_bytes: at least gptq_sweep_workspace_size(rows, n).
 *
 * Per group of 32 columns and row: the rung is chosen from the corrected tile (nominal from
 * its absmax, best of nominal-2 .. nominal+1 by the H_ii-weighted error of round-to-nearest-
 * even codes, strict improvement, lowest wins ties), then the columns are rounded in order
 * with error feedback inside the group.  The residuals of a block of up to 4 groups reach the
 * rest of the block column by column, the rest of its 512-column panel through one f32 MFMA
 * GEMM, W[:, c1:p1] -= E[:, c0:c1] U[c0:c1, c1:p1], and the columns right of the panel through
 * one K = 512 GEMM per panel, W[:, p1:] -= E[:, p0:p1] U[p0:p1, p1:].  Asynchronous.
 */
int gptq_sweep(const float* W, const float* U, const float* hdiag, const uint8_t* dead,
               const float* tab, const float* lost, int64_t rows, int64_t n, uint8_t* nib,
               uint8_t* rung, float* scale, float* E, void* workspace, size_t workspace_bytes,
               void* stream);

/* Bytes of device workspace gptq_sweep_inplace needs without E: two rows x 512 f32 panel
 * buffers of residuals.  (With E it needs none.) */
size_t gptq_sweep_inplace_workspace_size(int64_t rows, int64_t n);

/*
 * gptq_sweep_inplace -- gptq_sweep with W as its own working copy: the same codes, rungs,
 * scales and residuals, bit for bit, without the rows x n copy (356 MB at 5120 x 17408).
 *
 *   W      [rows, n] f32, device, IN/OUT: read as gptq_sweep reads it, then overwritten by the
 *          sweep's partially corrected weights (no meaning to the caller; keep a copy of W if it
 *          is still needed).
 *   E      [rows, n] f32 out or NULL.  With E the residuals are written straight into it and
 *          workspace may be NULL (workspace_bytes 0); without E the workspace holds them,
 *          at least gptq_sweep_inplace_workspace_size(rows, n) bytes.
 *   Every other argument as gptq_sweep.  Asynchronous.
 */
int gptq_sweep_inplace(float* W, const float* U, const float* hdiag, const uint8_t* dead,
                       const float* tab, const float* lost, int64_t rows, int64_t n, uint8_t* nib,
                       uint8_t* rung, float* scale, float* E, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * gptq_sweep_inplace_noalloc -- gptq_sweep_inplace for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that forbid allocation).
 * It allocates nothing and creates no stream or event: the residual panels live in a static
 * device array of the library, 2 x 8192 x 512 f32 = 32 MiB on each GPU it runs on (held until
 * the process ends), and every launch goes on `stream`.
 *   Arguments as gptq_sweep_inplace, without the workspace.  Without E, rows <= 8192, else
 *   GPTQ_ETOOBIG (nothing written); with E the static array is not used and rows is free.
 *   Results equal gptq_sweep_inplace's bit for bit.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on different
 *   streams, or from several threads) race.  Asynchronous.
 */
int gptq_sweep_inplace_noalloc(float* W, const float* U, const float* hdiag, const uint8_t* dead,
                               const float* tab, const float* lost, int64_t rows, int64_t n,
                               uint8_t* nib, uint8_t* rung, float* scale, float* E, void* stream);

/*
 * gptq_gram_add -- accumulate one batch of layer inputs into the device Hessian.
 * Source: page "cortiq-cli 0.8.45 src/gptq.rs" (calibration adds every window's inputs to a
 * device Hessian, gram_add_dev; the test device_fold_and_sweep_match_host accumulates
 * h[i][j] += x[r][i] x[r][j] over the rows of x [t, n]); the fold reads the upper triangle.
 *
 *   H      [n, ldh] f32, device, in/out: H[i][j] += sum_{k < t} X[k][i] X[k][j] for j >= i
 *          (the upper triangle with the diagonal, which gptq_fold reads).  A dense lower
 *          triangle is neither read nor written.  ldh = GPTQ_PACKED_UPPER accumulates into the
 *          packed upper triangle, the pages' device layout, with the same values bit for bit.
 *          f32 products, f32 MFMA accumulation (the pages' device Hessian is f32).
 *   n      channels: 4 <= n, n % 4 == 0, ldh >= n or GPTQ_PACKED_UPPER.
 *   X      [t, ldx] f32, device, row-major: one row per token, column i = input channel i;
 *          16-byte aligned, ldx >= n, ldx % 4 == 0.  Read only.
 *   t      tokens in this batch, >= 0 (0: nothing is done and X may be NULL).  Any t: the
 *          last block of 32 tokens is zero-filled.
 * Returns GPTQ_OK, GPTQ_EINVAL (nothing written) or GPTQ_EHIP.  Asynchronous on `stream`.
 */
int gptq_gram_add(float* H, int64_t n, int64_t ldh, const float* X, int64_t t, int64_t ldx,
                  void* stream);

/* Bytes of device workspace gptq_debias needs: n x n f32 (the symmetrised Hessian) plus
 * rows x n f32 (W H).  0 for rows <= 0 or n <= 0. */
size_t gptq_debias_workspace_size(int64_t rows, int64_t n);

/*
 * gptq_debias -- output debias of a quantized layer in the calibration metric.
 * Source: page "cortiq-cli 0.8.45 src/gptq.rs", q4tp_debias_hessian / q2tp_debias_hessian and
 * their GEMM form debias_gemm: per row, the regression slope b = (W^ H W^T)_rr / (W H W^T)_rr
 * is removed through the row's f16 lo; codes, rungs and steps stay.  The helper that applies b
 * is not printed on the pages; the reading implemented: lo <- f16(lo - log2 b) (round to
 * nearest even), kept when num or den is not positive and finite.
 *
 *   W      [rows, n] f32, device: the original weights (dead columns read as 0).
 *   H      [n, ldh] f32, device, or packed (ldh = GPTQ_PACKED_UPPER): the raw Hessian, upper
 *          triangle read (as gptq_fold).  Dead channels (dead[i] != 0) count as zero rows and
 *          columns.
 *   dead   [n] u8, device (gptq_fold's output).
 *   nib, rung   gptq_sweep's codes: nibble plane [rows, n/2] and rungs [rows, n/32].
 *   lost   [rows, 2] f32, device, in/out: (lo, step); lo is replaced.
 *   tab    [rows, 32] f32 out or NULL: the row's new rung scales f32(2^(lo + c*step)) (f64).
 *   scale  [rows, n/32] f32, device, in/out: in, the scales the codes were made with (W^ =
 *          (nib - 8) * scale); out, TAB_new[rung].
 *   slope  [rows] f64 out or NULL: b = num / den (num, den summed in f64 over f32 products;
 *          W H is an f32 MFMA product, as the pages' GEMM form).
 *   n % 32 == 0.  Workspace: gptq_debias_workspace_size(rows, n).
 * Returns GPTQ_OK, GPTQ_EINVAL / GPTQ_EWORKSPACE (nothing written) or GPTQ_EHIP.
 * Asynchronous on `stream`.
 */
int gptq_debias(const float* W, const float* H, int64_t ldh, const uint8_t* dead,
                const uint8_t* nib, const uint8_t* rung, float* lost, float* tab, float* scale,
                double* slope, int64_t rows, int64_t n, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * Act-order GPTQ.  Source: page "cortiq-cli 0.8.45 src/gptq.rs": act_order_perm, permute_sym,
 * gptq_quantize_q4tp_act_order.  The flow: gptq_act_order_perm(H) -> perm, dead;
 * gptq_permute_hessian(H, perm) -> Hp; gptq_fold(Hp) -> Up (elimination order);
 * gptq_ladder(W, dead); gptq_sweep_act_order(W, Up, dead, perm, ...).
 *
 * gptq_act_order_perm: perm [n] i32 out, the channels by descending H_ii compared in the f32
 *   total order (-NaN < -inf < ... < -0 < +0 < ... < +inf < +NaN), ties by ascending index;
 *   dead [n] u8 out, 1 where !(H_ii > 0) (original order).  H [n, ldh] f32 or packed
 *   (ldh = GPTQ_PACKED_UPPER), only its diagonal is read.
 */
int gptq_act_order_perm(const float* H, int64_t n, int64_t ldh, int32_t* perm, uint8_t* dead,
                        void* stream);

/* gptq_permute_hessian: Hp [n, n] f32 out (full, symmetric, dense) = H[perm][perm], H (dense or
 * packed) read through its upper triangle (H[min][max]).  perm must be a permutation of
 * 0..n-1; an entry outside that range gives zero rows and columns. */
int gptq_permute_hessian(const float* H, int64_t n, int64_t ldh, const int32_t* perm, float* Hp,
                         void* stream);

/* Bytes of device workspace gptq_sweep_act_order needs: gptq_sweep's plus rows x n f32 (the
 * per-column scales), rows x n bytes (the codes) and n i32. */
size_t gptq_sweep_act_order_workspace_size(int64_t rows, int64_t n);

/*
 * gptq_sweep_act_order -- the q4tp sweep with the columns eliminated in perm order ("static
 * groups": a tile's channels are no longer consecutive in time, so its rung is fixed up front).
 *
 *   W      [rows, n] f32 (original channel order), read only.
 *   U      [n, n] f32: gptq_fold of gptq_permute_hessian(H, perm) (elimination order).
 *   dead   [n] u8, original order (gptq_act_order_perm's output).
 *   perm   [n] i32, the elimination order.
 *   tab, lost   gptq_ladder(W, dead).
 *   nib, rung, scale  out, as gptq_sweep (original order).  rung / scale are the static choice:
 *          the sweep's rung rule on the dead-zeroed original tile with unit weights (the
 *          pages take it from their converter, whose rule is not printed: a stated reading),
 *          the error summed in f32 in column order.
 *   E      [rows, n] f32 out (elimination order) or NULL.
 *   Per column a of the elimination order: q = clamp(rne(w_a / s_a), -8, 7) with s_a the static
 *   scale of channel perm[a]'s group, e_a = (w_a - q s_a) / U_aa, w_t -= e_a U_at for t > a.
 *   rows <= 65535, n % 32 == 0.  Workspace: gptq_sweep_act_order_workspace_size(rows, n).
 */
int gptq_sweep_act_order(const float* W, const float* U, const uint8_t* dead, const int32_t* perm,
                         const float* tab, const float* lost, int64_t rows, int64_t n,
                         uint8_t* nib, uint8_t* rung, float* scale, float* E, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * gptq_sweep_act_order_q2 -- act order with 2-bit (q2tp) codes.  Source: page "cortiq-cli 0.8.45
 * src/gptq.rs", gptq_quantize_q2tp with a permutation (the sweep's perm branch: columns in perm
 * order, each group's rung fixed up front).  The pages fix the rungs with a placement helper
 * that is handed the clipped H_ii weights and is not printed; the rule implemented (a stated
 * reading) is the q2tp sweep's own search on the dead-zeroed original tile: rung 0 for an
 * all-zero tile, else the best of rungs 1..31 (TAB > 0) by sum_t max(H_tt, 0) (w_t - (q_t - 1.5)
 * s)^2 in f32, summed in column order, a strictly smaller error replacing the current best.
 *
 *   W [rows, n] f32 (original order, 16-byte aligned), read only.  U and hdiag: gptq_fold of
 *   gptq_permute_hessian(H, perm) (hdiag [n] is H_ii in elimination order, hdiag[a] =
 *   H[perm[a]][perm[a]]).  dead [n] in original order (gptq_act_order_perm's).  perm [n] i32.
 *   tab: gptq_ladder_q2(W, dead).
 *   plane [rows, n/4] u8 out (column 4m + i in bits 2i of byte m, original order), rung / scale
 *   [rows, n/32] out (the static choice), E [rows, n] f32 out (elimination order) or NULL.
 *   Per column a of the elimination order: q = clamp(rne(clamp(w_a / s_a + 1.5, -1, 4)), 0, 3),
 *   e_a = (w_a - (q - 1.5) s_a) / U_aa, w_t -= e_a U_at for t > a.
 *   rows <= 65535, n % 32 == 0.  Workspace: gptq_sweep_act_order_workspace_size(rows, n).
 */
int gptq_sweep_act_order_q2(const float* W, const float* U, const uint8_t* dead,
                            const float* hdiag, const int32_t* perm, const float* tab,
                            int64_t rows, int64_t n, uint8_t* plane, uint8_t* rung, float* scale,
                            float* E, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gptq_debias_q2 -- gptq_debias for 2-bit codes.  Source: page "cortiq-cli 0.8.45 src/gptq.rs",
 * q2tp_debias_hessian / q2tp_debias_gemm (the pages' primary use of the debias: the MSE-optimal
 * 2-bit rounding shrinks every output).  As gptq_debias with plane [rows, n/4] (gptq_sweep_q2's
 * layout) in place of the nibbles, W^ = (q - 1.5) scale, and the q2 ladder for the new scales:
 * TAB[0] = 0, TAB[c] = f32(2^(lo + (c - 1) step)) (f64).  lo <- f16(lo - log2 b) as there.
 * Workspace: gptq_debias_workspace_size(rows, n).
 */
int gptq_debias_q2(const float* W, const float* H, int64_t ldh, const uint8_t* dead,
                   const uint8_t* plane, const uint8_t* rung, float* lost, float* tab,
                   float* scale, double* slope, int64_t rows, int64_t n, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * q2tp, the "placed" rule.  Source: page "cortiq-engine 0.8.41 src/gpu_wgpu/gptq_dev.rs",
 * q2tp_group; page "cortiq-cli 0.8.45 src/gptq.rs", sweep_q2tp / gptq_quantize_q2tp_dev.
 *
 * gptq_ladder_q2: lost [rows, 2] (lo, step, binary16 values) and tab [rows, 32] with TAB[0] = 0
 *   (the all-zero group) and TAB[c] = f32(2^(lo + (c-1) step)), c = 1..31 (f64).  The pages
 *   place this ladder with a helper that is not printed; the rule implemented is a stated
 *   reading: over the groups with a_g = max |w| > 0 of the dead-zeroed row, lo = f16(log2(min
 *   a_g / 1.5)), step = f16((log2(max a_g / 1.5) - lo) / 30) if positive, else 0; an all-zero
 *   row gets lo = step = 0 and TAB[c >= 1] = 1.  n % 32 == 0.
 */
int gptq_ladder_q2(const float* W, const uint8_t* dead, int64_t rows, int64_t n, float* lost,
                   float* tab, void* stream);

/*
 * gptq_sweep_q2: the q2tp GPTQ sweep of W against U (gptq_fold's output), groups of 32.  Per
 * group: rung 0 if every corrected weight is 0, else the best of rungs 1..31 (TAB > 0) by
 * sum_t max(H_tt, 0) (w_t - (q_t - 1.5) s)^2 (a strictly smaller error replaces the current
 * best); then per column q = clamp(rne(clamp(w / s + 1.5, -1, 4)), 0, 3), e = (w - (q - 1.5) s)
 * / U_jj, w_t -= e U_jt.  Outputs: plane [rows, n/4] bytes (column 4m + i in bits 2i of byte
 * m; level (q - 1.5) * scale), rung [rows, n/32] u8, scale [rows, n/32] f32 = TAB[rung], E
 * [rows, n] f32 or NULL.  Workspace: gptq_sweep_workspace_size(rows, n).  W is read only.
 */
int gptq_sweep_q2(const float* W, const float* U, const float* hdiag, const uint8_t* dead,
                  const float* tab, int64_t rows, int64_t n, uint8_t* plane, uint8_t* rung,
                  float* scale, float* E, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The batched round: many Hessian groups on one GPU.  A group is one Hessian and the weight
 * matrices that share it (its members); the round folds each group once and ladders and sweeps
 * every member against that fold.  Source: page "cortiq-cli 0.8.45 src/gptq.rs",
 * run_quantize_gptq_tiled (workers take whole groups, widest Hessian first -- the
 * longest-processing-time order, which changes no result -- and sweep every member of a group
 * against the group's fold) and fold_concurrency (as many groups at once as the memory budget
 * holds over one group's peak, at least one).  Here the budget is the caller's workspace and a
 * group's peak is one slot (gptq_round_slot_size).
 */
enum { GPTQ_CODEC_Q4TP = 0, GPTQ_CODEC_Q2TP = 1 };

typedef struct {
    const float* W;  /* [rows, n] f32, device, 16-byte aligned; read only */
    int64_t rows;    /* >= 1 */
    int32_t codec;   /* GPTQ_CODEC_Q4TP (gptq_ladder, gptq_sweep) or GPTQ_CODEC_Q2TP
                        (gptq_ladder_q2, gptq_sweep_q2) */
    int32_t pad;
    float* lost;     /* [rows, 2] f32 out: (lo, step) */
    float* tab;      /* [rows, 32] f32 out: the rung scales */
    uint8_t* codes;  /* out: the nibble plane [rows, n/2] (q4tp) or the 2-bit plane [rows, n/4] */
    uint8_t* rung;   /* [rows, n/32] out */
    float* scale;    /* [rows, n/32] f32 out */
} gptq_member;

typedef struct {
    const float* H;           /* the group's Hessian, device: dense [n, ldh] or packed */
    int64_t n;                /* 1 <= n <= 2^20; n % 32 == 0 when the group has members */
    int64_t ldh;              /* >= n, or GPTQ_PACKED_UPPER */
    double lambda;            /* starting damping, as gptq_fold_ex */
    int32_t precision;        /* GPTQ_FOLD_* */
    int32_t members;          /* >= 0 */
    const gptq_member* member; /* host array of `members` entries */
    float* hdiag;             /* [n] f32 out, device, or NULL */
    uint8_t* dead;            /* [n] u8 out, device, or NULL */
    gptq_fold_report report;  /* out: the group's fold */
    int32_t status;           /* out: GPTQ_OK, GPTQ_DEGENERATE (U = I; the members are swept
                                 against it), or the status of the group's first failing call */
    int32_t pad;
} gptq_group;

/* Bytes of device workspace one group occupies while it runs (a slot): U, hdiag and dead, plus
 * the larger of the fold's workspace (at the group's precision) and, over its members, a
 * sweep's workspace (gptq_sweep_workspace_size) followed by the member's outputs (lost, tab,
 * codes at n/2 bytes a row, rung, scale), where a gang stages them; fold and sweeps share the
 * memory because the sweeps follow the fold on one stream.  Each part 256-byte aligned.  The
 * maximum over the groups; 0 when a group is invalid or count <= 0. */
size_t gptq_round_slot_size(const gptq_group* groups, int32_t count);

/* The round's schedule, on the host only.  order [count] i32 out: the groups widest first
 * (larger n, then more member rows, then the lower index).  Consecutive groups of that order
 * with the same shape -- n, precision (not GPTQ_FOLD_F64), lambda, and member by member rows
 * and codec -- form gangs of at most min(max_concurrency, 16, workspace_bytes / slot size)
 * groups (max_concurrency <= 0: no cap of the caller's).  *concurrency out: the slots the round
 * uses -- its largest gang when it forms a gang of two or more, else the groups run at once on
 * threads, min(max_concurrency, count, workspace_bytes / slot size) with max_concurrency <= 0
 * meaning 4.  GPTQ_EINVAL for an invalid group or count <= 0, GPTQ_EWORKSPACE when the
 * workspace holds no slot; nothing is written then. */
int gptq_round_plan(const gptq_group* groups, int32_t count, size_t workspace_bytes,
                    int32_t max_concurrency, int32_t* order, int32_t* concurrency);

/*
 * gptq_round -- run the round.  groups: host array; each entry's report and status are
 * written.  workspace: device, 256-byte aligned, cut into slots of gptq_round_slot_size bytes.
 * When the plan forms gangs, they run one after another on `stream` (and the library's helper
 * streams, joined back into it): a gang of G groups runs in lockstep, every kernel launch
 * covering all G, each in its own slot -- one f32 fold attempt for all of them (a group whose
 * attempt fails is then folded again on its own, from the start), then member by member a copy
 * of the G weight matrices into the slots, their ladders and in-place sweeps, and the copy of
 * the outputs to the members' buffers; a lone group runs as the separate calls do.  Otherwise
 * one host thread and one stream (the library's own, default priority) per slot: a thread
 * takes the next group of the plan's order, folds it (the host reads the pivot flag once per
 * attempt), then ladders and sweeps each member on the slot's stream (with more than one slot,
 * every launch of the group on that stream, no helper streams); the slot streams start after
 * `stream`, and `stream` waits for all of them.  Either way the round is ordered on `stream`;
 * the last sweeps may still run when the call returns.  Every result is bit for bit that of
 * the separate calls (gptq_fold_ex, gptq_ladder or gptq_ladder_q2, gptq_sweep or
 * gptq_sweep_q2).  Returns GPTQ_OK when every group ended GPTQ_OK or GPTQ_DEGENERATE, else the
 * first failing group's status in the groups' order; after a GPTQ_EHIP no group is started any
 * more and those not started report GPTQ_EHIP.  The buffers of different groups must be
 * disjoint.
 */
int gptq_round(gptq_group* groups, int32_t count, void* workspace, size_t workspace_bytes,
               int32_t max_concurrency, void* stream);

/* Static string for a GPTQ_* status. */
const char* gptq_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif
