/*
 * gptq_profile.h -- optional per-kernel timing of libgptq_mi355x (measurement only).
 *
 * For the kernel families whose bit is set in the mask, every launch is bracketed by two HIP events recorded
 * on the launch's own stream, and the algorithmic flops and bytes of that launch are noted.
 * gptq_profile_collect() waits for the recorded events and returns, per kernel family, the sum
 * of the event intervals, the launch count and the summed algorithmic flops / bytes, then
 * forgets the records.  Families (index: name):
 *   0 fold_update  bulk of the trailing Cholesky update + inverse update (one GEMM per step)
 *   1 fold_panel   panel solve + inverse row block (one GEMM launch per block step)
 *   2 fold_diag    diagonal block factor and inverse
 *   3 fold_build   prep, scaling and the reversed equilibrated matrix
 *   4 fold_make_u  U from L^-1
 *   5 sweep_group  rung choice, rounding, in-group feedback
 *   6 sweep_trail  bulk of the trailing E * U update (columns beyond the next panel)
 *   7 ladder
 *   8 fold_next    look-ahead part of the update: next block column and next block row
 *   9 sweep_next   sweep updates on the serial chain: rest of the panel, next panel
 *  10 gram         Hessian accumulation H += X^T X (gptq_gram_add)
 *  11 debias       output debias: symmetrised H, W H, per-row slopes (gptq_debias)
 * The recording adds two event records per timed launch; the mask is 0 by default.
 */
#ifndef GPTQ_MI355X_PROFILE_H
#define GPTQ_MI355X_PROFILE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

void gptq_profile_enable(unsigned family_mask); /* bit f set: time family f */
/* Arrays of length nfam (host memory).  Returns GPTQ_OK or GPTQ_EHIP. */
int gptq_profile_collect(double* ms, int64_t* launches, double* flops, double* bytes, int nfam);
int gptq_profile_family_count(void);
const char* gptq_profile_family_name(int fam);

#ifdef __cplusplus
}
#endif
#endif
