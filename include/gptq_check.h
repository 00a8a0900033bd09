/*
 * gptq_check.h -- schedule checking of libgptq_mi355x (a dry run for tests; no GPU needed).
 *
 * With check mode on, gptq_fold, gptq_ladder and gptq_sweep run their host-side schedule
 * without any HIP call: no kernel is launched, no stream or event is touched, device pointers
 * are never dereferenced (any distinct addresses of the right sizes will do) and the fold's
 * pivot flag reads as clear.  Every launch instead records the 2-D spans of memory it reads and
 * writes, and every event record / stream wait / host synchronisation is simulated with
 * vector clocks over the streams.  The call then returns GPTQ_ECHECK if
 *   - a span leaves every buffer the call was given (inputs, outputs, workspace), or
 *   - two launches on different streams touch overlapping memory, one of them writing, and
 *     neither is ordered before the other;
 * otherwise its usual status.  gptq_check_message() describes the first failure of the last
 * checked call on any thread ("" when it passed).  The mode is process-wide; calls made while
 * it is on must not expect results.
 */
#ifndef GPTQ_MI355X_CHECK_H
#define GPTQ_MI355X_CHECK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

void gptq_check_mode(int on);
const char* gptq_check_message(void);
/* The checker on a fixed hand-made schedule: 0 clean (GPTQ_OK), 1 an unordered overlapping
 * write (GPTQ_ECHECK), 2 the same ordered by an event (GPTQ_OK), 3 a read past the end of
 * its buffer (GPTQ_ECHECK). */
int gptq_check_selftest(int which);
/* The tile GEMM's map from workgroup to output tile, on the host: GPTQ_OK when the workgroups
 * of one launch over an M x N product (lower != 0: the lower tiles of an M x M product, N
 * ignored) cover every 128 x 128 tile exactly once, for each group of a batched launch (grid
 * z = 0 .. 15); GPTQ_ECHECK otherwise; GPTQ_EINVAL for sizes outside 1 .. 2^20. */
int gptq_check_tile_order(int64_t M, int64_t N, int lower);

#ifdef __cplusplus
}
#endif
#endif
