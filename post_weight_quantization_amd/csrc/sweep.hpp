// sweep.hpp -- the sweeps' stream-level forms (sweep.hip) for the library's own callers: the
// argument checks and results of gptq_sweep / gptq_sweep_q2, on a hipStream_t, with `single`
// keeping every launch on that stream (no helper stream or event; the same results bit for bit).
#pragma once
#include <stdint.h>

#include "common.hpp"

namespace gptq {

int sweep_run(const float* W, const float* U, const float* hdiag, const uint8_t* dead,
              const float* tab, const float* lost, int64_t rows, int64_t n, uint8_t* nib,
              uint8_t* rung, float* scale, float* E, void* workspace, size_t workspace_bytes,
              hipStream_t st, bool single);
int sweep_q2_run(const float* W, const float* U, const float* hdiag, const uint8_t* dead,
                 const float* tab, int64_t rows, int64_t n, uint8_t* plane, uint8_t* rung,
                 float* scale, float* E, void* workspace, size_t workspace_bytes, hipStream_t st,
                 bool single);

// Bytes of one residual panel buffer of a sweep of `rows` rows (the workspace holds the working
// copy, then two of these).
size_t sweep_panel_bytes(int64_t rows);

// A gang of G matrices of the same shape (common.hpp: slots gs bytes apart; every pointer is
// slot 0's): the ladder (q4tp, or q2tp when q2) of each working copy Wc, then its sweep in
// place, on st and a helper stream.  Each group's outputs are those of gptq_ladder and
// gptq_sweep (gptq_ladder_q2 and gptq_sweep_q2) on that matrix, bit for bit.
int sweep_gang(int G, int64_t gs, bool q2, float* Wc, const float* U, const float* hdiag,
               const uint8_t* dead, float* lost, float* tab, int64_t rows, int64_t n, uint8_t* nib,
               uint8_t* rung, float* scale, float* pan0, float* pan1, hipStream_t st);

}  // namespace gptq
