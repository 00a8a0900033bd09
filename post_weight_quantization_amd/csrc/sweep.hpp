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

}  // namespace gptq
