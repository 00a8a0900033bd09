// check.hpp -- schedule checking for libgptq_mi355x (dry run).
//
// In check mode (gptq_check_mode(1), include/gptq_check.h) an entry point runs its host-side
// schedule without touching the GPU: every kernel launch, event record, stream wait and host
// synchronisation goes through the functions below, which record it instead.  Each launch
// names the memory it reads and writes as 2-D spans (rows x cols elements, row stride ld).
// At the end of the call two properties are checked:
//   bounds   every span lies inside one buffer the call was given (inputs, outputs,
//            workspace), so no launch of the schedule can fault;
//   races    two launches on different streams that touch overlapping memory, one of them
//            writing, are ordered by the streams' event waits or a host synchronisation
//            (vector clocks over streams), so the multi-stream pipelines cannot race.
// Outside check mode the wrappers issue the HIP calls and the spans cost nothing.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gptq {

// Inside a gang (common.hpp) a launch touches each span once per group, the span moved by
// g * gs for group g, unless the span is fixed: memory of one group outside the slots (a
// caller's buffer), which the launch names for each group itself.
struct Span {
    const void* p;
    int64_t ld, rows, cols;  // elements
    int esize;               // bytes per element
    bool write;
    bool fixed;
};
inline Span rd(const void* p, int64_t ld, int64_t rows, int64_t cols, int esize = 4) {
    return Span{p, ld, rows, cols, esize, false, false};
}
inline Span wr(const void* p, int64_t ld, int64_t rows, int64_t cols, int esize = 4) {
    return Span{p, ld, rows, cols, esize, true, false};
}
inline Span fixed(Span s) {
    s.fixed = true;
    return s;
}
// The whole of a Hessian (f32) of either layout: its n x n rows when dense, its n (n + 1) / 2
// floats when packed (ldh < 0).
inline Span hessian_span(const void* H, int64_t n, int64_t ldh, bool write) {
    if (ldh < 0) {
        const int64_t P = n * (n + 1) / 2;
        return Span{H, P, 1, P, 4, write, false};
    }
    return Span{H, ldh, n, n, 4, write, false};
}

// True while the calling thread runs an entry point in check mode.
bool dry_run();
// True while check mode is switched on (gptq_check_mode), inside an entry point or not.
bool check_mode_on();

// One entry-point call.  In check mode the constructor starts a fresh record; finish() runs
// the checks and returns GPTQ_OK or GPTQ_ECHECK.  Outside check mode both do nothing.
struct CheckScope {
    CheckScope();
    ~CheckScope();
    int finish();
    CheckScope(const CheckScope&) = delete;
    CheckScope& operator=(const CheckScope&) = delete;
};

void check_buffer(const void* p, size_t bytes, const char* name);
// GPTQ_OK, or GPTQ_ECHECK when a span leaves every registered buffer.
int check_launch(const char* name, hipStream_t s, const Span* acc, int nacc);
int ev_record(hipEvent_t e, hipStream_t s);            // hipEventRecord
int stream_wait(hipStream_t s, hipEvent_t e);          // hipStreamWaitEvent
int launch_status();                                   // hipGetLastError (GPTQ_OK in a dry run)
void host_sync_record(hipStream_t s);                  // the host waits for s (dry run only)

// Fake stream / event handles for helper streams in a dry run.
hipStream_t dry_stream(int k);
hipEvent_t dry_event(int k);

}  // namespace gptq

// Launch a kernel after recording its accesses: LAUNCH is a parenthesised launch expression,
// the rest are Span values.  Returns the enclosing function's status on a check failure.
#define GPTQ_LAUNCH(stream, name, launch, ...)                                       \
    do {                                                                             \
        const ::gptq::Span acc_[] = {__VA_ARGS__};                                  \
        const int rc_ = ::gptq::check_launch(name, stream, acc_,                     \
                                             (int)(sizeof(acc_) / sizeof(acc_[0]))); \
        if (rc_ != GPTQ_OK) return rc_;                                              \
        if (!::gptq::dry_run()) launch;                                              \
    } while (0)
