// common.hpp -- shared host/device helpers of libgptq_mi355x: status codes, HIP error checks,
// and the optional per-kernel event timing used by the benchmark.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/gptq.h"

namespace gptq {

#define GPTQ_HIP(call)                                  \
    do {                                                \
        hipError_t e_ = (call);                         \
        if (e_ != hipSuccess) return GPTQ_EHIP;         \
    } while (0)

// Kernel families timed by the profiling hooks (include/gptq_profile.h).
enum Family {
    FAM_FOLD_UPDATE = 0,  // trailing Cholesky update + inverse update (one GEMM launch per step)
    FAM_FOLD_PANEL = 1,   // panel solve + inverse row block (one GEMM launch per step)
    FAM_FOLD_DIAG = 2,    // diagonal block factor + inverse
    FAM_FOLD_BUILD = 3,   // prep, scaling and the reversed equilibrated matrix
    FAM_FOLD_MAKEU = 4,
    FAM_SWEEP_GROUP = 5,  // rung choice + rounding + in-block feedback
    FAM_SWEEP_TRAIL = 6,  // bulk of the trailing E * U update (beyond the next panel)
    FAM_LADDER = 7,
    FAM_FOLD_NEXT = 8,    // look-ahead update of the next block column / block row
    FAM_SWEEP_NEXT = 9,   // sweep updates on the serial chain: rest of the panel, next panel
    FAM_GRAM = 10,        // Hessian accumulation H += X^T X
    FAM_DEBIAS = 11,      // output debias: symmetrised H, W H, per-row slopes
    FAM_COUNT = 12
};

// Two helper streams (non-blocking, default priority) and four events, taken from a
// per-process pool for the duration of one call so that independent calls never share one.
struct Helper {
    hipStream_t stream, stream2;
    hipEvent_t ev_a, ev_b, ev_c, ev_d;
    int device;
};
int helper_acquire(Helper* h);   // GPTQ_OK or GPTQ_EHIP
void helper_release(const Helper& h);

// Records an event pair around one launch when profiling is on; no-op otherwise.
struct ProfScope {
    int fam;
    hipStream_t s;
    double flops, bytes;
    bool on;
    void* rec;
    ProfScope(int fam, hipStream_t s, double flops, double bytes);
    ~ProfScope();
};

// Storage of a Hessian (ldh >= n: dense rows; ldh = GPTQ_PACKED_UPPER: the upper triangle
// packed by rows, element (i, j >= i) at i (2n - i + 1) / 2 + j - i).  The upper part of row i
// is contiguous in both, so element (i, j >= i) is at row(i) + j; in the packed layout row(i)
// is i (2n - i - 1) / 2, the packed offset of row i less i.  Any (i, j) inside n x n maps
// inside the buffer (for j < i to some other element of the triangle), so clamped reads that
// are never used stay in bounds.
struct HLayout {
    int64_t n, ldh;
    __host__ __device__ int64_t row(int64_t i) const {
        return ldh >= 0 ? i * ldh : (i * (2 * n - i - 1)) >> 1;
    }
    __host__ __device__ int64_t at(int64_t i, int64_t j) const { return row(i) + j; }
};
inline bool hessian_ld_ok(int64_t n, int64_t ldh) { return ldh == GPTQ_PACKED_UPPER || ldh >= n; }
// Floats a Hessian of the layout spans (n >= 1).
inline int64_t hessian_elems(int64_t n, int64_t ldh) {
    return ldh < 0 ? n * (n + 1) / 2 : (n - 1) * ldh + n;
}

// Wave priority (s_setprio, 0..3) of the kernels on a call's serial chain: the fold's diagonal
// blocks and panel products, the inverse's small steps, the sweep's blocks and in-panel products.
// The bulk updates that run beside them keep priority 0, so where both share a SIMD the chain's
// instructions issue first.  Same-box timing at n = 17408: fold 34.05 -> 33.75 ms, sweep
// 15.80 -> 15.55 ms.
constexpr int CHAIN_PRIO = 3;

// A gang: G groups of the same shape whose device data sit at the same offsets of G slots of
// memory gs bytes apart (the caller's inputs excepted).  While a GangScope is open on a
// thread, the launches it makes cover all G groups: grid dimension z is the group, and each
// kernel moves its slot pointers by blockIdx.z * gs.  Outside one, G = 1 and gs = 0.
constexpr int kMaxGang = 16;
struct Gang {
    int G;
    int64_t gs;
};
Gang gang_current();
struct GangScope {
    GangScope(int G, int64_t gs);
    ~GangScope();
    GangScope(const GangScope&) = delete;
    GangScope& operator=(const GangScope&) = delete;
};
// Launch grid with the gang's groups in z.
inline dim3 gang_grid(unsigned x, unsigned y = 1) { return dim3(x, y, (unsigned)gang_current().G); }
// Pointer p of slot 0 moved to this workgroup's slot.
template <class T>
__device__ __forceinline__ T* gang_ptr(T* p, int64_t gs) {
    // Byte arithmetic on the pointer itself (not through an integer), so that the compiler
    // still sees where it came from: a kernel argument, hence global memory, accessed with
    // global_load / global_store rather than FLAT instructions (which also count against the
    // LDS wait counter).
    using B = typename std::conditional<std::is_const<T>::value, const char, char>::type;
    return reinterpret_cast<T*>(reinterpret_cast<B*>(p) + (int64_t)blockIdx.z * gs);
}
// Per-group Hessians of a gang (the caller's buffers, not in the slots): the kernels that read
// H take entry blockIdx.z.
struct HTab {
    const float* H[kMaxGang];
    int64_t ldh[kMaxGang];
};
inline HTab htab_one(const float* H, int64_t ldh) {
    HTab t{};
    t.H[0] = H;
    t.ldh[0] = ldh;
    return t;
}

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
// 16-byte alignment, which every pointer the kernels read or write as float4 / double2 needs
// (NULL counts as aligned: optional outputs).
inline bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace gptq
