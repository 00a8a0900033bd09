// api.hip -- status strings and the optional per-kernel event timing of libgptq_mi355x.
#include <mutex>
#include <vector>

#include "../../include/gptq_profile.h"
#include "check.hpp"
#include "common.hpp"

namespace gptq {

namespace {
struct Rec {
    hipEvent_t a, b;
    int fam;
    double flops, bytes;
};
std::mutex g_mu;
unsigned g_mask = 0u;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;
std::mutex g_hmu;
std::vector<Helper> g_helpers;

hipEvent_t take_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    // Timing only: no system-scope fence when the event is recorded (the cache writeback it
    // would force lands between the kernels being timed).
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
}
}  // namespace

int helper_acquire(Helper* h) {
    if (dry_run()) {
        *h = Helper{dry_stream(1), dry_stream(2), dry_event(1), dry_event(2), dry_event(3), dry_event(4), -1};
        return GPTQ_OK;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GPTQ_EHIP;
    {
        std::lock_guard<std::mutex> lk(g_hmu);
        for (size_t i = 0; i < g_helpers.size(); ++i)
            if (g_helpers[i].device == dev) {
                *h = g_helpers[i];
                g_helpers.erase(g_helpers.begin() + (long)i);
                return GPTQ_OK;
            }
    }
    Helper n{};
    n.device = dev;
    if (hipStreamCreateWithFlags(&n.stream, hipStreamNonBlocking) != hipSuccess ||
        hipStreamCreateWithFlags(&n.stream2, hipStreamNonBlocking) != hipSuccess)
        return GPTQ_EHIP;
    // The helper events only order streams of one device (a stream waits for another's
    // kernels), so they record without the system-scope fence, which would also write the
    // caches back for the host and other devices at every record: about 0.1 ms per fold and per
    // sweep at n = 17408.  Visibility between streams of the device comes from the kernels' own
    // device-scope release and acquire.
    const unsigned ef = hipEventDisableTiming | hipEventDisableSystemFence;
    if (hipEventCreateWithFlags(&n.ev_a, ef) != hipSuccess ||
        hipEventCreateWithFlags(&n.ev_b, ef) != hipSuccess ||
        hipEventCreateWithFlags(&n.ev_c, ef) != hipSuccess ||
        hipEventCreateWithFlags(&n.ev_d, ef) != hipSuccess)
        return GPTQ_EHIP;
    *h = n;
    return GPTQ_OK;
}

void helper_release(const Helper& h) {
    if (h.device < 0) return;  // a dry run's stand-in
    std::lock_guard<std::mutex> lk(g_hmu);
    g_helpers.push_back(h);
}

ProfScope::ProfScope(int fam_, hipStream_t s_, double flops_, double bytes_)
    : fam(fam_), s(s_), flops(flops_), bytes(bytes_), on(false), rec(nullptr) {
    if (dry_run()) return;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!(g_mask >> fam & 1u)) return;
    Rec* r = new Rec{take_event(), take_event(), fam, flops, bytes};
    if (!r->a || !r->b) {
        delete r;
        return;
    }
    hipEventRecord(r->a, s);
    rec = r;
    on = true;
}

ProfScope::~ProfScope() {
    if (!on) return;
    Rec* r = (Rec*)rec;
    hipEventRecord(r->b, s);
    std::lock_guard<std::mutex> lk(g_mu);
    g_recs.push_back(*r);
    delete r;
}

}  // namespace gptq

using namespace gptq;

extern "C" const char* gptq_status_string(int status) {
    switch (status) {
        case GPTQ_OK: return "ok";
        case GPTQ_EINVAL: return "invalid argument";
        case GPTQ_EWORKSPACE: return "workspace too small";
        case GPTQ_EHIP: return "HIP runtime error";
        case GPTQ_DEGENERATE: return "damping passed 10 without a factor; U = I";
        case GPTQ_ECHECK: return "schedule check failed (check mode)";
        case GPTQ_ETOOBIG: return "more rows than the no-allocation sweep's static scratch holds (8192)";
        default: return "unknown status";
    }
}

extern "C" void gptq_profile_enable(unsigned family_mask) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_mask = family_mask;
}

extern "C" int gptq_profile_collect(double* ms, int64_t* launches, double* flops, double* bytes,
                                    int nfam) {
    std::vector<Rec> recs;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        recs.swap(g_recs);
    }
    for (int f = 0; f < nfam; ++f) {
        ms[f] = 0.0;
        launches[f] = 0;
        flops[f] = 0.0;
        bytes[f] = 0.0;
    }
    int status = GPTQ_OK;
    for (const Rec& r : recs) {
        float t = 0.0f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
            status = GPTQ_EHIP;
        if (r.fam >= 0 && r.fam < nfam) {
            ms[r.fam] += t;
            launches[r.fam] += 1;
            flops[r.fam] += r.flops;
            bytes[r.fam] += r.bytes;
        }
    }
    std::lock_guard<std::mutex> lk(g_mu);
    for (const Rec& r : recs) {
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    return status;
}

extern "C" int gptq_profile_family_count(void) { return FAM_COUNT; }

extern "C" const char* gptq_profile_family_name(int fam) {
    static const char* names[FAM_COUNT] = {"fold_update", "fold_panel", "fold_diag", "fold_build",
                                           "fold_make_u", "sweep_group", "sweep_trail", "ladder",
                                           "fold_next", "sweep_next", "gram", "debias"};
    return (fam >= 0 && fam < FAM_COUNT) ? names[fam] : "?";
}
