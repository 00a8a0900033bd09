// round.hip -- the batched round on one GPU (include/gptq.h, gptq_round): many Hessian groups,
// each folded once and its member weight matrices laddered and swept against that fold, as many
// groups at a time as the caller's workspace holds, the widest first.
//
// Source of the policy: page "cortiq-cli 0.8.45 src/gptq.rs", run_quantize_gptq_tiled (workers
// take whole groups in longest-processing-time order, widest Hessian first; a group's members
// are all swept against its fold) and fold_concurrency (the groups that run together: the memory
// budget over one group's peak, at least one).  Here the budget is the workspace and a group's
// peak is a slot: U, hdiag and dead, then a work area that the fold's workspace and the sweeps'
// workspaces share (the sweeps follow the fold on the same stream).
//
// Execution: one host thread and one stream per slot.  A thread takes the next group of the
// order from a shared counter, so a slot that finishes early takes the next group (list
// scheduling, the widest groups started first).  It folds the group -- the fold waits on the
// host for its pivot flag once per attempt, which is why every slot has a thread of its own --
// and then ladders and sweeps each member, all on the slot's stream.  With several slots the
// fold and the sweeps take their single-stream forms, so a slot occupies one hardware queue and
// the slots are the concurrency (on 11 groups of n = 4096 this ran 25-30% faster than slots
// that each add the calls' helper streams); a lone slot keeps the calls' helper-stream
// pipelines, which overlap a group's serial chain with its bulk updates.
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <thread>
#include <vector>

#include "check.hpp"
#include "common.hpp"
#include "fold.hpp"
#include "sweep.hpp"

namespace gptq {
namespace {

constexpr int kDefaultConcurrency = 4;

struct SlotLayout {
    size_t off_hd, off_dead, off_work, total;
};

bool member_ok(const gptq_member& m, int64_t n) {
    if (!m.W || !m.lost || !m.tab || !m.codes || !m.rung || !m.scale) return false;
    if (m.rows < 1 || m.rows > ((int64_t)1 << 31) - 64) return false;
    if (m.codec != GPTQ_CODEC_Q4TP && m.codec != GPTQ_CODEC_Q2TP) return false;
    return al16(m.W) && n % 32 == 0 && n >= 32;
}

bool group_ok(const gptq_group& g) {
    if (!g.H || g.n < 1 || g.n > ((int64_t)1 << 20) || !hessian_ld_ok(g.n, g.ldh)) return false;
    if (g.precision != GPTQ_FOLD_AUTO && g.precision != GPTQ_FOLD_F32 &&
        g.precision != GPTQ_FOLD_F64)
        return false;
    if (g.members < 0 || (g.members > 0 && !g.member)) return false;
    for (int32_t k = 0; k < g.members; ++k)
        if (!member_ok(g.member[k], g.n)) return false;
    return true;
}

SlotLayout slot_layout(const gptq_group& g) {
    const int64_t n = g.n;
    size_t work = gptq_fold_workspace_size_ex(n, g.precision);
    for (int32_t k = 0; k < g.members; ++k)
        work = std::max(work, gptq_sweep_workspace_size(g.member[k].rows, n));
    SlotLayout L{};
    size_t o = align256(sizeof(float) * (size_t)(n * n));
    L.off_hd = o;
    o += align256(sizeof(float) * (size_t)n);
    L.off_dead = o;
    o += align256((size_t)n);
    L.off_work = o;
    L.total = o + align256(work);
    return L;
}

int64_t member_rows(const gptq_group& g) {
    int64_t r = 0;
    for (int32_t k = 0; k < g.members; ++k) r += g.member[k].rows;
    return r;
}

// Widest first: larger n, then more member rows, then the lower index.
void plan_order(const gptq_group* groups, int32_t count, int32_t* order) {
    std::vector<int64_t> rows(count);
    for (int32_t i = 0; i < count; ++i) {
        order[i] = i;
        rows[i] = member_rows(groups[i]);
    }
    std::sort(order, order + count, [&](int32_t a, int32_t b) {
        if (groups[a].n != groups[b].n) return groups[a].n > groups[b].n;
        if (rows[a] != rows[b]) return rows[a] > rows[b];
        return a < b;
    });
}

// One group on one slot and stream.  The fold writes hdiag and dead into the caller's buffers
// when it gave them, else into the slot; the sweeps read them from there.
int run_group(gptq_group& g, char* slot, const SlotLayout& L, hipStream_t st, bool single) {
    float* U = (float*)slot;
    float* hd = g.hdiag ? g.hdiag : (float*)(slot + L.off_hd);
    uint8_t* dd = g.dead ? g.dead : (uint8_t*)(slot + L.off_dead);
    char* work = slot + L.off_work;
    const size_t work_bytes = L.total - L.off_work;
    const int64_t n = g.n;
    gptq_fold_report rep{};
    const int fs = fold_run(g.H, n, g.ldh, g.lambda, g.precision, U, hd, dd, work, work_bytes, st,
                            &rep, single);
    g.report = rep;
    if (fs != GPTQ_OK && fs != GPTQ_DEGENERATE) return fs;
    for (int32_t k = 0; k < g.members; ++k) {
        const gptq_member& m = g.member[k];
        int rc;
        if (m.codec == GPTQ_CODEC_Q4TP) {
            rc = gptq_ladder(m.W, dd, m.rows, n, m.lost, m.tab, st);
            if (rc == GPTQ_OK)
                rc = sweep_run(m.W, U, hd, dd, m.tab, m.lost, m.rows, n, m.codes, m.rung, m.scale,
                               nullptr, work, work_bytes, st, single);
        } else {
            rc = gptq_ladder_q2(m.W, dd, m.rows, n, m.lost, m.tab, st);
            if (rc == GPTQ_OK)
                rc = sweep_q2_run(m.W, U, hd, dd, m.tab, m.rows, n, m.codes, m.rung, m.scale,
                                  nullptr, work, work_bytes, st, single);
        }
        if (rc != GPTQ_OK) return rc;
    }
    return fs;
}

// Per-process pool of slot streams (non-blocking, default priority) with one event each.
struct SlotStream {
    hipStream_t s;
    hipEvent_t e;
    int device;
};
std::mutex g_smu;
std::vector<SlotStream> g_slots;

int slot_acquire(int dev, SlotStream* out) {
    {
        std::lock_guard<std::mutex> lk(g_smu);
        for (size_t i = 0; i < g_slots.size(); ++i)
            if (g_slots[i].device == dev) {
                *out = g_slots[i];
                g_slots.erase(g_slots.begin() + (long)i);
                return GPTQ_OK;
            }
    }
    SlotStream s{nullptr, nullptr, dev};
    if (hipStreamCreateWithFlags(&s.s, hipStreamNonBlocking) != hipSuccess) return GPTQ_EHIP;
    if (hipEventCreateWithFlags(&s.e, hipEventDisableTiming) != hipSuccess) {
        hipStreamDestroy(s.s);
        return GPTQ_EHIP;
    }
    *out = s;
    return GPTQ_OK;
}

void slot_release(const SlotStream& s) {
    std::lock_guard<std::mutex> lk(g_smu);
    g_slots.push_back(s);
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_round_slot_size(const gptq_group* groups, int32_t count) {
    if (!groups || count <= 0) return 0;
    size_t m = 0;
    for (int32_t i = 0; i < count; ++i) {
        if (!group_ok(groups[i])) return 0;
        m = std::max(m, slot_layout(groups[i]).total);
    }
    return m;
}

extern "C" int gptq_round_plan(const gptq_group* groups, int32_t count, size_t workspace_bytes,
                               int32_t max_concurrency, int32_t* order, int32_t* concurrency) {
    if (!groups || count <= 0 || !order || !concurrency) return GPTQ_EINVAL;
    const size_t slot = gptq_round_slot_size(groups, count);
    if (slot == 0) return GPTQ_EINVAL;
    if (workspace_bytes < slot) return GPTQ_EWORKSPACE;
    const int64_t cap = max_concurrency > 0 ? max_concurrency : kDefaultConcurrency;
    const int64_t fit = (int64_t)(workspace_bytes / slot);
    *concurrency = (int32_t)std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(cap, count), fit));
    plan_order(groups, count, order);
    return GPTQ_OK;
}

extern "C" int gptq_round(gptq_group* groups, int32_t count, void* workspace,
                          size_t workspace_bytes, int32_t max_concurrency, void* stream) {
    if (!workspace || ((uintptr_t)workspace & 255u) != 0) return GPTQ_EINVAL;
    std::vector<int32_t> order(count > 0 ? count : 1);
    int32_t conc = 0;
    const int rc = gptq_round_plan(groups, count, workspace_bytes, max_concurrency, order.data(), &conc);
    if (rc != GPTQ_OK) return rc;
    const size_t slot_bytes = gptq_round_slot_size(groups, count);
    std::vector<SlotLayout> layout(count);
    for (int32_t i = 0; i < count; ++i) {
        layout[i] = slot_layout(groups[i]);
        groups[i].status = GPTQ_EHIP;  // "not started" until the group runs
        groups[i].report = gptq_fold_report{};
    }
    char* ws = (char*)workspace;
    const hipStream_t caller = (hipStream_t)stream;

    if (check_mode_on()) {
        // Check mode: every call of the round is checked on its own (each is a checked entry),
        // in the plan's order, slot by slot on stand-in streams; nothing touches the GPU.
        for (int32_t i = 0; i < count; ++i) {
            const int k = i % conc;
            gptq_group& g = groups[order[i]];
            g.status = run_group(g, ws + (size_t)k * slot_bytes, layout[order[i]], dry_stream(16 + k),
                                 conc > 1);
        }
    } else {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return GPTQ_EHIP;
        std::vector<SlotStream> ss(conc);
        int got = 0;
        int err = GPTQ_OK;
        for (; got < conc; ++got)
            if ((err = slot_acquire(dev, &ss[got])) != GPTQ_OK) break;
        // Fork: every slot stream starts after the work already on the caller's stream.
        if (err == GPTQ_OK && hipEventRecord(ss[0].e, caller) != hipSuccess) err = GPTQ_EHIP;
        for (int k = 0; k < got && err == GPTQ_OK; ++k)
            if (hipStreamWaitEvent(ss[k].s, ss[0].e, 0) != hipSuccess) err = GPTQ_EHIP;
        if (err != GPTQ_OK) {
            for (int k = 0; k < got; ++k) slot_release(ss[k]);
            return err;
        }
        std::atomic<int32_t> next{0};
        std::atomic<bool> abort{false};
        auto worker = [&](int k) {
            if (hipSetDevice(dev) != hipSuccess) {
                abort.store(true);
                return;
            }
            char* slot = ws + (size_t)k * slot_bytes;
            for (;;) {
                if (abort.load()) break;
                const int32_t i = next.fetch_add(1);
                if (i >= count) break;
                gptq_group& g = groups[order[i]];
                g.status = run_group(g, slot, layout[order[i]], ss[k].s, conc > 1);
                if (g.status == GPTQ_EHIP) abort.store(true);
            }
        };
        // The calling thread is slot 0's worker; a slot whose thread cannot be started stays
        // idle and the others take its groups.
        std::vector<std::thread> th;
        for (int k = 1; k < conc; ++k) {
            try {
                th.emplace_back(worker, k);
            } catch (...) {
                break;
            }
        }
        worker(0);
        for (auto& t : th) t.join();
        // Join: the caller's stream waits for every slot stream.
        for (int k = 0; k < conc; ++k) {
            if (hipEventRecord(ss[k].e, ss[k].s) != hipSuccess ||
                hipStreamWaitEvent(caller, ss[k].e, 0) != hipSuccess)
                err = GPTQ_EHIP;
            slot_release(ss[k]);
        }
        if (err != GPTQ_OK) return err;
    }
    for (int32_t i = 0; i < count; ++i)
        if (groups[i].status != GPTQ_OK && groups[i].status != GPTQ_DEGENERATE) return groups[i].status;
    return GPTQ_OK;
}
