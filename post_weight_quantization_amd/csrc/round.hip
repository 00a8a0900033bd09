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
// Execution, when groups of the same shape follow each other in the order: gangs (below),
// run one after another on the caller's stream.  A gang's groups advance in lockstep, each
// launch covering all of them, so they share every step of the serial chains instead of
// queueing for the GPU's few hardware queues: 11 groups of n = 4096 take 16.9 ms as one gang,
// 21.4 ms as gangs of 4, and 25.4 ms on four threads.
//
// Otherwise: one host thread and one stream per slot.  A thread takes the next group of the
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

// Without a cap from the caller: gangs of up to kMaxGang groups; rounds that form no gang run
// kDefaultThreads groups at a time, one per hardware queue of the process.
constexpr int kDefaultThreads = 4;

struct SlotLayout {
    size_t off_hd, off_dead, off_work, total;
};

// A member's area inside a slot's work area, after the fold (the gang form): the working copy
// and residual panels of an in-place sweep, then its outputs, staged for the copy to the
// caller's buffers.
struct MemberArea {
    size_t off_wc, off_p0, off_p1, off_lost, off_tab, off_nib, off_rung, off_scale, total;
};

MemberArea member_area(int64_t rows, int64_t n) {
    MemberArea a{};
    size_t o = 0;
    a.off_wc = o; o += align256(sizeof(float) * (size_t)(rows * n));
    a.off_p0 = o; o += sweep_panel_bytes(rows);
    a.off_p1 = o; o += sweep_panel_bytes(rows);
    a.off_lost = o; o += align256(sizeof(float) * (size_t)(rows * 2));
    a.off_tab = o; o += align256(sizeof(float) * (size_t)(rows * 32));
    a.off_nib = o; o += align256((size_t)(rows * (n / 2)));
    a.off_rung = o; o += align256((size_t)(rows * (n / 32)));
    a.off_scale = o; o += align256(sizeof(float) * (size_t)(rows * (n / 32)));
    a.total = o;
    return a;
}

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
        work = std::max(work, member_area(g.member[k].rows, n).total);
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

// ---------------------------------------------------------------------------------------------
// Gangs.  Groups of the same shape (n, precision, damping, and member by member the rows and
// codec) run in lockstep, as many as there are slots: every launch covers all of them, one
// slot each (common.hpp).  A lone group's serial chains (the fold's diagonal blocks, the
// sweep's column blocks) leave most of the GPU idle at small n; G groups share each step's
// latency and give its products G times the work.  The caller's matrices are copied into the
// slots first, and the outputs out of them at the end.

struct CopyTab {
    const void* src[kMaxGang];
    void* dst[kMaxGang];
};

// bytes from src[z] to dst[z] for group z (null: nothing); 16-byte moves when both are aligned.
__global__ __launch_bounds__(256) void gang_copy_kernel(CopyTab t, int64_t bytes) {
    const char* src = (const char*)t.src[blockIdx.z];
    char* dst = (char*)t.dst[blockIdx.z];
    if (!src || !dst) return;
    const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t step = (int64_t)gridDim.x * 256;
    int64_t done = 0;
    if ((((uintptr_t)src | (uintptr_t)dst) & 15u) == 0) {
        const int64_t n16 = bytes / 16;
        for (int64_t i = i0; i < n16; i += step)
            reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
        done = n16 * 16;
    }
    for (int64_t i = done + i0; i < bytes; i += step) dst[i] = src[i];
}

// Copies bytes for each of the G pairs (a null pointer skips the group), checked as one call.
int gang_copy(const char* name, const CopyTab& t, int G, int64_t bytes, hipStream_t st) {
    if (bytes <= 0) return GPTQ_OK;
    CheckScope check;
    std::vector<Span> acc;
    for (int g = 0; g < G; ++g) {
        if (!t.src[g] || !t.dst[g]) continue;
        check_buffer(t.src[g], (size_t)bytes, "copy source");
        check_buffer(t.dst[g], (size_t)bytes, "copy destination");
        acc.push_back(fixed(rd(t.src[g], bytes, 1, bytes, 1)));
        acc.push_back(fixed(wr(t.dst[g], bytes, 1, bytes, 1)));
    }
    int rc = check_launch(name, st, acc.data(), (int)acc.size());
    if (rc != GPTQ_OK) return rc;
    const unsigned gx = (unsigned)std::min<int64_t>(1024, std::max<int64_t>(1, (bytes / 16 + 255) / 256));
    if (!dry_run()) gang_copy_kernel<<<dim3(gx, 1, (unsigned)G), 256, 0, st>>>(t, bytes);
    if (launch_status() != GPTQ_OK) return GPTQ_EHIP;
    return check.finish();
}

bool same_shape(const gptq_group& a, const gptq_group& b) {
    if (a.n != b.n || a.precision != b.precision || a.lambda != b.lambda || a.members != b.members)
        return false;
    if (a.precision == GPTQ_FOLD_F64) return false;  // the gang's attempt is an f32 one
    for (int32_t k = 0; k < a.members; ++k)
        if (a.member[k].rows != b.member[k].rows || a.member[k].codec != b.member[k].codec) return false;
    return true;
}

// Gangs of the plan's order: runs of consecutive groups of the same shape, at most cap long.
std::vector<std::pair<int32_t, int32_t>> gangs_of(const gptq_group* groups, const int32_t* order,
                                                  int32_t count, int cap) {
    std::vector<std::pair<int32_t, int32_t>> out;  // (first position in the order, length)
    for (int32_t i = 0; i < count;) {
        int32_t j = i + 1;
        if (groups[order[i]].precision != GPTQ_FOLD_F64)
            while (j < count && j - i < cap && same_shape(groups[order[i]], groups[order[j]])) ++j;
        out.emplace_back(i, j - i);
        i = j;
    }
    return out;
}

// One gang of G groups (order[0 .. G-1]) in slots 0 .. G-1, on st.
int run_gang(gptq_group* groups, const int32_t* idx, int G, char* ws, size_t slot_bytes,
             const SlotLayout& L, hipStream_t st) {
    const gptq_group& g0 = groups[idx[0]];
    const int64_t n = g0.n;
    const int64_t gs = (int64_t)slot_bytes;
    HTab ht{};
    for (int k = 0; k < G; ++k) {
        ht.H[k] = groups[idx[k]].H;
        ht.ldh[k] = groups[idx[k]].ldh;
    }
    float* U0 = (float*)ws;
    float* hd0 = (float*)(ws + L.off_hd);
    uint8_t* dd0 = (uint8_t*)(ws + L.off_dead);
    char* work0 = ws + L.off_work;
    const size_t work_bytes = L.total - L.off_work;
    FoldState host[kMaxGang];
    unsigned failed[kMaxGang];
    gptq_fold_report rep[kMaxGang];
    int rc = fold_gang(ht, G, gs, n, g0.lambda, g0.precision, U0, hd0, dd0, work0, work_bytes, st,
                       host, failed, rep);
    if (rc != GPTQ_OK) return rc;
    // A group whose attempt failed is folded again on its own, from the start: the same
    // schedule of dampings and precisions as a call of its own.
    for (int k = 0; k < G; ++k) {
        gptq_group& g = groups[idx[k]];
        int fs = GPTQ_OK;
        if (failed[k]) {
            char* slot = ws + (size_t)k * slot_bytes;
            fs = fold_run(g.H, n, g.ldh, g.lambda, g.precision, (float*)slot,
                          (float*)(slot + L.off_hd), (uint8_t*)(slot + L.off_dead),
                          slot + L.off_work, work_bytes, st, &rep[k], false);
            if (fs != GPTQ_OK && fs != GPTQ_DEGENERATE) return fs;
        }
        g.report = rep[k];
        g.status = fs;
    }
    CopyTab th{}, td{};
    for (int k = 0; k < G; ++k) {
        const gptq_group& g = groups[idx[k]];
        char* slot = ws + (size_t)k * slot_bytes;
        th.src[k] = slot + L.off_hd;
        th.dst[k] = g.hdiag;
        td.src[k] = slot + L.off_dead;
        td.dst[k] = g.dead;
    }
    if ((rc = gang_copy("gang_hdiag_out", th, G, sizeof(float) * n, st)) != GPTQ_OK) return rc;
    if ((rc = gang_copy("gang_dead_out", td, G, n, st)) != GPTQ_OK) return rc;
    for (int32_t m = 0; m < g0.members; ++m) {
        const int64_t rows = g0.member[m].rows;
        const bool q2 = g0.member[m].codec == GPTQ_CODEC_Q2TP;
        const MemberArea a = member_area(rows, n);
        char* w0 = work0;
        CopyTab tin{};
        for (int k = 0; k < G; ++k) {
            tin.src[k] = groups[idx[k]].member[m].W;
            tin.dst[k] = w0 + (size_t)k * slot_bytes + a.off_wc;
        }
        if ((rc = gang_copy("gang_w_in", tin, G, (int64_t)sizeof(float) * rows * n, st)) != GPTQ_OK)
            return rc;
        rc = sweep_gang(G, gs, q2, (float*)(w0 + a.off_wc), U0, hd0, dd0, (float*)(w0 + a.off_lost),
                        (float*)(w0 + a.off_tab), rows, n, (uint8_t*)(w0 + a.off_nib),
                        (uint8_t*)(w0 + a.off_rung), (float*)(w0 + a.off_scale),
                        (float*)(w0 + a.off_p0), (float*)(w0 + a.off_p1), st);
        if (rc != GPTQ_OK) return rc;
        struct Out {
            size_t off;
            int64_t bytes;
            const char* name;
        };
        const Out outs[5] = {
            {a.off_lost, (int64_t)sizeof(float) * rows * 2, "gang_lost_out"},
            {a.off_tab, (int64_t)sizeof(float) * rows * 32, "gang_tab_out"},
            {a.off_nib, rows * (n / (q2 ? 4 : 2)), "gang_codes_out"},
            {a.off_rung, rows * (n / 32), "gang_rung_out"},
            {a.off_scale, (int64_t)sizeof(float) * rows * (n / 32), "gang_scale_out"},
        };
        for (int q = 0; q < 5; ++q) {
            CopyTab t{};
            for (int k = 0; k < G; ++k) {
                const gptq_member& mm = groups[idx[k]].member[m];
                void* dst = q == 0 ? (void*)mm.lost : q == 1 ? (void*)mm.tab : q == 2 ? (void*)mm.codes
                          : q == 3 ? (void*)mm.rung : (void*)mm.scale;
                t.src[k] = w0 + (size_t)k * slot_bytes + outs[q].off;
                t.dst[k] = dst;
            }
            if ((rc = gang_copy(outs[q].name, t, G, outs[q].bytes, st)) != GPTQ_OK) return rc;
        }
    }
    return GPTQ_OK;
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

namespace gptq {
namespace {

// The order, the gangs (empty when the round forms none: then it runs on threads) and the
// slots in use.
int plan_round(const gptq_group* groups, int32_t count, size_t workspace_bytes,
               int32_t max_concurrency, int32_t* order, int32_t* concurrency,
               std::vector<std::pair<int32_t, int32_t>>* gangs_out) {
    if (!groups || count <= 0 || !order || !concurrency) return GPTQ_EINVAL;
    const size_t slot = gptq_round_slot_size(groups, count);
    if (slot == 0) return GPTQ_EINVAL;
    if (workspace_bytes < slot) return GPTQ_EWORKSPACE;
    const int64_t fit = (int64_t)(workspace_bytes / slot);
    plan_order(groups, count, order);
    const int64_t gcap = std::min<int64_t>(max_concurrency > 0 ? max_concurrency : kMaxGang, kMaxGang);
    auto gangs = gangs_of(groups, order, count, (int)std::max<int64_t>(1, std::min(gcap, fit)));
    int32_t widest = 1;
    for (const auto& gg : gangs) widest = std::max(widest, gg.second);
    if (widest > 1) {
        *concurrency = widest;
    } else {
        gangs.clear();
        const int64_t cap = max_concurrency > 0 ? max_concurrency : kDefaultThreads;
        *concurrency = (int32_t)std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(cap, count), fit));
    }
    if (gangs_out) *gangs_out = std::move(gangs);
    return GPTQ_OK;
}

}  // namespace
}  // namespace gptq

extern "C" int gptq_round_plan(const gptq_group* groups, int32_t count, size_t workspace_bytes,
                               int32_t max_concurrency, int32_t* order, int32_t* concurrency) {
    return plan_round(groups, count, workspace_bytes, max_concurrency, order, concurrency, nullptr);
}

extern "C" int gptq_round(gptq_group* groups, int32_t count, void* workspace,
                          size_t workspace_bytes, int32_t max_concurrency, void* stream) {
    if (!workspace || ((uintptr_t)workspace & 255u) != 0) return GPTQ_EINVAL;
    std::vector<int32_t> order(count > 0 ? count : 1);
    int32_t conc = 0;
    std::vector<std::pair<int32_t, int32_t>> gangs;
    const int rc = plan_round(groups, count, workspace_bytes, max_concurrency, order.data(), &conc,
                              &gangs);
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

    if (!gangs.empty()) {
        // The gangs one after another on the caller's stream, from slot 0 (a lone group on its
        // own, with its helper streams).
        const hipStream_t st = check_mode_on() ? dry_stream(16) : caller;
        for (const auto& gg : gangs) {
            const int32_t* idx = order.data() + gg.first;
            int rc;
            if (gg.second == 1) {
                gptq_group& g = groups[idx[0]];
                rc = g.status = run_group(g, ws, layout[idx[0]], st, false);
                if (rc == GPTQ_DEGENERATE) rc = GPTQ_OK;
            } else {
                rc = run_gang(groups, idx, gg.second, ws, slot_bytes, layout[idx[0]], st);
                if (rc != GPTQ_OK)
                    for (int32_t k = 0; k < gg.second; ++k) groups[idx[k]].status = rc;
            }
            if (rc != GPTQ_OK) return rc;
        }
    } else if (check_mode_on()) {
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
