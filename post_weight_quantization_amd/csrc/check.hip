// check.hip -- the dry-run schedule checker declared in check.hpp (host code only).
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gptq_check.h"
#include "check.hpp"
#include "common.hpp"
#include "gemm_mfma.hpp"

namespace gptq {

namespace {

std::atomic<int> g_mode{0};
std::mutex g_msg_mu;
std::string g_msg;  // message of the last checked call (empty when it passed)

struct Launch {
    std::string name;
    int stream;
    uint64_t clock;              // this launch's position on its stream
    std::vector<uint64_t> vc;    // what it happens after: vc[t] launches of stream t
    std::vector<Span> acc;
};

struct Buffer {
    const char* lo;
    const char* hi;
    std::string name;
};

struct Sim {
    std::vector<hipStream_t> streams;
    std::vector<std::vector<uint64_t>> vc;   // per stream
    std::vector<std::pair<hipEvent_t, std::vector<uint64_t>>> events;
    std::vector<uint64_t> host;              // what the host has waited for
    std::vector<Launch> launches;
    std::vector<Buffer> bufs;
    std::string err;

    int sidx(hipStream_t s) {
        for (size_t i = 0; i < streams.size(); ++i)
            if (streams[i] == s) return (int)i;
        streams.push_back(s);
        vc.emplace_back();
        return (int)streams.size() - 1;
    }
    static void join(std::vector<uint64_t>& a, const std::vector<uint64_t>& b) {
        if (a.size() < b.size()) a.resize(b.size(), 0);
        for (size_t i = 0; i < b.size(); ++i) a[i] = std::max(a[i], b[i]);
    }
    std::vector<uint64_t>* event(hipEvent_t e, bool create) {
        for (auto& p : events)
            if (p.first == e) return &p.second;
        if (!create) return nullptr;
        events.emplace_back(e, std::vector<uint64_t>());
        return &events.back().second;
    }
};

thread_local Sim* t_sim = nullptr;
thread_local Gang t_gang{1, 0};

// Byte range [lo, hi) of a span; empty spans give lo == hi.
void span_range(const Span& s, const char*& lo, const char*& hi) {
    lo = hi = (const char*)s.p;
    if (s.rows <= 0 || s.cols <= 0) return;
    hi = lo + ((s.rows - 1) * s.ld + s.cols) * (int64_t)s.esize;
}

struct Rect {
    int64_t r0, r1, c0, c1;  // [r0, r1) x [c0, c1)
};

bool rect_meet(const Rect& a, const Rect& b) {
    return a.r0 < b.r1 && b.r0 < a.r1 && a.c0 < b.c1 && b.c0 < a.c1;
}

// Do two spans share a byte?  Exact for spans with the same row stride and element size whose
// starts differ by whole elements (each span is cut into at most two rectangles in the other's
// row/column frame); otherwise the byte ranges are compared (conservative).
bool spans_meet(const Span& a, const Span& b) {
    const char *alo, *ahi, *blo, *bhi;
    span_range(a, alo, ahi);
    span_range(b, blo, bhi);
    if (alo == ahi || blo == bhi) return false;
    if (!(alo < bhi && blo < ahi)) return false;
    const int64_t d = (const char*)b.p - (const char*)a.p;
    if (a.ld != b.ld || a.esize != b.esize || d % a.esize != 0 || a.cols > a.ld || b.cols > b.ld)
        return true;
    const int64_t ld = a.ld;
    const int64_t off = d / a.esize;
    int64_t rb = off / ld, cb = off % ld;
    if (cb < 0) {
        cb += ld;
        rb -= 1;
    }
    const Rect ra{0, a.rows, 0, a.cols};
    if (cb + b.cols <= ld) return rect_meet(ra, Rect{rb, rb + b.rows, cb, cb + b.cols});
    // b's rows wrap past the end of a row of the frame: two pieces.
    return rect_meet(ra, Rect{rb, rb + b.rows, cb, ld}) ||
           rect_meet(ra, Rect{rb + 1, rb + b.rows + 1, 0, cb + b.cols - ld});
}

void fail(Sim* s, const std::string& m) {
    if (s->err.empty()) s->err = m;
}

std::string span_str(const Span& s) {
    char b[200];
    snprintf(b, sizeof b, "%s %p ld %lld rows %lld cols %lld x%d B", s.write ? "write" : "read",
             s.p, (long long)s.ld, (long long)s.rows, (long long)s.cols, s.esize);
    return b;
}

}  // namespace

bool dry_run() { return t_sim != nullptr; }

Gang gang_current() { return t_gang; }
GangScope::GangScope(int G, int64_t gs) { t_gang = Gang{G, gs}; }
GangScope::~GangScope() { t_gang = Gang{1, 0}; }
bool check_mode_on() { return g_mode.load() != 0; }

CheckScope::CheckScope() {
    if (g_mode.load() && !t_sim) t_sim = new Sim();
}

CheckScope::~CheckScope() {
    if (t_sim) {
        delete t_sim;
        t_sim = nullptr;
    }
}

int CheckScope::finish() {
    Sim* s = t_sim;
    if (!s) return GPTQ_OK;
    // Races: pairs on different streams, unordered, with overlapping accesses and a write.
    const size_t N = s->launches.size();
    for (size_t i = 0; i < N && s->err.empty(); ++i) {
        const Launch& a = s->launches[i];
        for (size_t j = i + 1; j < N && s->err.empty(); ++j) {
            const Launch& b = s->launches[j];
            if (a.stream == b.stream) continue;
            const bool ab = (size_t)a.stream < b.vc.size() && b.vc[a.stream] >= a.clock;
            const bool ba = (size_t)b.stream < a.vc.size() && a.vc[b.stream] >= b.clock;
            if (ab || ba) continue;
            for (const Span& x : a.acc)
                for (const Span& y : b.acc)
                    if ((x.write || y.write) && spans_meet(x, y)) {
                        fail(s, "race: '" + a.name + "' (stream " + std::to_string(a.stream) +
                                    ") " + span_str(x) + " and '" + b.name + "' (stream " +
                                    std::to_string(b.stream) + ") " + span_str(y) +
                                    " are not ordered");
                        goto next;
                    }
        next:;
        }
    }
    std::lock_guard<std::mutex> lk(g_msg_mu);
    g_msg = s->err;
    return s->err.empty() ? GPTQ_OK : GPTQ_ECHECK;
}

void check_buffer(const void* p, size_t bytes, const char* name) {
    Sim* s = t_sim;
    if (!s || !p) return;
    s->bufs.push_back(Buffer{(const char*)p, (const char*)p + bytes, name});
}

int check_launch(const char* name, hipStream_t st, const Span* acc0, int nacc0) {
    Sim* s = t_sim;
    if (!s) return GPTQ_OK;
    const int k = s->sidx(st);
    Sim::join(s->vc[k], s->host);
    if (s->vc[k].size() <= (size_t)k) s->vc[k].resize(k + 1, 0);
    s->vc[k][k] += 1;
    // A gang's launch touches every group's slot: each span that is not fixed, once per group.
    std::vector<Span> all;
    for (int i = 0; i < nacc0; ++i) {
        const int reps = acc0[i].fixed ? 1 : t_gang.G;
        for (int g = 0; g < reps; ++g) {
            Span x = acc0[i];
            x.p = (const char*)x.p + (int64_t)g * t_gang.gs;
            all.push_back(x);
        }
    }
    const Span* acc = all.data();
    const int nacc = (int)all.size();
    Launch L{name, k, s->vc[k][k], s->vc[k], all};
    for (int i = 0; i < nacc; ++i) {
        const char *lo, *hi;
        span_range(acc[i], lo, hi);
        if (lo == hi) continue;
        bool inside = false;
        for (const Buffer& b : s->bufs)
            if (lo >= b.lo && hi <= b.hi) {
                inside = true;
                break;
            }
        if (!inside) {
            fail(s, std::string("bounds: '") + name + "' " + span_str(acc[i]) +
                        " lies outside every buffer of the call");
            std::lock_guard<std::mutex> lk(g_msg_mu);
            g_msg = s->err;
            return GPTQ_ECHECK;
        }
    }
    s->launches.push_back(std::move(L));
    return GPTQ_OK;
}

int ev_record(hipEvent_t e, hipStream_t st) {
    Sim* s = t_sim;
    if (!s) return hipEventRecord(e, st) == hipSuccess ? GPTQ_OK : GPTQ_EHIP;
    const int k = s->sidx(st);
    Sim::join(s->vc[k], s->host);
    *s->event(e, true) = s->vc[k];
    return GPTQ_OK;
}

int stream_wait(hipStream_t st, hipEvent_t e) {
    Sim* s = t_sim;
    if (!s) return hipStreamWaitEvent(st, e, 0) == hipSuccess ? GPTQ_OK : GPTQ_EHIP;
    const int k = s->sidx(st);
    const std::vector<uint64_t>* v = s->event(e, false);
    if (v) Sim::join(s->vc[k], *v);
    return GPTQ_OK;
}

int launch_status() {
    if (t_sim) return GPTQ_OK;
    return hipGetLastError() == hipSuccess ? GPTQ_OK : GPTQ_EHIP;
}

void host_sync_record(hipStream_t st) {
    Sim* s = t_sim;
    if (!s) return;
    const int k = s->sidx(st);
    Sim::join(s->host, s->vc[k]);
}

hipStream_t dry_stream(int k) { return (hipStream_t)(uintptr_t)(0x5000 + 16 * k); }
hipEvent_t dry_event(int k) { return (hipEvent_t)(uintptr_t)(0x9000 + 16 * k); }

}  // namespace gptq

using namespace gptq;

extern "C" void gptq_check_mode(int on) { g_mode.store(on ? 1 : 0); }

extern "C" const char* gptq_check_message(void) {
    static thread_local std::string copy;
    std::lock_guard<std::mutex> lk(g_msg_mu);
    copy = g_msg;
    return copy.c_str();
}

// The checker on a hand-made schedule: case 0 is clean, case 1 has two unordered writers of
// one row block, case 2 orders them by an event, case 3 reads past the end of its buffer.
extern "C" int gptq_check_selftest(int which) {
    const int saved = g_mode.exchange(1);
    int rc = GPTQ_OK;
    {
        CheckScope cs;
        static float buf[64 * 64];
        check_buffer(buf, sizeof buf, "buf");
        const hipStream_t s0 = dry_stream(0), s1 = dry_stream(1);
        const hipEvent_t e = dry_event(0);
        auto body = [&]() -> int {
            // Two column halves of the same rows: disjoint, may run unordered.
            const Span a[] = {wr(buf, 64, 64, 32)};
            const Span b[] = {wr(buf + 32, 64, 64, 32)};
            int r = check_launch("left", s0, a, 1);
            if (r) return r;
            if (which == 2) {
                ev_record(e, s0);
                stream_wait(s1, e);
            }
            if (which == 1 || which == 2) {
                const Span c[] = {wr(buf + 16, 64, 8, 32)};  // overlaps both halves
                r = check_launch("overlap", s1, c, 1);
                if (r) return r;
            } else {
                r = check_launch("right", s1, b, 1);
                if (r) return r;
            }
            if (which == 3) {
                const Span d[] = {rd(buf + 40 * 64, 64, 25, 64)};  // one row too many
                r = check_launch("past the end", s0, d, 1);
                if (r) return r;
            }
            return GPTQ_OK;
        };
        rc = body();
        if (rc == GPTQ_OK) rc = cs.finish();
    }
    g_mode.store(saved);
    return rc;
}

// The GEMM's workgroup -> tile map (XCD renumbering, then the super-tile order) on the host:
// every workgroup of a launch must get a distinct tile of the problem's tile set.
extern "C" int gptq_check_tile_order(int64_t M, int64_t N, int lower) {
    if (M <= 0 || N <= 0 || M > ((int64_t)1 << 20) || N > ((int64_t)1 << 20)) return GPTQ_EINVAL;
    const GemmProblem P = lower ? gemm_syrk_lower(nullptr, 32, nullptr, nullptr, M, (int)M, 32, 1.0f, 0)
                                : gemm_full(nullptr, 32, nullptr, 32, nullptr, nullptr, N, (int)M,
                                            (int)N, 32, 1.0f, 0);
    const int TN = P.tiles_n, TM = lower ? P.tiles_n : P.ntiles / P.tiles_n;
    // Every group of a gang (grid z) must cover the grid once as well.
    for (int z = 0; z < kMaxGang; ++z) {
        std::vector<unsigned char> seen((size_t)TM * TN, 0);
        for (int b = 0; b < P.ntiles; ++b) {
            const int g = gang_block(b, z, P.ntiles);
            if (g < 0 || g >= P.ntiles) return GPTQ_ECHECK;
            int tm = -1, tn = -1;
            tile_of(P, xcd_order(g, P.ntiles), tm, tn);
            if (tm < 0 || tm >= TM || tn < 0 || tn >= TN || (lower && tn > tm)) return GPTQ_ECHECK;
            unsigned char& f = seen[(size_t)tm * TN + tn];
            if (f) return GPTQ_ECHECK;
            f = 1;
        }
    }
    return GPTQ_OK;
}
