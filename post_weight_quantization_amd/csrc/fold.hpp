// fold.hpp -- state and workspace layout shared by the f32 fold (fold.hip) and the f64 fold
// (fold64.hip).
#pragma once
#include <stdint.h>

#include "common.hpp"

namespace gptq {

constexpr int NB = 128;     // f32: diagonal block and inner step
constexpr int NB64 = 64;    // f64: diagonal block and inner step
constexpr int W64 = 256;    // f64: outer panel (the K of its bulk updates)

// Device-side record of one fold call.
//   flag  bit 0: a pivot that is not positive (or not finite); the attempt failed.
//         bit 1: an f32 pivot at or below the f32 accuracy floor, or one that failed (precision
//                "auto" only): the attempt is abandoned and repeated in f64 at the same damping.
//   minp32 / minp64: the smallest accepted pivot of the attempt, as the bits of a positive f32
//         / f64 (their integer order is their value order).
struct FoldState {
    double base;
    unsigned flag;
    int n_dead;
    unsigned minp32;
    unsigned pad0;
    unsigned long long minp64;
    double pad[4];
};

struct FoldLayout {
    int64_t np, nbk, nb2;
    // f32 path
    size_t off_state, off_dinv, off_mi, off_t, off_xt, off_a, off_x, total_f32;
    // f64 path: A64 overlays the f32 A and X (8 n_p^2 bytes), the rest follows the f32 layout
    size_t off_x64, off_dinv64, off_mi64, off_tb64, off_xt64, total;
};

inline int64_t fold_outer_width(int64_t np) { return np >= 2048 ? 4 * NB : (np >= 512 ? 2 * NB : NB); }

inline FoldLayout fold_layout(int64_t n) {
    FoldLayout L{};
    L.np = round_up(n, NB);
    L.nbk = L.np / NB;
    L.nb2 = fold_outer_width(L.np);
    size_t o = 0;
    L.off_state = o; o += align256(sizeof(FoldState));
    L.off_dinv = o; o += align256(sizeof(float) * (size_t)L.np);
    L.off_mi = o; o += align256(sizeof(float) * (size_t)(L.nbk * NB * NB));
    L.off_t = o; o += align256(sizeof(float) * (size_t)(NB * L.nb2));
    L.off_xt = o; o += align256(sizeof(float) * (size_t)(L.nb2 * L.np));
    L.off_a = o; o += align256(sizeof(float) * (size_t)(L.np * L.np));
    L.off_x = o; o += align256(sizeof(float) * (size_t)(L.np * L.np));
    L.total_f32 = o;
    L.off_x64 = o; o += align256(sizeof(double) * (size_t)(L.np * L.np));
    L.off_dinv64 = o; o += align256(sizeof(double) * (size_t)L.np);
    L.off_mi64 = o; o += align256(sizeof(double) * (size_t)(L.np * NB64));
    L.off_tb64 = o; o += align256(sizeof(double) * (size_t)(NB64 * W64));
    L.off_xt64 = o; o += align256(sizeof(double) * (size_t)(W64 * L.np));
    L.total = o;
    return L;
}

// The f64 fold of one damping value (fold64.hip).  ws is the whole workspace (layout above);
// H has n = hl.n channels in either Hessian layout.  Enqueues on st: the f64 scales, the
// reversed equilibrated matrix, the blocked Cholesky with the blocked inverse trailing it
// panel by panel, on st and the helper streams of hp (single: st alone).  Pivots that are not
// positive and finite set flag bit 0 and make the remaining launches of the attempt return at
// once.  Ends with the helper streams joined into st.
int fold64_attempt(const float* H, HLayout hl, const float* hdiag, const uint8_t* dead,
                   FoldState* state, double lam, char* ws, const FoldLayout& L, hipStream_t st,
                   const Helper& hp, bool single);
// U = P X P D^-1 from the f64 inverse (rounded to f32 once).
int fold64_make_u(float* U, int64_t n, char* ws, const FoldLayout& L, hipStream_t st);

// gptq_fold_ex on a stream; single: no helper streams, every launch on st in program order
// (the same results bit for bit), for callers that run several folds side by side.
int fold_run(const float* H, int64_t n, int64_t ldh, double lambda, int precision, float* U,
             float* hdiag, uint8_t* dead, void* workspace, size_t workspace_bytes, hipStream_t st,
             gptq_fold_report* report, bool single);

// A gang of G groups of the same n (common.hpp: their data at the same offsets of slots gs
// bytes apart; U, hdiag, dead and ws are slot 0's, ws_bytes the workspace of one slot; ht the
// caller's Hessians).  Runs one f32 attempt at damping lambda for all of them in lockstep on
// st and its helper streams, and makes U.  A group whose attempt failed (failed[g] != 0, its
// flag bits) must be folded again on its own (fold_run), which repeats exactly what a call of
// its own would do; for the others, host[g] and reports[g] are what that call would return.
// precision: "auto" or "f32".
int fold_gang(const HTab& ht, int G, int64_t gs, int64_t n, double lambda, int precision,
              float* U, float* hdiag, uint8_t* dead, char* ws, size_t ws_bytes, hipStream_t st,
              FoldState* host, unsigned* failed, gptq_fold_report* reports);

}  // namespace gptq
