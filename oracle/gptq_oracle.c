/*
 * gptq_oracle.c -- the plain, slow CPU oracle of the GPTQ fold and the q4tp sweep.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls this file:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It shares no
 * code, header, table or constant with the HIP library.
 *
 * Sources it follows (docs.rs source pages of the cortiq project):
 *   [gptq.rs]      "cortiq-cli 0.8.45 src/gptq.rs": gptq_fold_operator_par (what the fold
 *                  computes: dead channels, damping, the retry schedule, U = the upper Cholesky
 *                  factor of H_d^-1; computed here from that definition, not by the page's
 *                  route), gptq_quantize_q4tp (rung rule, per-column rounding, full-row error
 *                  feedback).
 *   [gptq_dev.rs]  "cortiq-engine 0.8.41 src/gpu_wgpu/gptq_dev.rs": module documentation
 *                  (steps 1-5 of the method) and the q4tp_group kernel (the same rung rule).
 *
 * Arithmetic: f64 for every value (H, L, L^-1, H^-1, U, the corrected weights, the residuals).
 * Where floating point decides an integer (a rounded code, the chosen rung) the decision is
 * taken on the f32 value of the corrected weight in f32 arithmetic, the precision of the
 * pages' own sweep; the nominal rung is evaluated in f64 on that f32 absmax.
 *
 * Parallelism: OpenMP over independent rows (or independent column blocks).  Every entry is
 * produced by exactly one thread with a fixed summation order, so results do not depend on
 * the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORC_OK 0
#define ORC_FAILED 1
#define ORC_DEGENERATE 4

/* Columns per cache block.  Only the loop order depends on it, never an entry's arithmetic. */
#define BLK 32

static int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }

/* Dot product of two contiguous f64 vectors in a fixed order: four interleaved partial sums,
 * combined pairwise, then the tail.  The order is the same for every call site and thread. */
static double dot(const double* a, const double* b, int64_t len) {
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    int64_t k = 0;
    for (; k + 4 <= len; k += 4) {
        s0 += a[k] * b[k];
        s1 += a[k + 1] * b[k + 1];
        s2 += a[k + 2] * b[k + 2];
        s3 += a[k + 3] * b[k + 3];
    }
    double s = (s0 + s1) + (s2 + s3);
    for (; k < len; ++k) s += a[k] * b[k];
    return s;
}

/* In-place lower Cholesky factor A = C C^T of a dense row-major n x n f64 matrix (lower
 * triangle read, upper triangle zeroed on success), by the textbook entry formula
 *     c_jj = sqrt(a_jj - sum_{k<j} c_jk^2),     c_ij = (a_ij - sum_{k<j} c_ik c_jk) / c_jj  (i > j)
 * (Golub and Van Loan, "Matrix Computations", the Cholesky algorithm), failing when a pivot is
 * not positive or not finite: the pivot rule of the host fold ([gptq.rs]).  Columns are visited
 * in blocks of BLK so that the rows of a block stay in cache; the rows below a block are
 * independent given the block and run in parallel. */
static int chol_lower(double* a, int64_t n, int nt) {
    for (int64_t jb = 0; jb < n; jb += BLK) {
        int64_t je = imin(jb + BLK, n);
        for (int64_t i = jb; i < je; ++i) {
            for (int64_t j = jb; j <= i; ++j) {
                double s = a[i * n + j] - dot(a + i * n, a + j * n, j);
                if (i == j) {
                    if (!(s > 0.0) || !isfinite(s)) return 0;
                    a[i * n + i] = sqrt(s);
                } else {
                    a[i * n + j] = s / a[j * n + j];
                }
            }
        }
#pragma omp parallel for num_threads(nt) schedule(static)
        for (int64_t i = je; i < n; ++i)
            for (int64_t j = jb; j < je; ++j)
                a[i * n + j] = (a[i * n + j] - dot(a + i * n, a + j * n, j)) / a[j * n + j];
    }
    for (int64_t i = 0; i < n; ++i)
        for (int64_t k = i + 1; k < n; ++k) a[i * n + k] = 0.0;
    return 1;
}

/* The inverse of a lower triangular C by triangular solves: column j of C^-1 is the solution y
 * of C y = e_j, by forward substitution
 *     y_i = 0 (i < j),   y_j = 1 / c_jj,   y_i = -(sum_{k=j}^{i-1} c_ik y_k) / c_ii  (i > j).
 * Column j is stored as row j of yt (yt[j][i] = (C^-1)_ij), so each sum is a contiguous dot
 * product.  The columns are independent; a block of BLK of them walks the rows of C once. */
static void lower_inverse_cols(const double* c, double* yt, int64_t n, int nt) {
    int64_t nblk = (n + BLK - 1) / BLK;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b) {
        int64_t c0 = b * BLK, c1 = imin(c0 + BLK, n);
        for (int64_t j = c0; j < c1; ++j) memset(yt + j * n, 0, sizeof(double) * (size_t)n);
        for (int64_t i = c0; i < n; ++i) {
            const double* ci = c + i * n;
            for (int64_t j = c0; j < c1 && j <= i; ++j) {
                double* y = yt + j * n;
                y[i] = (i == j) ? 1.0 / ci[i] : -dot(ci + j, y + j, i - j) / ci[i];
            }
        }
    }
}

static void set_identity(double* u, int64_t n) {
    memset(u, 0, sizeof(double) * (size_t)(n * n));
    for (int64_t i = 0; i < n; ++i) u[i * n + i] = 1.0;
}

/*
 * The fold: U, the upper triangular factor with a positive diagonal of H_d^-1 = U^T U
 * ([gptq.rs] gptq_fold_operator_par; [gptq_dev.rs] module documentation, steps 1-4).
 *
 * Decision rules fixed by the method:
 *   1. h = H in f64, symmetric, read from the UPPER triangle of H (ldh = row stride).
 *   2. hdiag_i = H_ii (raw f32); dead_i = !(H_ii > 0) (so NaN is dead).
 *   3. a dead channel's row and column are zeroed and its diagonal set to 1.
 *   4. base = max(mean_i h_ii, 1e-12);  damp = lam * base;  H_d = h + damp I.
 *   5. lam = max(lambda, 0); a factorization that meets a pivot that is not positive or not
 *      finite is redone at lam -> 1e-4 (from 0) or 10 lam; past 10 the result is U = I with
 *      status DEGENERATE.  With retry == 0 the first failure returns FAILED.
 *
 * How U is computed (from the definition; the factor is unique):  with J the order reversal,
 * let J H_d J = C C^T (lower Cholesky).  Then H_d = (J C J)(J C J)^T, where R = J C J is upper
 * triangular with a positive diagonal, so H_d^-1 = R^-T R^-1 and U = R^-1 = J C^-1 J:
 *     U[j][k] = (C^-1)[n-1-j][n-1-k]  for k >= j, 0 below.
 *   route 0: exactly that.
 *   route 1: the same on the equilibrated matrix, J D^-1 H_d D^-1 J = C~ C~^T with
 *            D = sqrt(diag H_d), then U = J C~^-1 J D^-1 (the device's arrangement in f64;
 *            different rounding, the same U).  Used to cross-check route 0.
 * info[0] = lam used, info[1] = base, info[2] = damp, info[3] = attempts.
 * Returns ORC_OK, ORC_FAILED (retry == 0 and the factor failed) or ORC_DEGENERATE.
 */
int orc_fold(const float* H, int64_t n, int64_t ldh, double lambda, int retry, int route,
             double* U, float* hdiag, uint8_t* dead, double* info, int nt) {
    if (n <= 0 || route < 0 || route > 1) return ORC_FAILED;
    size_t nn = (size_t)(n * n);
    double* h = (double*)malloc(sizeof(double) * nn);
    double* a = (double*)malloc(sizeof(double) * nn);
    double* dsc = (double*)malloc(sizeof(double) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) {
        float d = H[i * ldh + i];
        hdiag[i] = d;
        dead[i] = !(d > 0.0f);
    }
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < n; ++j) {
            int64_t r = i < j ? i : j, c = i < j ? j : i;
            h[i * n + j] = (double)H[r * ldh + c];
        }
    for (int64_t i = 0; i < n; ++i) {
        if (!dead[i]) continue;
        for (int64_t k = 0; k < n; ++k) h[i * n + k] = h[k * n + i] = 0.0;
        h[i * n + i] = 1.0;
    }
    double mean = 0.0;
    for (int64_t i = 0; i < n; ++i) mean += h[i * n + i];
    mean /= (double)n;
    double base = mean > 1e-12 ? mean : 1e-12;
    double lam = lambda > 0.0 ? lambda : 0.0;
    int attempts = 0;
    int status = ORC_OK;
    int ok;
    for (;;) {
        double damp = lam * base;
        for (int64_t i = 0; i < n; ++i) dsc[i] = (route == 1) ? sqrt(h[i * n + i] + damp) : 1.0;
        /* a = J (D^-1) H_d (D^-1) J, lower triangle (the factorization reads no more) */
        for (int64_t i = 0; i < n; ++i)
            for (int64_t j = 0; j <= i; ++j) {
                int64_t ii = n - 1 - i, jj = n - 1 - j;
                double v = h[ii * n + jj] + (ii == jj ? damp : 0.0);
                a[i * n + j] = v / (dsc[ii] * dsc[jj]);
            }
        ++attempts;
        ok = chol_lower(a, n, nt);
        if (ok > 0) break;
        if (!retry) { ok = 0; break; }
        lam = (lam == 0.0) ? 1e-4 : lam * 10.0;
        if (lam > 10.0) { ok = -1; break; }
    }
    if (ok <= 0) {
        status = ok == 0 ? ORC_FAILED : ORC_DEGENERATE;
        set_identity(U, n);
    } else {
        double* yt = h; /* h is no longer needed: yt[j][i] = (C^-1)_ij */
        lower_inverse_cols(a, yt, n, nt);
#pragma omp parallel for num_threads(nt) schedule(static)
        for (int64_t j = 0; j < n; ++j)
            for (int64_t k = 0; k < n; ++k)
                U[j * n + k] = (k >= j) ? yt[(n - 1 - k) * n + (n - 1 - j)] / dsc[k] : 0.0;
    }
    info[0] = lam;
    info[1] = base;
    info[2] = lam * base;
    info[3] = (double)attempts;
    free(dsc);
    free(h);
    free(a);
    return status;
}

/* ------------------------------------------------------------------------------------------ */
/* Binary16 rounding (IEEE 754, round to nearest, ties to even), from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; normals down to 2^-14, subnormal
 * quantum 2^-24, largest finite 65504.  Scaling by powers of two is exact in f64, so the
 * rounding below is a single correctly rounded step. */
double orc_f16_round(double x) {
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    double a = fabs(x);
    if (a >= 65520.0) return copysign(INFINITY, x); /* half-way to 2^16 and beyond */
    int e2;
    frexp(a, &e2);         /* a = m 2^e2, m in [0.5, 1) */
    int e = e2 - 1;        /* a in [2^e, 2^(e+1)) */
    int qexp = (e < -14) ? -24 : e - 10;
    double q = ldexp(a, -qexp);
    double r = nearbyint(q); /* default rounding mode: to nearest, ties to even */
    return copysign(ldexp(r, qexp), x);
}

/*
 * The per-row rung ladder (lo, step) and TAB[c] = 2^(lo + c step), c = 0..31, from the
 * dead-zeroed original weights.  The pages take it from their converter, whose rule is not on
 * the pages; the reading used here: with a_g = max_t |W[r, gs g + t]| over the groups g of the
 * row and only a_g > 0 counted,
 *     lo   = f16(log2(min a_g / 7)),
 *     hi   = log2(max a_g / 7),
 *     step = f16((hi - lo) / 31) if hi > lo, else 0,
 *     TAB[c] = f32(2^(lo + c step)) evaluated in f64;
 * a row with no nonzero group gets lo = 0, step = 0, TAB = 1.  ([gptq.rs] gptq_quantize_q4tp
 * and gptq_quantize_q4tp_dev: the ladder is fixed per row from the original weights and its lo
 * and step are stored as f16.)
 */
void orc_ladder(const float* W0, const uint8_t* dead, int64_t rows, int64_t n, int64_t gs,
                float* lost, float* tab) {
    for (int64_t r = 0; r < rows; ++r) {
        double amin = INFINITY, amax = 0.0;
        for (int64_t g = 0; g < n / gs; ++g) {
            float a = 0.0f;
            for (int64_t t = 0; t < gs; ++t) {
                int64_t j = g * gs + t;
                float v = dead[j] ? 0.0f : fabsf(W0[r * n + j]);
                if (v > a) a = v;
            }
            if (a > 0.0f) {
                if (a < amin) amin = a;
                if (a > amax) amax = a;
            }
        }
        double lo = 0.0, st = 0.0;
        if (amax > 0.0) {
            lo = orc_f16_round(log2(amin / 7.0));
            double hi = log2(amax / 7.0);
            st = (hi > lo) ? orc_f16_round((hi - lo) / 31.0) : 0.0;
            if (!(st > 0.0)) st = 0.0;
        }
        lost[r * 2] = (float)lo;
        lost[r * 2 + 1] = (float)st;
        for (int c = 0; c < 32; ++c)
            tab[r * 32 + c] = (amax > 0.0) ? (float)exp2(lo + (double)c * st) : 1.0f;
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Decisions in f32 (the pages' sweep precision).  Every step is a separately rounded f32
 * operation; the file is compiled without contraction of multiply-add. */
static float rne_f32(float x) { return nearbyintf(x); } /* ties to even */
static float clampf(float x, float lo, float hi) { return x < lo ? lo : (x > hi ? hi : x); }
static double round_half_away(double x) { return (x < 0.0) ? -floor(-x + 0.5) : floor(x + 0.5); }

/* Nominal rung of a tile from its f32 absmax ([gptq_dev.rs] q4tp_group; [gptq.rs]
 * gptq_quantize_q4tp): clamp(round_half_away((log2(amax/7) - lo) / step), 0, 31), or 0 when
 * amax = 0 or step <= 0.  Evaluated in f64.  *v_out receives the unrounded value. */
static int nominal_rung(float amax, float lo, float st, double* v_out) {
    *v_out = 0.0;
    if (amax == 0.0f || st <= 0.0f) return 0;
    double v = (log2((double)amax / 7.0) - (double)lo) / (double)st;
    *v_out = v;
    double r = round_half_away(v);
    if (r < 0.0) r = 0.0;
    if (r > 31.0) r = 31.0;
    return (int)r;
}

/* H_ii-weighted rounding error of a tile at scale s, accumulated in f32 in column order:
 * sum_t h_t (w_t - clamp(rne(w_t / s), -8, 7) s)^2. */
static float tile_error(const float* wf, const float* hd, int64_t gs, float s) {
    float err = 0.0f;
    for (int64_t t = 0; t < gs; ++t) {
        float q = clampf(rne_f32(wf[t] / s), -8.0f, 7.0f);
        float d = wf[t] - q * s;
        float hd_d = hd[t] * d;
        err = err + hd_d * d;
    }
    return err;
}

/*
 * The q4tp sweep of rows x n weights in groups of gs columns ([gptq.rs] gptq_quantize_q4tp;
 * [gptq_dev.rs] module documentation, step 5, and q4tp_group):
 *   w = W0 with dead columns zeroed (f64 state).
 *   For each group g (c0 = gs g), each row:
 *     wf = f32(w[c0 .. c0+gs)), amax = max |wf|, nominal rung as above;
 *     if amax > 0: candidates max(nominal-2, 0) .. min(nominal+1, 31) ascending, skipping
 *       TAB <= 0; keep a candidate only when its error is strictly below the best so far;
 *       with no valid candidate keep nominal;
 *     s = TAB[rung];  for j = c0 .. c0+gs-1 in order:
 *       q = (s > 0) ? clamp(rne(f32(w_j) / s), -8, 7) : 0,   code = q + 8,
 *       e_j = (U_jj > 0) ? (w_j - q s) / U_jj : 0,
 *       w_t -= e_j U_jt for every t > j (column-by-column full-row feedback).
 * Outputs: code[rows*n] (q + 8, one per byte), rung[rows*(n/gs)], scale = TAB[rung],
 * E[rows*n] = e (optional), Wc[rows*n] = the corrected weight each column was rounded from
 * (optional).
 *
 * Tie-forced replay (force_code / force_rung non-NULL): wherever the oracle's decision differs
 * from the forced one, it is a TIE when
 *   code:  |frac(|f32(w_j)/s|) - 0.5| < tie_band and the codes differ by one, or
 *   rung:  the two candidates' f32 errors differ by at most rung_band relative to the smaller,
 *          or the unrounded nominal value lies within tie_band of a half-integer;
 * otherwise it is HARD.  Either way the forced decision is adopted and the sweep continues,
 * so later comparisons stay aligned.  stats = {code ties, code hard, rung ties, rung hard}.
 */
int orc_sweep(const float* W0, int64_t rows, int64_t n, int64_t gs, const double* U,
              const float* hdiag, const uint8_t* dead, const float* tab, const float* lost,
              uint8_t* code, uint8_t* rung, float* scale, double* E, double* Wc,
              const uint8_t* force_code, const uint8_t* force_rung, double tie_band,
              double rung_band, int64_t* stats, int nt) {
    if (gs <= 0 || n % gs != 0 || gs > 64) return ORC_FAILED;
    const int64_t ng = n / gs;
    const int64_t RB = 16; /* rows per task: a row of U is read once for the whole block */
    int64_t ct = 0, ch = 0, rt = 0, rh = 0;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1) reduction(+ : ct, ch, rt, rh)
    for (int64_t r0 = 0; r0 < rows; r0 += RB) {
        int64_t rb = imin(RB, rows - r0);
        double* w = (double*)malloc(sizeof(double) * (size_t)(rb * n));
        double e[16];
        float sc[16];
        for (int64_t k = 0; k < rb; ++k)
            for (int64_t j = 0; j < n; ++j)
                w[k * n + j] = dead[j] ? 0.0 : (double)W0[(r0 + k) * n + j];
        for (int64_t g = 0; g < ng; ++g) {
            int64_t c0 = g * gs;
            const float* hd = hdiag + c0;
            for (int64_t k = 0; k < rb; ++k) {
                int64_t r = r0 + k;
                const float* tb = tab + r * 32;
                float wf[64];
                float amax = 0.0f;
                for (int64_t t = 0; t < gs; ++t) {
                    wf[t] = (float)w[k * n + c0 + t];
                    float a = fabsf(wf[t]);
                    if (a > amax) amax = a;
                }
                double v;
                int nominal = nominal_rung(amax, lost[r * 2], lost[r * 2 + 1], &v);
                int best = nominal;
                float best_e = INFINITY;
                if (amax > 0.0f) {
                    int lo_c = nominal >= 2 ? nominal - 2 : 0;
                    int hi_c = nominal + 1 < 31 ? nominal + 1 : 31;
                    for (int cand = lo_c; cand <= hi_c; ++cand) {
                        float s_c = tb[cand];
                        if (s_c <= 0.0f) continue;
                        float err = tile_error(wf, hd, gs, s_c);
                        if (err < best_e) {
                            best_e = err;
                            best = cand;
                        }
                    }
                }
                if (force_rung) {
                    int fr = force_rung[r * ng + g];
                    if (fr != best) {
                        int tie = 0;
                        if (fr >= 0 && fr < 32 && tb[fr] > 0.0f && amax > 0.0f) {
                            float ef = tile_error(wf, hd, gs, tb[fr]);
                            float lo_e = ef < best_e ? ef : best_e;
                            if (fabs((double)ef - (double)best_e) <= rung_band * (double)lo_e)
                                tie = 1;
                        }
                        if (amax > 0.0f && lost[r * 2 + 1] > 0.0f) {
                            double fr_v = v - floor(v);
                            if (fabs(fr_v - 0.5) < tie_band) tie = 1;
                        }
                        if (tie) ++rt; else ++rh;
                        best = fr;
                    }
                }
                rung[r * ng + g] = (uint8_t)best;
                sc[k] = tb[best];
                scale[r * ng + g] = sc[k];
            }
            for (int64_t j = c0; j < c0 + gs; ++j) {
                double ujj = U[j * n + j];
                for (int64_t k = 0; k < rb; ++k) {
                    int64_t r = r0 + k;
                    double wj = w[k * n + j];
                    float s = sc[k];
                    float q = 0.0f;
                    if (s > 0.0f) q = clampf(rne_f32((float)wj / s), -8.0f, 7.0f);
                    if (force_code) {
                        float fq = (float)force_code[r * n + j] - 8.0f;
                        if (fq != q) {
                            double x = fabs((double)((float)wj / s));
                            double fr = x - floor(x);
                            if (fabsf(fq - q) == 1.0f && fabs(fr - 0.5) < tie_band) ++ct; else ++ch;
                            q = fq;
                        }
                    }
                    code[r * n + j] = (uint8_t)(q + 8.0f);
                    if (Wc) Wc[r * n + j] = wj;
                    e[k] = (ujj > 0.0) ? (wj - (double)q * (double)s) / ujj : 0.0;
                    if (E) E[r * n + j] = e[k];
                }
                const double* urow = U + j * n;
                for (int64_t k = 0; k < rb; ++k) {
                    double ek = e[k];
                    if (ek == 0.0) continue;
                    double* wr = w + k * n;
                    for (int64_t t = j + 1; t < n; ++t) wr[t] -= ek * urow[t];
                }
            }
        }
        free(w);
    }
    if (stats) {
        stats[0] = ct;
        stats[1] = ch;
        stats[2] = rt;
        stats[3] = rh;
    }
    return ORC_OK;
}

/*
 * Act-order sweep with static groups ([gptq.rs] gptq_quantize_q4tp_act_order; for 2-bit codes,
 * gptq_quantize_q2tp with a permutation): the columns of Wp (rows x n, already in elimination
 * order and dead-zeroed) are eliminated in order with the fold operator Up of the permuted
 * Hessian, each column a with its own fixed scale sp[r][a] (the rung of its original group,
 * chosen up front):
 *   4-bit: q = (s > 0) ? clamp(rne(f32(w_a) / s), -8, 7) : 0,  code = q + 8,  level q;
 *   2-bit: q = (s > 0) ? q2_level(f32(w_a) / s + 1.5) : 0,      code = q,      level q - 1.5;
 *   e_a = (Up_aa > 0) ? (w_a - level s) / Up_aa : 0,  w_t -= e_a Up_at for every t > a.
 * code_p and E are in elimination order.  force_code: tie-forced replay as in orc_sweep (for
 * 2-bit codes a tie is a difference of one where f32(w_a)/s + 1.5 lies within tie_band of a
 * half-integer).
 */
static float q2_level(float x);

int orc_sweep_static(const float* Wp, int64_t rows, int64_t n, const double* Up, const float* sp,
                     int two_bit, uint8_t* code_p, double* E, const uint8_t* force_code,
                     double tie_band, int64_t* stats, int nt) {
    const int64_t RB = 16;
    int64_t ct = 0, ch = 0;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1) reduction(+ : ct, ch)
    for (int64_t r0 = 0; r0 < rows; r0 += RB) {
        int64_t rb = imin(RB, rows - r0);
        double* w = (double*)malloc(sizeof(double) * (size_t)(rb * n));
        double e[16];
        for (int64_t k = 0; k < rb; ++k)
            for (int64_t a = 0; a < n; ++a) w[k * n + a] = (double)Wp[(r0 + k) * n + a];
        for (int64_t a = 0; a < n; ++a) {
            double uaa = Up[a * n + a];
            for (int64_t k = 0; k < rb; ++k) {
                int64_t r = r0 + k;
                double wa = w[k * n + a];
                float s = sp[r * n + a];
                float q = 0.0f, x = 0.0f;
                if (s > 0.0f) {
                    if (two_bit) {
                        x = (float)wa / s + 1.5f;
                        q = q2_level(x);
                    } else {
                        x = (float)wa / s;
                        q = clampf(rne_f32(x), -8.0f, 7.0f);
                    }
                }
                if (force_code) {
                    float fq = (float)force_code[r * n + a] - (two_bit ? 0.0f : 8.0f);
                    if (fq != q) {
                        double ax = two_bit ? (double)x : fabs((double)x);
                        double fr = ax - floor(ax);
                        if (fabsf(fq - q) == 1.0f && fabs(fr - 0.5) < tie_band) ++ct; else ++ch;
                        q = fq;
                    }
                }
                code_p[r * n + a] = (uint8_t)(two_bit ? q : q + 8.0f);
                double lev = two_bit ? (double)q - 1.5 : (double)q;
                e[k] = (uaa > 0.0) ? (wa - lev * (double)s) / uaa : 0.0;
                if (E) E[r * n + a] = e[k];
            }
            const double* urow = Up + a * n;
            for (int64_t k = 0; k < rb; ++k) {
                double ek = e[k];
                if (ek == 0.0) continue;
                double* wr = w + k * n;
                for (int64_t t = a + 1; t < n; ++t) wr[t] -= ek * urow[t];
            }
        }
        free(w);
    }
    if (stats) {
        stats[0] = ct;
        stats[1] = ch;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* q2tp ("placed" rule).  [gptq_dev.rs] q2tp_group and [gptq.rs] sweep_q2tp /
 * gptq_quantize_q2tp: 2-bit levels (q - 1.5) s with q = q2_level(w / s + 1.5),
 * q2_level(x) = clamp(rne(clamp(x, -1, 4)), 0, 3); rung 0 is the all-zero group (TAB[0] = 0);
 * a group with a nonzero entry takes the best of rungs 1..31 by the clipped-H_ii-weighted
 * rounding error (a strictly smaller error replaces the current best, starting from rung 1). */
static float q2_level(float x) {
    float c = clampf(x, -1.0f, 4.0f);
    return clampf(rne_f32(c), 0.0f, 3.0f);
}

static float q2_tile_error(const float* wf, const float* hw, int64_t gs, float s) {
    float err = 0.0f;
    for (int64_t t = 0; t < gs; ++t) {
        float q = q2_level(wf[t] / s + 1.5f);
        float qs = (q - 1.5f) * s;
        float d = wf[t] - qs;
        float hd = hw[t] * d;
        err = err + hd * d;
    }
    return err;
}

/*
 * The q2tp ladder.  The pages place it with a helper that is not printed (q2tp_place_row, "the
 * ladder placed at the H_ii-weighted MSE-optimal group scales"); the reading used here is the
 * absmax rule of the q4tp ladder moved to the 2-bit grid, whose outer level is 1.5 s: over the
 * groups with a_g > 0, lo = f16(log2(min a_g / 1.5)), hi = log2(max a_g / 1.5),
 * step = f16((hi - lo) / 30) if hi > lo else 0, TAB[0] = 0 and TAB[c] = f32(2^(lo + (c-1) step))
 * for c = 1..31 (f64); a row with no nonzero group gets lo = step = 0 and TAB[c >= 1] = 1.
 * The sweep's full rung search then picks the best rung of this ladder.
 */
void orc_ladder_q2(const float* W0, const uint8_t* dead, int64_t rows, int64_t n, int64_t gs,
                   float* lost, float* tab) {
    for (int64_t r = 0; r < rows; ++r) {
        double amin = INFINITY, amax = 0.0;
        for (int64_t g = 0; g < n / gs; ++g) {
            float a = 0.0f;
            for (int64_t t = 0; t < gs; ++t) {
                int64_t j = g * gs + t;
                float v = dead[j] ? 0.0f : fabsf(W0[r * n + j]);
                if (v > a) a = v;
            }
            if (a > 0.0f) {
                if (a < amin) amin = a;
                if (a > amax) amax = a;
            }
        }
        double lo = 0.0, st = 0.0;
        if (amax > 0.0) {
            lo = orc_f16_round(log2(amin / 1.5));
            double hi = log2(amax / 1.5);
            st = (hi > lo) ? orc_f16_round((hi - lo) / 30.0) : 0.0;
            if (!(st > 0.0)) st = 0.0;
        }
        lost[r * 2] = (float)lo;
        lost[r * 2 + 1] = (float)st;
        tab[r * 32] = 0.0f;
        for (int c = 1; c < 32; ++c)
            tab[r * 32 + c] = (amax > 0.0) ? (float)exp2(lo + (double)(c - 1) * st) : 1.0f;
    }
}

/*
 * The q2tp sweep, column by column (f64 state; decisions in f32 as orc_sweep):
 *   for each group g (c0 = gs g), each row: wf = f32(w[c0 .. c0+gs)); rung 0 if max |wf| = 0,
 *   else the best of rungs 1..31 with TAB > 0 by q2_tile_error (weights hw = max(H_ii, 0));
 *   s = TAB[rung]; for j in the group in order: q = (s > 0) ? q2_level(f32(w_j) / s + 1.5) : 0,
 *   code = q (0..3), e_j = (U_jj > 0) ? (w_j - (q - 1.5) s) / U_jj : 0, w_t -= e_j U_jt (t > j).
 * Tie-forced replay as orc_sweep; a code tie is a difference of one where f32(w_j)/s + 1.5
 * lies within tie_band of a half-integer.
 */
int orc_sweep_q2(const float* W0, int64_t rows, int64_t n, int64_t gs, const double* U,
                 const float* hw, const uint8_t* dead, const float* tab, uint8_t* code,
                 uint8_t* rung, float* scale, double* E, const uint8_t* force_code,
                 const uint8_t* force_rung, double tie_band, double rung_band, int64_t* stats,
                 int nt) {
    if (gs <= 0 || n % gs != 0 || gs > 64) return ORC_FAILED;
    const int64_t ng = n / gs;
    const int64_t RB = 16;
    int64_t ct = 0, ch = 0, rt = 0, rh = 0;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1) reduction(+ : ct, ch, rt, rh)
    for (int64_t r0 = 0; r0 < rows; r0 += RB) {
        int64_t rb = imin(RB, rows - r0);
        double* w = (double*)malloc(sizeof(double) * (size_t)(rb * n));
        double e[16];
        float sc[16];
        for (int64_t k = 0; k < rb; ++k)
            for (int64_t j = 0; j < n; ++j)
                w[k * n + j] = dead[j] ? 0.0 : (double)W0[(r0 + k) * n + j];
        for (int64_t g = 0; g < ng; ++g) {
            int64_t c0 = g * gs;
            const float* hg = hw + c0;
            for (int64_t k = 0; k < rb; ++k) {
                int64_t r = r0 + k;
                const float* tb = tab + r * 32;
                float wf[64];
                float amax = 0.0f;
                for (int64_t t = 0; t < gs; ++t) {
                    wf[t] = (float)w[k * n + c0 + t];
                    float a = fabsf(wf[t]);
                    if (a > amax) amax = a;
                }
                int best = 0;
                float best_e = INFINITY;
                if (amax > 0.0f) {
                    best = 1;
                    for (int cand = 1; cand < 32; ++cand) {
                        float s_c = tb[cand];
                        if (!(s_c > 0.0f)) continue;
                        float err = q2_tile_error(wf, hg, gs, s_c);
                        if (err < best_e) {
                            best_e = err;
                            best = cand;
                        }
                    }
                }
                if (force_rung) {
                    int fr = force_rung[r * ng + g];
                    if (fr != best) {
                        int tie = 0;
                        if (fr >= 1 && fr < 32 && tb[fr] > 0.0f && amax > 0.0f && best_e < INFINITY) {
                            float ef = q2_tile_error(wf, hg, gs, tb[fr]);
                            float lo_e = ef < best_e ? ef : best_e;
                            if (fabs((double)ef - (double)best_e) <= rung_band * (double)lo_e) tie = 1;
                        }
                        if (tie) ++rt; else ++rh;
                        best = fr;
                    }
                }
                rung[r * ng + g] = (uint8_t)best;
                sc[k] = tb[best & 31];
                scale[r * ng + g] = sc[k];
            }
            for (int64_t j = c0; j < c0 + gs; ++j) {
                double ujj = U[j * n + j];
                for (int64_t k = 0; k < rb; ++k) {
                    int64_t r = r0 + k;
                    double wj = w[k * n + j];
                    float s = sc[k];
                    float q = 0.0f;
                    float x = 0.0f;
                    if (s > 0.0f) {
                        x = (float)wj / s + 1.5f;
                        q = q2_level(x);
                    }
                    if (force_code) {
                        float fq = (float)force_code[r * n + j];
                        if (fq != q) {
                            double fr = (double)x - floor((double)x);
                            if (fabsf(fq - q) == 1.0f && fabs(fr - 0.5) < tie_band) ++ct; else ++ch;
                            q = fq;
                        }
                    }
                    code[r * n + j] = (uint8_t)q;
                    e[k] = (ujj > 0.0) ? (wj - ((double)q - 1.5) * (double)s) / ujj : 0.0;
                    if (E) E[r * n + j] = e[k];
                }
                const double* urow = U + j * n;
                for (int64_t k = 0; k < rb; ++k) {
                    double ek = e[k];
                    if (ek == 0.0) continue;
                    double* wr = w + k * n;
                    for (int64_t t = j + 1; t < n; ++t) wr[t] -= ek * urow[t];
                }
            }
        }
        free(w);
    }
    if (stats) {
        stats[0] = ct;
        stats[1] = ch;
        stats[2] = rt;
        stats[3] = rh;
    }
    return ORC_OK;
}

int orc_max_threads(void) { return omp_get_max_threads(); }
