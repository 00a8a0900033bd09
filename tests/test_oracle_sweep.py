"""Pins of the oracle's q4tp sweep against facts fixed outside the oracle itself.

The sweep ("cortiq-cli 0.8.45 src/gptq.rs", gptq_quantize_q4tp; "cortiq-engine 0.8.41
src/gpu_wgpu/gptq_dev.rs", q4tp_group and the module documentation, step 5) rounds the columns
left to right and feeds each scaled residual e_j = (w_j - q_j s)/U_jj into the later columns
through row j of U.  The pins: column-sequential OBS with explicit re-inversion (the update the
pages say the fold makes exact), the identity Hessian (plain rounding), the algebraic identity
dW = E U, hand-built rung cases, a property of the method, and the storage layout.
"""
import numpy as np
import pytest

import oracle
import workloads


def _ladder(W, lo_off=-1.0, st=1.0 / 16):
    """A spread ladder (valid sweep input) independent of the ladder rule under test."""
    rows = W.shape[0]
    amax = np.abs(W).max(axis=1).astype(np.float64)
    lo = np.array([oracle.f16_round(np.log2(a / 7.0) + lo_off) for a in amax])
    lost = np.stack([lo, np.full(rows, st)], axis=1).astype(np.float32)
    tab = np.exp2(lo[:, None] + np.arange(32)[None, :] * st).astype(np.float32)
    return lost, tab


def _obs_bruteforce(W0, hd, s):
    """Column-sequential OBS: for each column j, with F the columns not yet rounded,
    Hinv_F = inv(H_d[F, F]) and w_F -= (w_j - q_j s) / Hinv_F[j, j] * Hinv_F[j, F]."""
    n = W0.shape[0]
    w = W0.astype(np.float64).copy()
    codes = np.zeros(n, dtype=np.uint8)
    e = np.zeros(n)
    for j in range(n):
        F = np.arange(j, n)
        hinv = np.linalg.inv(hd[np.ix_(F, F)])
        q = np.float32(np.clip(np.rint(np.float32(w[j]) / np.float32(s)), -8, 7))
        codes[j] = int(q) + 8
        r = w[j] - float(q) * float(s)
        e[j] = r / np.sqrt(hinv[0, 0])
        w[F] -= r / hinv[0, 0] * hinv[0, :]
    return codes, e


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("n", [1, 3, 5, 8])
def test_matches_column_sequential_obs(seed, n):
    rng = np.random.default_rng(100 + seed)
    X = rng.standard_normal((n, 2 * n + 3)) * np.exp(rng.standard_normal(n))[:, None]
    H = (X @ X.T).astype(np.float32)
    rows = 6
    W = (rng.standard_normal((rows, n)) * 0.05).astype(np.float32)
    f = oracle.fold(H, 0.01)
    lost, tab = _ladder(W)
    hd = np.triu(H.astype(np.float64))
    hd = hd + np.triu(hd, 1).T + f["damp"] * np.eye(n)
    s_ = oracle.sweep(W, f["U"], f["hdiag"], f["dead"], tab, lost, gs=n)
    for r in range(rows):
        s = s_["scale"][r, 0]
        codes, e = _obs_bruteforce(W[r], hd, s)
        np.testing.assert_array_equal(s_["code"][r], codes)
        np.testing.assert_allclose(s_["E"][r], e, rtol=1e-9, atol=1e-14)
    t_orc = oracle.output_error(W, f["dead"], s_["code"], s_["scale"], H, gs=n)
    assert t_orc >= 0.0


def test_identity_hessian_is_round_to_nearest():
    rng = np.random.default_rng(7)
    n, rows, lam = 96, 40, 0.01
    W = (rng.standard_normal((rows, n)) * 0.02).astype(np.float32)
    f = oracle.fold(np.eye(n, dtype=np.float32), lam)
    lost, tab = oracle.ladder(W, f["dead"])
    s = oracle.sweep(W, f["U"], f["hdiag"], f["dead"], tab, lost)
    sc = np.repeat(s["scale"], 32, axis=1)
    q = np.clip(np.rint(W / sc), -8, 7)          # f32 division, ties to even
    np.testing.assert_array_equal(s["code"].astype(np.int16) - 8, q.astype(np.int16))
    np.testing.assert_allclose(s["E"], (W.astype(np.float64) - q.astype(np.float64) * sc) * np.sqrt(1 + lam),
                               rtol=1e-12, atol=1e-18)


def test_residuals_reproduce_the_error_exactly():
    """dW = E U column by column, hence tr(dW H_d dW^T) = ||E||_F^2 and, with dead columns of
    dW zero, tr(dW H dW^T) = ||E||_F^2 - damp ||dW||_F^2."""
    H, W, lam = workloads.make("tiny")
    H, W = H.numpy(), W.numpy()
    f = oracle.fold(H, lam)
    lost, tab = oracle.ladder(W, f["dead"])
    s = oracle.sweep(W, f["U"], f["hdiag"], f["dead"], tab, lost)
    Wz = W.astype(np.float64)
    Wz[:, f["dead"]] = 0.0
    dW = Wz - oracle.dequant(s["code"], s["scale"])
    np.testing.assert_allclose(s["E"] @ f["U"], dW, rtol=0, atol=1e-12 * np.abs(dW).max())
    assert np.all(dW[:, f["dead"]] == 0.0)
    t = oracle.output_error(W, f["dead"], s["code"], s["scale"], H)
    e2 = float((s["E"] ** 2).sum())
    np.testing.assert_allclose(t, e2 - f["damp"] * float((dW ** 2).sum()), rtol=1e-9)


def test_gptq_beats_round_to_nearest_on_correlated_inputs():
    """The pages' property test: on correlated activations the output error of the sweep is
    below 0.8x that of plain rounding with the same ladder."""
    H, W, X = workloads.lcg_fixture()
    f = oracle.fold(H, 0.01)
    assert not f["dead"].any()
    lost, tab = oracle.ladder(W, f["dead"])
    g = oracle.sweep(W, f["U"], f["hdiag"], f["dead"], tab, lost)
    ident = np.eye(W.shape[1])
    rtn = oracle.sweep(W, ident, np.ones(W.shape[1], np.float32), f["dead"], tab, lost)

    def out_err(s):
        dW = W.astype(np.float64) - oracle.dequant(s["code"], s["scale"])
        return float(((X.astype(np.float64) @ dW.T) ** 2).sum())

    assert out_err(g) < 0.8 * out_err(rtn), (out_err(g), out_err(rtn))


def _tile_errors(w, h, tab):
    out = []
    for s in tab:
        err = np.float32(0.0)
        for t in range(len(w)):
            q = np.float32(np.clip(np.rint(w[t] / s), -8, 7))
            d = np.float32(w[t] - q * s)
            err = np.float32(err + np.float32(h[t] * d) * d)
        out.append(err)
    return np.array(out, dtype=np.float32)


def _one_tile(w, h, lo, st):
    n = len(w)
    lost = np.array([[lo, st]], dtype=np.float32)
    tab = np.exp2(lo + np.arange(32) * np.float64(st)).astype(np.float32)[None, :]
    s = oracle.sweep(w[None, :].astype(np.float32), np.eye(n), h.astype(np.float32),
                     np.zeros(n, bool), tab, lost, gs=n)
    return int(s["rung"][0, 0]), tab[0]


def test_rung_rule_hand_built_tiles():
    # Small weights that are exact multiples of rung 16's scale 2^-4, plus an outlier in a
    # channel with tiny H_ii: the absmax 0.9 sets the nominal rung to 18 (log2(0.9/7) = -2.96,
    # (-2.96 + 12) / 0.5 = 18.08), but the weighted error is smallest at nominal - 2 = 16.
    w = np.where(np.arange(32) % 2 == 0, 0.0625, -0.125).astype(np.float32)
    w[5] = 0.9
    h = np.ones(32, dtype=np.float32)
    h[5] = 1e-6
    lo, st = -12.0, 0.5
    nominal = 18
    rung, tab = _one_tile(w, h, lo, st)
    assert tab[16] == np.float32(0.0625)
    assert rung == nominal - 2
    errs = _tile_errors(w, h, tab)
    assert errs[rung] == errs[nominal - 2:nominal + 2].min()
    # Same tile with a unit weight on the outlier channel: rung 16 clamps the outlier at 7 s
    # and loses to a larger rung.
    rung_u, _ = _one_tile(w, np.ones(32, np.float32), lo, st)
    errs_u = _tile_errors(w, np.ones(32, np.float32), tab)
    assert rung_u > 16 and errs_u[rung_u] == errs_u[16:20].min()
    # All-zero tile: no search, rung 0.
    rung0, _ = _one_tile(np.zeros(32, np.float32), h, lo, st)
    assert rung0 == 0
    # step 0: nominal 0, window {0, 1}; both rungs equal -> strict '<' keeps the lower.
    rung_flat, _ = _one_tile(w, h, -5.0, 0.0)
    assert rung_flat == 0


def test_rung_rule_exhaustive_window_random_tiles():
    rng = np.random.default_rng(3)
    for trial in range(40):
        w = (rng.standard_normal(32) * np.exp(rng.standard_normal())).astype(np.float32) * 0.01
        h = np.exp(2 * rng.standard_normal(32)).astype(np.float32)
        lo = float(np.floor(np.log2(np.abs(w).min() + 1e-9) - 1))
        st = 0.25
        rung, tab = _one_tile(w, h, lo, st)
        errs = _tile_errors(w, h, tab)
        v = (np.log2(np.float64(np.abs(w).max()) / 7.0) - lo) / st
        nominal = int(np.clip(np.sign(v) * np.floor(abs(v) + 0.5), 0, 31))
        lo_c, hi_c = max(nominal - 2, 0), min(nominal + 1, 31)
        assert lo_c <= rung <= hi_c
        win = errs[lo_c:hi_c + 1]
        assert errs[rung] == win.min()
        assert rung == lo_c + int(np.argmin(win))     # first minimum: ties keep the lower


def test_layout_round_trip_and_dead_columns():
    H, W, lam = workloads.make("tiny")
    H, W = H.numpy(), W.numpy()
    f = oracle.fold(H, lam)
    lost, tab = oracle.ladder(W, f["dead"])
    s = oracle.sweep(W, f["U"], f["hdiag"], f["dead"], tab, lost)
    nib = oracle.pack_nibbles(s["code"])
    assert nib.shape == (W.shape[0], W.shape[1] // 2)
    np.testing.assert_array_equal(oracle.unpack_nibbles(nib), s["code"])
    np.testing.assert_array_equal(nib[:, 0] & 0x0F, s["code"][:, 0])
    np.testing.assert_array_equal(nib[:, 0] >> 4, s["code"][:, 1])
    wh = oracle.dequant(s["code"], s["scale"])
    assert np.all(wh[:, f["dead"]] == 0.0)
    np.testing.assert_array_equal(s["scale"], np.take_along_axis(tab, s["rung"].astype(int), 1))


def test_thread_count_does_not_change_bits():
    H, W, lam = workloads.make("fixture")
    H, W = H.numpy(), W.numpy()
    f = oracle.fold(H, lam)
    lost, tab = oracle.ladder(W, f["dead"])
    a = oracle.sweep(W, f["U"], f["hdiag"], f["dead"], tab, lost, nt=1)
    b = oracle.sweep(W, f["U"], f["hdiag"], f["dead"], tab, lost, nt=5)
    for k in ("code", "rung", "scale", "E"):
        np.testing.assert_array_equal(a[k], b[k])


def test_replay_counts_ties_and_hard_disagreements():
    H, W, lam = workloads.make("fixture")
    H, W = H.numpy(), W.numpy()
    f = oracle.fold(H, lam)
    lost, tab = oracle.ladder(W, f["dead"])
    s = oracle.sweep(W, f["U"], f["hdiag"], f["dead"], tab, lost, want_Wc=True)
    same = oracle.sweep(W, f["U"], f["hdiag"], f["dead"], tab, lost,
                        force_code=s["code"], force_rung=s["rung"])
    assert same["stats"] == dict(code_ties=0, code_hard=0, rung_ties=0, rung_hard=0)
    # Planted mistakes in the last column of a row (nothing downstream depends on it): far
    # from a rounding tie it is hard; near one (band widened to 0.2) it is a tie.
    n = W.shape[1]
    sc = s["scale"][:, -1]
    x = np.abs(s["Wc"][:, -1].astype(np.float32) / sc)
    frac = x - np.floor(x)
    code = s["code"][:, -1].astype(int)
    live = (code > 1) & (code < 14)
    far = int(np.nonzero(live & (np.abs(frac - 0.5) > 0.3))[0][0])
    bad = s["code"].copy()
    bad[far, n - 1] += 1
    r = oracle.sweep(W, f["U"], f["hdiag"], f["dead"], tab, lost, force_code=bad,
                     force_rung=s["rung"])
    assert r["stats"] == dict(code_ties=0, code_hard=1, rung_ties=0, rung_hard=0)
    near = int(np.nonzero(live & (np.abs(frac - 0.5) < 0.2))[0][0])
    away = 1 if frac[near] >= 0.5 else -1        # the other neighbour of |w/s|
    sign = 1 if s["Wc"][near, -1] >= 0 else -1
    bad2 = s["code"].copy()
    q = code[near] - 8
    bad2[near, n - 1] = (sign * (abs(q) - away) if abs(q) - away >= 0 else q - sign) + 8
    r2 = oracle.sweep(W, f["U"], f["hdiag"], f["dead"], tab, lost, force_code=bad2,
                      force_rung=s["rung"], tie_band=0.2)
    assert r2["stats"] == dict(code_ties=1, code_hard=0, rung_ties=0, rung_hard=0)
