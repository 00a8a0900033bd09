"""Pins of the oracle's q2tp sweep ("placed" rule; "cortiq-engine 0.8.41 src/gpu_wgpu/
gptq_dev.rs", q2tp_group; "cortiq-cli 0.8.45 src/gptq.rs", sweep_q2tp) against facts fixed
outside it: nearest-level rounding under the identity Hessian (no feedback), column-sequential
OBS with explicit re-inversion on tiny inputs, the full rung search against an exhaustive
enumeration of rungs 1..31 with clipped weights, rung 0 for an all-zero group, dW = E U, the
2-bit plane layout, and GPTQ beating round-to-nearest on correlated inputs."""
import numpy as np
import pytest

import oracle
import workloads


def q2_level(x):
    return np.clip(np.rint(np.clip(np.float32(x), -1.0, 4.0)), 0.0, 3.0).astype(np.float32)


def test_identity_hessian_is_nearest_level():
    rng = np.random.default_rng(1)
    n, rows, lam = 64, 20, 0.01
    W = (rng.standard_normal((rows, n)) * 0.02).astype(np.float32)
    f = oracle.fold(np.eye(n, dtype=np.float32), lam)
    lost, tab = oracle.ladder_q2(W, f["dead"])
    s = oracle.sweep_q2(W, f["U"], f["hdiag"], f["dead"], tab)
    sc = np.repeat(s["scale"], 32, axis=1)
    q = q2_level((W / sc).astype(np.float32) + np.float32(1.5))
    assert np.array_equal(s["code"], q.astype(np.uint8))
    np.testing.assert_allclose(s["E"], (W - (q.astype(np.float64) - 1.5) * sc) * np.sqrt(1 + lam),
                               rtol=1e-12, atol=1e-18)


def _obs_q2(w0, hd, s):
    n = w0.shape[0]
    w = w0.astype(np.float64).copy()
    codes = np.zeros(n, np.uint8)
    e = np.zeros(n)
    for j in range(n):
        F = np.arange(j, n)
        hinv = np.linalg.inv(hd[np.ix_(F, F)])
        q = q2_level(np.float32(np.float32(w[j]) / np.float32(s)) + np.float32(1.5))
        codes[j] = int(q)
        r = w[j] - (float(q) - 1.5) * float(s)
        e[j] = r / np.sqrt(hinv[0, 0])
        w[F] -= r / hinv[0, 0] * hinv[0, :]
    return codes, e


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
@pytest.mark.parametrize("n", [2, 5, 8])
def test_matches_column_sequential_obs(seed, n):
    rng = np.random.default_rng(200 + seed)
    X = rng.standard_normal((n, 2 * n + 3)) * np.exp(rng.standard_normal(n))[:, None]
    H = (X @ X.T).astype(np.float32)
    W = (rng.standard_normal((5, n)) * 0.05).astype(np.float32)
    f = oracle.fold(H, 0.01)
    lost, tab = oracle.ladder_q2(W, f["dead"], gs=n)
    s_ = oracle.sweep_q2(W, f["U"], f["hdiag"], f["dead"], tab, gs=n)
    hd = oracle.symmetric_from_upper(H) + f["damp"] * np.eye(n)
    for r in range(5):
        codes, e = _obs_q2(W[r], hd, s_["scale"][r, 0])
        assert np.array_equal(s_["code"][r], codes)
        np.testing.assert_allclose(s_["E"][r], e, rtol=1e-9, atol=1e-14)


def test_full_search_is_exhaustive_with_clipped_weights():
    rng = np.random.default_rng(3)
    rows, n = 6, 64
    W = (rng.standard_normal((rows, n)) * np.exp(rng.standard_normal((rows, 1)))).astype(np.float32)
    hd = rng.uniform(-0.5, 3.0, n).astype(np.float32)   # negative weights must count as 0
    dead = np.zeros(n, bool)
    lost, tab = oracle.ladder_q2(W, dead)
    s = oracle.sweep_q2(W, np.eye(n), hd, dead, tab)
    hw = np.maximum(hd, 0)
    for r in range(rows):
        for g in range(n // 32):
            w = W[r, 32 * g:32 * g + 32]
            best, best_e = 1, np.inf
            for c in range(1, 32):
                sc = tab[r, c]
                err = np.float32(0)
                for t in range(32):
                    q = q2_level(np.float32(w[t] / sc) + np.float32(1.5))
                    d = np.float32(w[t] - np.float32((q - np.float32(1.5)) * sc))
                    err = np.float32(err + np.float32(np.float32(hw[32 * g + t] * d) * d))
                if err < best_e:
                    best, best_e = c, err
            assert s["rung"][r, g] == best


def test_zero_group_and_dead_columns():
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((3, 64)) * 0.1).astype(np.float32)
    W[1, 32:] = 0.0
    dead = np.zeros(64, bool)
    dead[[0, 7]] = True
    lost, tab = oracle.ladder_q2(W, dead)
    assert np.all(tab[:, 0] == 0.0)
    s = oracle.sweep_q2(W, np.eye(64), np.ones(64, np.float32), dead, tab)
    assert s["rung"][1, 1] == 0 and s["scale"][1, 1] == 0.0
    What = oracle.dequant_q2(s["code"], s["scale"])
    assert np.all(What[1, 32:] == 0.0)
    assert np.all(np.abs(What[:, dead]) <= 1.5 * s["scale"][:, :1])


def test_residuals_reproduce_the_error():
    H, W, lam = workloads.make("tiny")
    H, W = H.numpy(), W.numpy()
    f = oracle.fold(H, lam)
    lost, tab = oracle.ladder_q2(W, f["dead"])
    s = oracle.sweep_q2(W, f["U"], f["hdiag"], f["dead"], tab)
    Wz = W.astype(np.float64)
    Wz[:, f["dead"]] = 0.0
    dW = Wz - oracle.dequant_q2(s["code"], s["scale"])
    np.testing.assert_allclose(dW, s["E"] @ f["U"], rtol=1e-9, atol=1e-12)


def test_plane_layout_round_trip():
    rng = np.random.default_rng(5)
    code = rng.integers(0, 4, size=(7, 96)).astype(np.uint8)
    plane = oracle.pack_q2(code)
    assert plane.shape == (7, 24)
    assert plane[0, 0] == (code[0, 0] | code[0, 1] << 2 | code[0, 2] << 4 | code[0, 3] << 6)
    assert np.array_equal(oracle.unpack_q2(plane), code)


def test_gptq_beats_rounding_on_correlated_inputs():
    H, W, X = workloads.lcg_fixture()
    f = oracle.fold(H, 0.01)
    lost, tab = oracle.ladder_q2(W, f["dead"])
    g = oracle.sweep_q2(W, f["U"], f["hdiag"], f["dead"], tab)
    r = oracle.sweep_q2(W, np.eye(W.shape[1]), f["hdiag"], f["dead"], tab)
    def out_err(code, scale):
        dW = W.astype(np.float64) - oracle.dequant_q2(code, scale)
        return float(np.sum((X.astype(np.float64) @ dW.T) ** 2))
    assert out_err(g["code"], g["scale"]) < out_err(r["code"], r["scale"])


def _f16_half_ulp(x):
    return 0.5 * oracle.f16_ulp(x)


def test_q2_ladder_reading_is_pinned():
    """The q2tp ladder reading: lo and step are binary16 values; TAB[0] = 0 (the all-zero
    group), TAB[1] = 2^lo exactly in f32, TAB non-decreasing from rung 1; lo sits within half an
    f16 step of log2(min a_g / 1.5) and lo + 30 step within the f16 rounding of step of
    log2(max a_g / 1.5), so the outer level 1.5 TAB of the lowest and highest rungs spans the
    row's smallest and largest group absmax.  A divisor of 31, or rungs counted from c instead
    of c - 1, fails these."""
    rng = np.random.default_rng(77)
    rows, n = 40, 256
    W = (rng.standard_normal((rows, n)) * np.exp(rng.standard_normal((rows, 1)))
         * np.exp(0.8 * rng.standard_normal((1, n)))).astype(np.float32)
    dead = np.zeros(n, bool)
    dead[[3, 100]] = True
    lost, tab = oracle.ladder_q2(W, dead)
    Wd = W.copy()
    Wd[:, dead] = 0.0
    a = np.abs(Wd).reshape(rows, n // 32, 32).max(axis=2).astype(np.float64)
    for r in range(rows):
        lo, st = float(lost[r, 0]), float(lost[r, 1])
        assert np.float16(lo) == lo and np.float16(st) == st
        assert tab[r, 0] == 0.0
        assert tab[r, 1] == np.float32(2.0 ** lo)
        assert np.all(np.diff(tab[r, 1:]) >= 0)
        ag = a[r][a[r] > 0]
        lo_t, hi_t = np.log2(ag.min() / 1.5), np.log2(ag.max() / 1.5)
        assert abs(lo - lo_t) <= _f16_half_ulp(lo_t) * (1 + 1e-12)
        assert abs(lo + 30 * st - hi_t) <= 30 * _f16_half_ulp(st) + _f16_half_ulp(lo_t) + 1e-12
        for c in range(1, 32):
            assert tab[r, c] == np.float32(2.0 ** (lo + (c - 1) * st))
    # An all-zero row: lo = step = 0 and every rung from 1 is 1.
    lost0, tab0 = oracle.ladder_q2(np.zeros((1, 64), np.float32), np.zeros(64, bool))
    assert lost0[0, 0] == 0.0 and lost0[0, 1] == 0.0 and tab0[0, 0] == 0.0 and np.all(tab0[0, 1:] == 1.0)


# --- act order with static groups, 2-bit levels ------------------------------------------------

def _problem(n, rows, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, 2 * n + 5)) * np.exp(rng.standard_normal(n))[:, None]
    H = (X @ X.T).astype(np.float32)
    W = (rng.standard_normal((rows, n)) * 0.05).astype(np.float32)
    return H, W


def test_act_order_identity_order_reduces_to_plain_q2_sweep():
    """With the identity order and the plain sweep's own rungs, the static sweep makes the same
    codes and residuals as the plain q2tp sweep."""
    n, rows = 96, 9
    H, W = _problem(n, rows, 1)
    d = np.sort(np.diag(H))[::-1] + np.arange(n)[::-1] * 1e-3
    H = H - np.diag(np.diag(H)) + np.diag(d.astype(np.float32))
    perm = oracle.act_order_perm(np.diag(H))
    assert np.array_equal(perm, np.arange(n))
    f = oracle.fold(H, 0.01)
    lost, tab = oracle.ladder_q2(W, f["dead"])
    plain = oracle.sweep_q2(W, f["U"], f["hdiag"], f["dead"], tab)
    Up = oracle.fold(oracle.permute_sym(H, perm).astype(np.float32), 0.01)["U"]
    ao = oracle.sweep_act_order(W, Up, f["dead"], perm, tab, lost, rung=plain["rung"], two_bit=True)
    assert np.array_equal(ao["code"], plain["code"])
    np.testing.assert_allclose(ao["E"], plain["E"], rtol=1e-12, atol=1e-18)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("n", [3, 6, 8])
def test_act_order_brute_force_obs_in_permuted_order(seed, n):
    """Column-sequential OBS with explicit re-inversion of the permuted damped Hessian, 2-bit
    levels at each row's fixed scale: the codes and residuals of the static q2 sweep."""
    H, W = _problem(n, 4, 70 + seed)
    perm = oracle.act_order_perm(np.diag(H))
    Hp = oracle.permute_sym(H, perm).astype(np.float32)
    f = oracle.fold(Hp, 0.01)
    dead = np.zeros(n, bool)
    lost, tab = oracle.ladder_q2(W, dead, gs=n)
    rung = np.random.default_rng(seed).integers(1, 32, size=(4, 1)).astype(np.uint8)
    ao = oracle.sweep_act_order(W, f["U"], dead, perm, tab, lost, gs=n, rung=rung, two_bit=True)
    hd = oracle.symmetric_from_upper(Hp) + f["damp"] * np.eye(n)
    for r in range(4):
        s = float(tab[r, rung[r, 0]])
        w = W[r, perm].astype(np.float64)
        for a in range(n):
            F = np.arange(a, n)
            hinv = np.linalg.inv(hd[np.ix_(F, F)])
            q = q2_level(np.float32(np.float32(w[a]) / np.float32(s)) + np.float32(1.5))
            assert ao["code"][r, perm[a]] == int(q)
            res = w[a] - (float(q) - 1.5) * s
            np.testing.assert_allclose(ao["E"][r, a], res / np.sqrt(hinv[0, 0]), rtol=1e-9, atol=1e-14)
            w[F] -= res / hinv[0, 0] * hinv[0, :]


def test_static_q2_rungs_are_the_exhaustive_best_of_the_original_tile():
    """Static q2 rungs: over rungs 1..31 the smallest max(H_ii, 0)-weighted f32 error of the
    dead-zeroed original tile, summed in column order, the lowest rung on a tie; rung 0 for an
    all-zero tile."""
    rng = np.random.default_rng(5)
    rows, n = 6, 96
    W = (rng.standard_normal((rows, n)) * np.exp(rng.standard_normal((rows, 1)))).astype(np.float32)
    W[2, 32:64] = 0.0
    dead = np.zeros(n, bool)
    dead[7] = True
    hdiag = np.exp(rng.standard_normal(n)).astype(np.float32)
    hdiag[11] = -3.0  # clipped to 0
    lost, tab = oracle.ladder_q2(W, dead)
    rung, scale = oracle.static_rungs_q2(W, dead, tab, hdiag)
    Wd = W.copy()
    Wd[:, dead] = 0.0
    hw = np.maximum(hdiag, 0.0).astype(np.float32)
    for r in range(rows):
        for g in range(n // 32):
            w = Wd[r, 32 * g:32 * g + 32]
            h = hw[32 * g:32 * g + 32]
            if not np.any(w != 0):
                assert rung[r, g] == 0 and scale[r, g] == 0.0
                continue
            best, best_e = 1, np.float32(np.inf)
            for c in range(1, 32):
                s = tab[r, c]
                if not s > 0:
                    continue
                err = np.float32(0.0)
                for t in range(32):
                    q = q2_level(np.float32(w[t] / s) + np.float32(1.5))
                    d = np.float32(w[t] - np.float32(np.float32(q - np.float32(1.5)) * s))
                    err = np.float32(err + np.float32(np.float32(h[t] * d) * d))
                if err < best_e:
                    best, best_e = c, err
            assert rung[r, g] == best and scale[r, g] == tab[r, best]


def test_act_order_residuals_reproduce_the_error():
    n, rows = 128, 10
    H, W = _problem(n, rows, 4)
    perm = oracle.act_order_perm(np.diag(H))
    Hp = oracle.permute_sym(H, perm).astype(np.float32)
    f = oracle.fold(Hp, 0.01)
    dead = np.zeros(n, bool)
    lost, tab = oracle.ladder_q2(W, dead)
    ao = oracle.sweep_act_order(W, f["U"], dead, perm, tab, lost, two_bit=True,
                                hdiag=np.diag(H).astype(np.float32))
    dW = W.astype(np.float64) - oracle.dequant_q2(ao["code"], ao["scale"])
    dWp = dW[:, perm]
    np.testing.assert_allclose(dWp, ao["E"] @ f["U"], rtol=1e-10, atol=1e-14)


# --- output debias of 2-bit codes --------------------------------------------------------------

def test_q2_debias_closed_form_exact_scaling():
    """Codes and scales that decode to exactly k W give the slope k; lo moves by -log2 k, and
    the new scales are the q2 ladder's TAB[rung] = 2^(lo_new + (rung - 1) step)."""
    rng = np.random.default_rng(12)
    rows, n = 5, 64
    A = rng.standard_normal((n, 2 * n))
    H = (A @ A.T).astype(np.float32)
    for k, shift in [(0.5, 1.0), (2.0, -1.0), (0.25, 2.0)]:
        code = rng.integers(0, 4, size=(rows, n)).astype(np.uint8)
        s_true = (2.0 ** rng.integers(-8, -4, size=(rows, n // 32))).astype(np.float32)
        W = ((code.astype(np.float64) - 1.5) * np.repeat(s_true, 32, axis=1)).astype(np.float32)
        scale = (s_true * np.float32(k)).astype(np.float32)
        lost = np.stack([np.full(rows, -6.0, np.float32), np.full(rows, 0.125, np.float32)], 1)
        rung = rng.integers(1, 32, size=(rows, n // 32)).astype(np.uint8)
        r = oracle.debias(W, H, np.zeros(n, bool), code, rung, lost, scale, two_bit=True)
        assert np.allclose(r["b"], k, rtol=1e-12)
        assert np.array_equal(r["lo"], lost[:, 0] + shift)
        assert np.all(r["tab"][:, 0] == 0.0)
        want = np.float32(2.0 ** ((lost[:, 0] + shift)[:, None] + (rung.astype(np.float64) - 1) * 0.125))
        assert np.array_equal(r["scale"], want)


def test_q2_debias_brute_force_double_sum():
    rng = np.random.default_rng(13)
    rows, n = 3, 32
    W = rng.standard_normal((rows, n)).astype(np.float32) * 0.1
    code = rng.integers(0, 4, size=(rows, n)).astype(np.uint8)
    scale = rng.uniform(0.01, 0.05, size=(rows, 1)).astype(np.float32)
    A = rng.standard_normal((n, 2 * n))
    H = (A @ A.T).astype(np.float32)
    dead = np.zeros(n, bool)
    dead[[4, 9]] = True
    lost = np.stack([np.full(rows, -5.0, np.float32), np.full(rows, 0.25, np.float32)], 1)
    r = oracle.debias(W, H, dead, code, np.ones((rows, 1), np.uint8), lost, scale, two_bit=True)
    for i in range(rows):
        num = den = 0.0
        for a in range(n):
            for b in range(n):
                if dead[a] or dead[b]:
                    continue
                h = float(H[min(a, b), max(a, b)])
                wh = (float(code[i, a]) - 1.5) * float(scale[i, 0])
                num += wh * h * float(W[i, b])
                den += float(W[i, a]) * h * float(W[i, b])
        np.testing.assert_allclose(r["num"][i], num, rtol=1e-10)
        np.testing.assert_allclose(r["den"][i], den, rtol=1e-10)
