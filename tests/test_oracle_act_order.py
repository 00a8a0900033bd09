"""Pins of the oracle's act-order GPTQ ("cortiq-cli 0.8.45 src/gptq.rs": act_order_perm,
permute_sym, gptq_quantize_q4tp_act_order) against what the pages and the mathematics fix:
the channel order (descending H_ii in the f32 total order, ties by index), the reduction to the
plain sweep when the order is the identity and the rungs are the same, column-sequential OBS
with explicit re-inversion on the permuted Hessian (brute force on tiny inputs), the static
rung rule against an exhaustive scan of its window, and the identity dW = E U in elimination
order."""
import numpy as np
import pytest

import oracle


def test_perm_order_ties_and_total_order():
    assert list(oracle.act_order_perm([1.0, 3.0, 2.0])) == [1, 2, 0]
    assert list(oracle.act_order_perm([2.0, 2.0, 1.0, 2.0])) == [0, 1, 3, 2]
    h = np.array([0.0, -0.0, np.inf, 5.0, np.nan, -1.0], dtype=np.float32)
    # total order descending: NaN (positive) > inf > 5 > +0 > -0 > -1
    assert list(oracle.act_order_perm(h)) == [4, 2, 3, 0, 1, 5]


def _spread_ladder(W, st=1.0 / 16):
    amax = np.abs(W).max(axis=1).astype(np.float64)
    lo = np.array([oracle.f16_round(np.log2(a / 7.0) - 1.0) for a in amax])
    lost = np.stack([lo, np.full(W.shape[0], st)], 1).astype(np.float32)
    tab = np.exp2(lo[:, None] + np.arange(32)[None, :] * st).astype(np.float32)
    return lost, tab


def _problem(n, rows, seed, gs):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, 2 * n + 5)) * np.exp(rng.standard_normal(n))[:, None]
    H = (X @ X.T).astype(np.float32)
    W = (rng.standard_normal((rows, n)) * 0.05).astype(np.float32)
    lost, tab = _spread_ladder(W)
    return H, W, lost, tab


def test_identity_order_reduces_to_plain_sweep():
    n, rows = 64, 9
    H, W, lost, tab = _problem(n, rows, 1, 32)
    # Make the diagonal strictly decreasing so that the order is the identity.
    d = np.sort(np.diag(H))[::-1] + np.arange(n)[::-1] * 1e-3
    H = H - np.diag(np.diag(H)) + np.diag(d.astype(np.float32))
    perm = oracle.act_order_perm(np.diag(H))
    assert np.array_equal(perm, np.arange(n))
    f = oracle.fold(H, 0.01)
    plain = oracle.sweep(W, f["U"], f["hdiag"], f["dead"], tab, lost)
    ao = oracle.sweep_act_order(W, oracle.fold(oracle.permute_sym(H, perm).astype(np.float32), 0.01)["U"],
                                f["dead"], perm, tab, lost, rung=plain["rung"])
    assert np.array_equal(ao["code"], plain["code"])
    np.testing.assert_allclose(ao["E"], plain["E"], rtol=1e-12, atol=1e-18)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
@pytest.mark.parametrize("n", [2, 5, 8])
def test_brute_force_obs_in_permuted_order(seed, n):
    H, W, lost, tab = _problem(n, 4, 50 + seed, n)
    perm = oracle.act_order_perm(np.diag(H))
    Hp = oracle.permute_sym(H, perm).astype(np.float32)
    f = oracle.fold(Hp, 0.01)
    dead = np.zeros(n, bool)
    rung = np.random.default_rng(seed).integers(8, 24, size=(4, 1)).astype(np.uint8)
    ao = oracle.sweep_act_order(W, f["U"], dead, perm, tab, lost, gs=n, rung=rung)
    hd = oracle.symmetric_from_upper(Hp) + f["damp"] * np.eye(n)
    for r in range(4):
        s = float(tab[r, rung[r, 0]])
        w = W[r, perm].astype(np.float64)
        for a in range(n):
            F = np.arange(a, n)
            hinv = np.linalg.inv(hd[np.ix_(F, F)])
            q = np.float32(np.clip(np.rint(np.float32(w[a]) / np.float32(s)), -8, 7))
            assert ao["code"][r, perm[a]] == int(q) + 8
            res = w[a] - float(q) * s
            np.testing.assert_allclose(ao["E"][r, a], res / np.sqrt(hinv[0, 0]), rtol=1e-9, atol=1e-14)
            w[F] -= res / hinv[0, 0] * hinv[0, :]


def test_static_rungs_scan_their_window():
    rng = np.random.default_rng(9)
    rows, n = 7, 96
    W = (rng.standard_normal((rows, n)) * np.exp(rng.standard_normal((rows, 1)))).astype(np.float32)
    dead = np.zeros(n, bool)
    dead[5] = True
    lost, tab = _spread_ladder(W)
    rung, scale = oracle.static_rungs(W, dead, tab, lost)
    Wd = W.copy()
    Wd[:, dead] = 0.0
    for r in range(rows):
        for g in range(n // 32):
            w = Wd[r, 32 * g:32 * g + 32]
            amax = float(np.abs(w).max())
            v = (np.log2(amax / 7.0) - float(lost[r, 0])) / float(lost[r, 1])
            nom = int(min(max(np.floor(v + 0.5) if v >= 0 else -np.floor(-v + 0.5), 0), 31))
            best, best_e = nom, np.inf
            for c in range(max(nom - 2, 0), min(nom + 1, 31) + 1):
                s = tab[r, c]
                q = np.clip(np.rint(w / s), -8, 7).astype(np.float32)
                err = np.float32(0.0)
                for t in range(32):
                    d = np.float32(w[t] - np.float32(q[t] * s))
                    err = np.float32(err + np.float32(d * d))
                if err < best_e:
                    best, best_e = c, err
            assert rung[r, g] == best and scale[r, g] == tab[r, best]


def test_residuals_reproduce_the_error_in_elimination_order():
    n, rows = 96, 12
    H, W, lost, tab = _problem(n, rows, 4, 32)
    perm = oracle.act_order_perm(np.diag(H))
    Hp = oracle.permute_sym(H, perm).astype(np.float32)
    f = oracle.fold(Hp, 0.01)
    dead = np.zeros(n, bool)
    ao = oracle.sweep_act_order(W, f["U"], dead, perm, tab, lost)
    dW = W.astype(np.float64) - oracle.dequant(ao["code"], ao["scale"])
    dWp = dW[:, perm]
    np.testing.assert_allclose(dWp, ao["E"] @ f["U"], rtol=1e-10, atol=1e-14)
    hd = oracle.symmetric_from_upper(Hp) + f["damp"] * np.eye(n)
    t = np.einsum("ij,jk,ik->", dWp, hd, dWp)
    assert abs(t - np.sum(ao["E"] ** 2)) <= 1e-10 * t
