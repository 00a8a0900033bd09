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
