"""Pins of the oracle's Hessian accumulation (oracle.gram) against what the pages and the
mathematics fix: brute-force sums on tiny inputs (a transposed operand or a dropped term fails
them), symmetry, the trace identity tr(X^T X) = ||X||_F^2, positive semidefiniteness, dead
(all-zero) channels giving zero rows and columns, and additivity over token batches (the
calibration loop adds one window at a time).  The fixture is the activation pattern of the
pages' device-versus-host test ("cortiq-cli 0.8.45 src/gptq.rs",
device_fold_and_sweep_match_host), rebuilt from its formulas."""
import numpy as np

import oracle
import workloads


def brute(X):
    t, n = X.shape
    H = [[0.0] * n for _ in range(n)]
    for r in range(t):
        for i in range(n):
            for j in range(n):
                H[i][j] += float(X[r][i]) * float(X[r][j])
    return np.array(H)


def test_brute_force_tiny():
    rng = np.random.default_rng(7)
    for t, n in [(1, 1), (3, 2), (5, 7), (11, 4)]:
        X = rng.standard_normal((t, n)).astype(np.float32)
        H, mag = oracle.gram(X)
        assert np.allclose(H, brute(X), rtol=0, atol=1e-12)
        assert np.allclose(mag, brute(np.abs(X)), rtol=0, atol=1e-12)


def test_rectangular_orientation():
    """X [t, n] with t != n: H is n x n, indexed by channels, not tokens."""
    X = np.zeros((3, 5), np.float32)
    X[0, 1] = 2.0
    X[2, 4] = 3.0
    X[1, 1] = 1.0
    H, _ = oracle.gram(X)
    assert H.shape == (5, 5)
    expect = np.zeros((5, 5))
    expect[1, 1] = 5.0
    expect[4, 4] = 9.0
    assert np.array_equal(H, expect)


def test_invariants_on_pages_fixture():
    X = workloads.pages_fixture_activations()
    H, mag = oracle.gram(X)
    n = X.shape[1]
    assert np.array_equal(H, H.T)
    assert abs(np.trace(H) - float(np.sum(X.astype(np.float64) ** 2))) <= 1e-9 * np.trace(H)
    assert np.linalg.eigvalsh(H).min() >= -1e-9 * np.trace(H)
    for c in (17, 90):  # the fixture's dead channels
        assert not H[c].any() and not H[:, c].any()
    assert np.all(mag >= np.abs(H) - 1e-9 * np.abs(H).max())
    assert n == 160


def test_additive_over_batches():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((97, 12)).astype(np.float32)
    H1, _ = oracle.gram(X[:40])
    H2, _ = oracle.gram(X[40:], H0=H1)
    Hall, _ = oracle.gram(X)
    assert np.allclose(H2, Hall, rtol=1e-13, atol=1e-12)
