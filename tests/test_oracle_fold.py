"""Pins of the oracle's fold against facts fixed outside the oracle itself.

The fold computes U, the upper Cholesky factor of H_d^-1 with H_d = H' + lambda*base*I
("cortiq-cli 0.8.45 src/gptq.rs", gptq_fold_operator_par; "cortiq-engine 0.8.41
src/gpu_wgpu/gptq_dev.rs", module documentation, steps 1-4).  Each test below checks it against
something independent: closed forms, LAPACK, the inverse identity, the uniqueness of the factor
(two other routes), hand-derived retry cases, or the block structure of the factor.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden", "fold_closed_forms.json")


def _spd(n, seed, cond_spread=2.0):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, 3 * n))
    X *= np.exp(cond_spread * rng.standard_normal(n))[:, None]
    return (X @ X.T).astype(np.float32)


def _hd(H, res):
    """H_d from the f32 input the way the definition states it (upper triangle, dead rows)."""
    Hu = np.triu(H.astype(np.float64))
    h = Hu + np.triu(Hu, 1).T
    dead = res["dead"]
    h[dead, :] = 0.0
    h[:, dead] = 0.0
    h[dead, dead] = 1.0
    return h + res["damp"] * np.eye(len(h))


def test_identity_hessian_closed_form():
    for n, lam in [(1, 0.0), (8, 0.01), (40, 0.5)]:
        r = oracle.fold(np.eye(n, dtype=np.float32), lam)
        assert r["status"] == oracle.OK and r["attempts"] == 1
        np.testing.assert_allclose(r["U"], np.eye(n) / np.sqrt(1.0 + lam), rtol=2e-16, atol=0)


def test_diagonal_hessian_closed_form():
    d = np.array([3.0, 0.25, 7.5, 1e4, 2.0], dtype=np.float32)
    lam = 0.01
    r = oracle.fold(np.diag(d), lam)
    base = d.astype(np.float64).mean()
    np.testing.assert_allclose(r["base"], base, rtol=1e-15)
    np.testing.assert_allclose(r["U"], np.diag(1.0 / np.sqrt(d + lam * base)), rtol=1e-15)


def test_two_by_two_hand_derived():
    g = json.load(open(GOLD))["two_by_two"]
    r = oracle.fold(np.array(g["H"], dtype=np.float32), g["lambda"])
    assert r["status"] == oracle.OK
    np.testing.assert_allclose(r["U"], np.array(g["U"]), rtol=1e-15, atol=1e-16)


@pytest.mark.parametrize("case", json.load(open(GOLD))["retry_cases"])
def test_retry_schedule_hand_cases(case):
    r = oracle.fold(np.array(case["H"], dtype=np.float32), case["lambda"])
    np.testing.assert_allclose(r["lam"], case["lambda_used"], rtol=1e-12)
    assert r["attempts"] == case["attempts"]
    if case["status"] == "degenerate":
        assert r["status"] == oracle.DEGENERATE
        np.testing.assert_array_equal(r["U"], np.eye(2))
    else:
        assert r["status"] == oracle.OK
        h = np.array(case["H"], dtype=np.float64) + r["damp"] * np.eye(2)
        np.testing.assert_allclose(r["U"].T @ r["U"] @ h, np.eye(2), atol=1e-8)


def test_no_retry_reports_failure():
    r = oracle.fold(np.array([[1, 1], [1, 1]], dtype=np.float32), 0.0, retry=False)
    assert r["status"] == oracle.FAILED


def test_dead_channels_closed_form():
    H = _spd(12, 3)
    for j in (2, 7):
        H[j, :] = H[:, j] = 0.0
    H[9, 9] = -1.0            # a negative diagonal is dead as well
    H[4, 4] = np.nan          # NaN is not > 0: dead
    lam = 0.02
    r = oracle.fold(H, lam)
    dead = r["dead"]
    assert list(np.nonzero(dead)[0]) == [2, 4, 7, 9]
    # The mean counts a dead diagonal as 1.
    diag = np.where(dead, 1.0, np.diag(H).astype(np.float64))
    np.testing.assert_allclose(r["base"], diag.mean(), rtol=1e-15)
    U = r["U"]
    for j in np.nonzero(dead)[0]:
        off = np.delete(np.arange(12), j)
        assert np.all(U[j, off] == 0.0) and np.all(U[off, j] == 0.0)
        np.testing.assert_allclose(U[j, j], 1.0 / np.sqrt(1.0 + r["damp"]), rtol=1e-15)


def test_matches_lapack_cholesky_of_inverse():
    for n, seed in [(17, 1), (96, 2), (300, 3)]:
        H = _spd(n, seed)
        r = oracle.fold(H, 0.01)
        hd = _hd(H, r)
        ref = np.linalg.cholesky(np.linalg.inv(hd)).T
        err = np.linalg.norm(r["U"] - ref) / np.linalg.norm(ref)
        assert err < 1e-10, err


def test_first_row_is_scaled_inverse_row():
    H = _spd(64, 5)
    r = oracle.fold(H, 0.01)
    hinv = np.linalg.inv(_hd(H, r))
    np.testing.assert_allclose(r["U"][0], hinv[0] / np.sqrt(hinv[0, 0]), rtol=1e-9, atol=1e-14)


def _inverse_identity_residual(H, r):
    """max |D (U^T U H_d - I) D^-1|, the equilibrated residual of U^T U H_d = I."""
    hd = _hd(H, r)
    d = np.sqrt(np.diag(hd))
    res = (r["U"].T @ r["U"] @ hd - np.eye(len(hd))) * d[:, None] / d[None, :]
    return float(np.abs(res).max())


def test_inverse_identity_on_tiny_workload():
    H, W, lam = workloads.make("tiny")
    H = H.numpy()
    r = oracle.fold(H, lam)
    assert r["status"] == oracle.OK and r["attempts"] == 1
    res = _inverse_identity_residual(H, r)
    assert res < 1e-10, res


@pytest.mark.slow
def test_inverse_identity_on_attention_workload():
    """U^T U H_d = I to 1e-10 (equilibrated) at the attention-projection size, n = 4096 with
    its lognormal channels and dead channels."""
    H, W, lam = workloads.make("attn")
    H = H.numpy()
    r = oracle.fold(H, lam)
    assert r["status"] == oracle.OK and r["attempts"] == 1 and r["dead"].sum() == 20
    res = _inverse_identity_residual(H, r)
    assert res < 1e-10, res


def test_two_routes_agree():
    """The factor is unique, so the reversed route and the reversed equilibrated route (other
    rounding) give the same U up to rounding."""
    for H in (_spd(77, 7), workloads.make("tiny")[0].numpy(), workloads.fixture()[0].numpy()):
        ref = oracle.fold(H, 0.01, route=0)
        r = oracle.fold(H, 0.01, route=1)
        assert r["status"] == oracle.OK and r["lam"] == ref["lam"]
        err = np.linalg.norm(r["U"] - ref["U"]) / np.linalg.norm(ref["U"])
        assert err < 1e-12, err


def test_every_row_is_the_obs_row_of_its_trailing_hessian():
    """Row j of U is the first row of the inverse of H_d's trailing principal block F = {j..n-1},
    divided by the square root of its first entry (the pages' OBS reading of the operator: the
    feedback of column j reaches only the columns not yet quantized).  Each row is checked
    against its own LAPACK inverse, so a wrong index anywhere in the factor or its inverse
    fails it; the entries left of the diagonal are exactly 0."""
    for n, seed, lam in [(9, 21, 0.0), (40, 22, 0.01), (73, 23, 1e-4)]:
        H = _spd(n, seed)
        H[5, :] = H[:, 5] = 0.0
        r = oracle.fold(H, lam)
        assert r["status"] == oracle.OK
        hd = _hd(H, r)
        for j in range(n):
            g = np.linalg.inv(hd[j:, j:])[0]
            np.testing.assert_allclose(r["U"][j, j:], g / np.sqrt(g[0]), rtol=1e-9, atol=1e-12)
            assert np.all(r["U"][j, :j] == 0.0)


def test_reads_upper_triangle_only():
    H = _spd(50, 9)
    G = H.copy()
    il = np.tril_indices(50, -1)
    G[il] = np.random.default_rng(0).standard_normal(len(il[0])).astype(np.float32) * 1e6
    a, b = oracle.fold(H, 0.01), oracle.fold(G, 0.01)
    np.testing.assert_array_equal(a["U"], b["U"])


def test_nan_off_diagonal_is_degenerate():
    H = _spd(10, 4)
    H[2, 6] = np.nan
    r = oracle.fold(H, 0.01)
    assert r["status"] == oracle.DEGENERATE
    np.testing.assert_array_equal(r["U"], np.eye(10))


def test_thread_count_does_not_change_bits():
    H = _spd(211, 11)
    a = oracle.fold(H, 0.01, nt=1)
    b = oracle.fold(H, 0.01, nt=4)
    np.testing.assert_array_equal(a["U"], b["U"])


def test_trailing_block_is_fold_of_trailing_hessian():
    """H_d = R R^T with R = U^-1 upper, so H_d[m:, m:] = R[m:, m:] R[m:, m:]^T and the
    trailing block of U is the fold of the trailing block of H_d at the same damping.  The
    GPU parity tests at full size rely on this to check sampled blocks."""
    H = _spd(120, 12)
    r = oracle.fold(H, 0.01)
    m = 70
    sub = H[m:, m:].copy()
    base_sub = np.diag(sub).astype(np.float64).mean()
    rs = oracle.fold(sub, r["damp"] / base_sub, retry=False)
    assert rs["status"] == oracle.OK
    np.testing.assert_allclose(rs["U"], r["U"][m:, m:], rtol=1e-10, atol=1e-13)
