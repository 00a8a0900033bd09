"""Pins of the oracle's output debias (oracle.debias) against what the pages and the mathematics
fix.  The pages define the slope b = (W^ H W^T)_rr / (W H W^T)_rr and its removal through lo
("cortiq-cli 0.8.45 src/gptq.rs", q4tp_debias_hessian); pinned here by a closed form (codes that
decode to exactly k W give b = k, and lo moves by -log2 k), brute-force double sums on tiny
inputs, H = I (plain dot products), invariance to scaling H, the guards (zero or negative
slope keeps lo), and the fixed point: after the debias the slope recomputed with the new
scales is 1 within half an f16 step of lo."""
import numpy as np

import oracle


def make_exact(rows, n, rng, k):
    """W on a quantization grid, codes and scales decoding to exactly k * W."""
    gs = 32
    code = rng.integers(0, 16, size=(rows, n)).astype(np.uint8)
    s_true = (2.0 ** rng.integers(-8, -4, size=(rows, n // gs))).astype(np.float32)
    W = ((code.astype(np.float64) - 8.0) * np.repeat(s_true, gs, axis=1)).astype(np.float32)
    scale = (s_true * np.float32(k)).astype(np.float32)
    lost = np.stack([np.full(rows, -6.0, np.float32), np.full(rows, 0.125, np.float32)], 1)
    rung = np.zeros((rows, n // gs), np.uint8)
    return W, code, scale, lost, rung


def spd(n, rng):
    A = rng.standard_normal((n, 2 * n))
    return (A @ A.T).astype(np.float32)


def test_closed_form_exact_scaling():
    rng = np.random.default_rng(1)
    for k, shift in [(0.5, 1.0), (2.0, -1.0), (0.25, 2.0)]:
        W, code, scale, lost, rung = make_exact(5, 64, rng, k)
        H = spd(64, rng)
        r = oracle.debias(W, H, np.zeros(64, bool), code, rung, lost, scale)
        assert np.allclose(r["b"], k, rtol=1e-12)
        assert np.array_equal(r["lo"], lost[:, 0] + shift)
        # New scales: 2^(lo_new + rung * step) with rung 0.
        assert np.array_equal(r["scale"], np.float32(2.0 ** (lost[:, 0] + shift))[:, None].repeat(2, 1))


def test_brute_force_double_sum():
    rng = np.random.default_rng(2)
    rows, n = 3, 32
    W = rng.standard_normal((rows, n)).astype(np.float32) * 0.1
    code = rng.integers(0, 16, size=(rows, n)).astype(np.uint8)
    scale = rng.uniform(0.01, 0.03, size=(rows, 1)).astype(np.float32)
    H = spd(n, rng)
    dead = np.zeros(n, bool)
    dead[[3, 11]] = True
    lost = np.array([[-5.0, 0.1]] * rows, np.float32)
    r = oracle.debias(W, H, dead, code, np.zeros((rows, 1), np.uint8), lost, scale)
    for k in range(rows):
        num = den = 0.0
        for i in range(n):
            for j in range(n):
                if dead[i] or dead[j]:
                    continue
                hij = float(H[min(i, j), max(i, j)])
                wi, wj = float(W[k, i]), float(W[k, j])
                qi = (float(code[k, i]) - 8.0) * float(scale[k, 0])
                num += qi * hij * wj
                den += wi * hij * wj
        assert abs(r["num"][k] - num) <= 1e-9 * abs(num) + 1e-15
        assert abs(r["den"][k] - den) <= 1e-9 * abs(den) + 1e-15


def test_identity_hessian_and_scale_invariance():
    rng = np.random.default_rng(3)
    rows, n = 4, 64
    W = rng.standard_normal((rows, n)).astype(np.float32)
    code = rng.integers(0, 16, size=(rows, n)).astype(np.uint8)
    scale = rng.uniform(0.1, 0.3, size=(rows, 2)).astype(np.float32)
    lost = np.array([[-3.0, 0.05]] * rows, np.float32)
    rung = np.zeros((rows, 2), np.uint8)
    dead = np.zeros(n, bool)
    r = oracle.debias(W, np.eye(n, dtype=np.float32), dead, code, rung, lost, scale)
    What = oracle.dequant(code, scale)
    assert np.allclose(r["b"], np.sum(What * W, 1) / np.sum(W.astype(np.float64) ** 2, 1), rtol=1e-12)
    H = spd(n, rng)
    r1 = oracle.debias(W, H, dead, code, rung, lost, scale)
    r2 = oracle.debias(W, np.float32(8.0) * H, dead, code, rung, lost, scale)
    assert np.allclose(r1["b"], r2["b"], rtol=1e-12)


def test_guards_keep_lo():
    rng = np.random.default_rng(4)
    W, code, scale, lost, rung = make_exact(3, 32, rng, 1.0)
    H = spd(32, rng)
    neg = (scale * np.float32(-1.0)).astype(np.float32)   # W^ = -W: slope -1
    r = oracle.debias(W, H, np.zeros(32, bool), code, rung, lost, neg)
    assert np.array_equal(r["lo"], lost[:, 0].astype(np.float64))
    Z = np.zeros_like(W)                                  # all-zero row: den = 0
    r = oracle.debias(Z, H, np.zeros(32, bool), code, rung, lost, scale)
    assert np.array_equal(r["lo"], lost[:, 0].astype(np.float64))


def test_fixed_point_after_debias():
    rng = np.random.default_rng(5)
    rows, n = 6, 96
    W = (rng.standard_normal((rows, n)) * 0.02).astype(np.float32)
    lost = np.array([[-9.0, 0.06]] * rows, np.float32)
    rung = rng.integers(0, 32, size=(rows, n // 32)).astype(np.uint8)
    tab = np.float32(np.exp2(lost[:, :1].astype(np.float64) + np.arange(32) * 0.06))
    scale = np.take_along_axis(tab, rung.astype(np.int64), 1)
    code = np.clip(np.rint(W / np.repeat(scale, 32, 1)), -8, 7).astype(np.int64) + 8
    H = spd(n, rng)
    r = oracle.debias(W, H, np.zeros(n, bool), code.astype(np.uint8), rung, lost, scale)
    lost2 = lost.copy()
    lost2[:, 0] = r["lo"]
    r2 = oracle.debias(W, H, np.zeros(n, bool), code.astype(np.uint8), rung, lost2, r["scale"])
    for k in range(rows):
        assert abs(np.log2(r2["b"][k])) <= 0.5 * oracle.f16_ulp(r["lo"][k]) + 1e-9
