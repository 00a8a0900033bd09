"""GPU parity on seeded random shapes (the fold and sweep; then the q2tp sweep, act order and
the output debias): n a random multiple of 32 up to 1248, 1-399 rows, Hessians
from 0.6-3 n tokens (so some are rank-deficient and take the retry path), random dead
channels, heavy-tailed channel scales, λ in {0, 1e-4, 1e-2, 0.1}, and now and then an all-zero
row of W.  Every case is held to the fold and sweep bars of the other parity tests."""
import numpy as np
import pytest
import torch

from parity import assert_sweep_bar, check_fold, check_sweep_isolated, say

pytestmark = pytest.mark.gpu


def _case(rng):
    n = int(rng.integers(1, 40)) * 32
    rows = int(rng.integers(1, 400))
    t = int(n * rng.uniform(0.6, 3.0)) + 1
    X = rng.standard_normal((n, t)) * np.exp(rng.uniform(0, 1.5) * rng.standard_normal(n))[:, None]
    nd = int(rng.integers(0, max(1, n // 20)))
    if nd:
        X[rng.choice(n, size=nd, replace=False), :] = 0.0
    H = (X @ X.T).astype(np.float32)
    lam = float(rng.choice([0.0, 1e-4, 1e-2, 0.1]))
    W = (rng.standard_normal((rows, n)) * rng.uniform(0.005, 0.05)).astype(np.float32)
    if rng.random() < 0.2:
        W[rng.integers(0, rows), :] = 0.0
    return H, W, lam, t, nd


@pytest.mark.parametrize("seed", [101, 202, 303])
def test_random_shapes(gpu, seed):
    rng = np.random.default_rng(seed)
    for i in range(12):
        H, W, lam, t, nd = _case(rng)
        say(f"seed {seed} case {i}: n={H.shape[0]} rows={W.shape[0]} t={t} dead={nd} lam={lam}")
        (U, hdiag, dead, rep), orc, err = check_fold(gpu, torch.as_tensor(H).cuda(), lam, H_np=H)
        st, _ = check_sweep_isolated(gpu, torch.as_tensor(W).cuda(), U, hdiag, dead)
        assert_sweep_bar(st)


@pytest.mark.parametrize("seed", [404, 505])
def test_random_shapes_next_rows(gpu, seed):
    """The same generator for the q2tp sweep, act order (4- and 2-bit) and the output debias
    (4- and 2-bit), each against its own checker (the bars of its parity tests)."""
    from test_gpu_act_order import check_order, check_sweep, check_sweep_q2, run_gpu
    from test_gpu_debias import check as check_debias
    from test_gpu_q2 import check_q2
    rng = np.random.default_rng(seed)
    for i in range(6):
        H, W, lam, t, nd = _case(rng)
        say(f"seed {seed} case {i}: n={H.shape[0]} rows={W.shape[0]} t={t} dead={nd} lam={lam}")
        Hd, Wd = torch.as_tensor(H).cuda(), torch.as_tensor(W).cuda()
        (U, hdiag, dead, rep), _, _ = check_fold(gpu, Hd, lam, H_np=H)
        check_q2(gpu, Wd, U, hdiag, dead)
        perm, dead_a, Hp = run_gpu(gpu, Hd, Wd, lam)
        p_o = check_order(perm, dead_a, Hp, H)
        (Up, hdiag_p, _, _), _, _ = check_fold(gpu, Hp, lam)
        check_sweep(gpu, Wd, Up, dead_a, perm, p_o)
        check_sweep_q2(gpu, Wd, Up, hdiag_p, dead_a, perm, p_o)
        check_debias(gpu, Hd, Wd, lam, label=f"random n={H.shape[0]}")
        check_debias(gpu, Hd, Wd, lam, label=f"random q2 n={H.shape[0]}", two_bit=True)


def test_near_tie_rungs_decided_like_the_oracle(gpu):
    """Regression: the 215th case of seed 7 (n = 32, 211 rows) has rows whose candidate rungs'
    f32 errors lie within an ulp of each other.  The rung decisions are taken in f32 with every
    product and sum rounded separately; when the build fused them into multiply-adds, the
    act-order static rungs differed from the oracle's here.  They must now agree exactly."""
    from test_gpu_act_order import check_order, check_sweep, run_gpu
    rng = np.random.default_rng(7)
    for _ in range(215):
        H, W, lam, t, nd = _case(rng)
    assert H.shape == (32, 32) and W.shape == (211, 32)
    Hd, Wd = torch.as_tensor(H).cuda(), torch.as_tensor(W).cuda()
    (U, hdiag, dead, rep), _, _ = check_fold(gpu, Hd, lam, H_np=H)
    st, _ = check_sweep_isolated(gpu, Wd, U, hdiag, dead)
    assert_sweep_bar(st)
    assert st["rung_hard"] == 0 and st["rung_ties"] == 0, st
    perm, dead_a, Hp = run_gpu(gpu, Hd, Wd, lam)
    p_o = check_order(perm, dead_a, Hp, H)
    (Up, _, _, _), _, _ = check_fold(gpu, Hp, lam)
    check_sweep(gpu, Wd, Up, dead_a, perm, p_o)


def test_random_larger_shapes(gpu):
    """Three seeded cases at n = 1280-4096 (several 512-column panels; H formed on the GPU), 64
    sampled rows each, with and without the residual output."""
    rng = np.random.default_rng(11)
    for i in range(3):
        n = int(rng.integers(40, 129)) * 32
        rows = int(rng.integers(64, 600))
        t = int(n * rng.uniform(0.8, 2.5)) + 1
        X = rng.standard_normal((n, t)).astype(np.float32)
        X *= np.exp(rng.uniform(0, 1.5) * rng.standard_normal(n)).astype(np.float32)[:, None]
        nd = int(rng.integers(0, max(1, n // 50)))
        if nd:
            X[rng.choice(n, size=nd, replace=False), :] = 0.0
        Xd = torch.as_tensor(X).cuda()
        Hd = (Xd @ Xd.T).contiguous()
        lam = float(rng.choice([0.0, 1e-4, 1e-2]))
        W = (rng.standard_normal((rows, n)) * rng.uniform(0.005, 0.05)).astype(np.float32)
        say(f"larger case {i}: n={n} rows={rows} t={t} dead={nd} lam={lam}")
        (U, hdiag, dead, rep), _, _ = check_fold(gpu, Hd, lam, H_np=Hd.cpu().numpy())
        sel = np.sort(rng.choice(rows, size=64, replace=False))
        st, _ = check_sweep_isolated(gpu, torch.as_tensor(W).cuda(), U, hdiag, dead, rows_sel=sel,
                                     want_E=(i % 2 == 0))
        assert_sweep_bar(st)
