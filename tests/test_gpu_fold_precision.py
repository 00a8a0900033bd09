"""The fold's arithmetic (include/gptq.h, GPTQ_FOLD_*): the f32 factor is accurate to about
u32 / (smallest pivot of the equilibrated matrix), so the default "auto" precision repeats any
damping value whose f32 pivots reach the floor 1e-2 in f64, with the f64 host's pivot rule.
These tests hold the fold to the parity bars on the inputs where the f32 factor cannot meet
them: rank-deficient Hessians (fewer tokens than channels) at small damping."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import (FOLD_TOL, OUT_ERR_TOL, assert_sweep_bar, check_fold, check_sweep_isolated,
                    fold_rel_err, hd_diag, output_error, say)

pytestmark = pytest.mark.gpu

PIVOT_FLOOR = 1e-2


def _dev(x):
    return torch.as_tensor(np.ascontiguousarray(x)).cuda()


def _rank_deficient_case(rng, heavy):
    """n <= 1024 channels from 0.3-1 n tokens, damping 1e-6 .. 1e-4; ``heavy`` adds lognormal
    channel energies and dead channels."""
    n = int(rng.integers(2, 33)) * 32
    rows = int(rng.integers(16, 161))
    t = int(n * rng.uniform(0.3, 1.0)) + 1
    X = rng.standard_normal((n, t))
    nd = 0
    if heavy:
        X *= np.exp(rng.uniform(0, 2.0) * rng.standard_normal(n))[:, None]
        nd = int(rng.integers(0, max(1, n // 20)))
        if nd:
            X[rng.choice(n, size=nd, replace=False), :] = 0.0
    H = (X @ X.T).astype(np.float32)
    lam = float(rng.choice([1e-6, 1e-5, 1e-4]))
    W = (rng.standard_normal((rows, n)) * 0.02).astype(np.float32)
    return H, W, lam, t, nd


@pytest.mark.parametrize("seed", [61, 62])
def test_rank_deficient_small_damping(gpu, seed):
    """Seeded random Hessians of the class: the damping equals the f64 oracle's from the same
    start, U meets the fold bar there, the sweep meets its bar on the GPU's U, and the
    layer-output error is within 1% (two-sided) of the free-running oracle's."""
    rng = np.random.default_rng(seed)
    n_f64 = 0
    for i in range(12):
        H, W, lam, t, nd = _rank_deficient_case(rng, heavy=(i % 2 == 1))
        n, rows = H.shape[0], W.shape[0]
        say(f"seed {seed} case {i}: n={n} rows={rows} t={t} dead={nd} lam={lam}")
        (U, hdiag, dead, rep), orc, err = check_fold(gpu, _dev(H), lam, H_np=H)
        free = oracle.fold(H, lam)
        assert rep["lambda_used"] == free["lam"], (rep, free["lam"])
        assert err <= FOLD_TOL
        n_f64 += rep["precision"] == 64
        Wd = _dev(W)
        st, (nib, rung, scale, E, lost, tab) = check_sweep_isolated(gpu, Wd, U, hdiag, dead)
        assert_sweep_bar(st)
        lo, tb = oracle.ladder(W, free["dead"])
        os_ = oracle.sweep(W, free["U"], free["hdiag"], free["dead"], tb, lo, want_E=False)
        t_orc = oracle.output_error(W, free["dead"], os_["code"], os_["scale"], H)
        t_gpu = output_error(W, free["dead"], nib.cpu().numpy(), scale.cpu().numpy(), H)
        say(f"  precision={rep['precision']} min_pivot={rep['min_pivot']:.3e} relF={err:.2e} "
            f"out rel={(t_gpu - t_orc) / t_orc:+.2e}")
        assert abs(t_gpu - t_orc) <= OUT_ERR_TOL * t_orc
    assert n_f64 >= 6  # most of the class needs the f64 factor


@pytest.mark.parametrize("name", ["tiny", "fixture", "attn"])
def test_f64_fold_is_f64_accurate(gpu, name):
    """The f64 fold against the oracle: relative error of U D at f64 level (the bar is 2e-3;
    the f32 fold sits near 1e-7 here), the same damping, the pivots reported."""
    H, W, lam = workloads.make(name, device="cuda")
    Hn = H.cpu().numpy()
    U, hd, dd, rep = gpu.gptq_fold(H, lam, precision="f64")
    torch.cuda.synchronize()
    orc = oracle.fold(Hn, lam)
    Dk = np.sqrt(hd_diag(Hn, orc["dead"], orc["damp"]))
    err = fold_rel_err(U.cpu().numpy(), orc["U"], Dk)
    say(f"{name} f64: relF={err:.2e} min_pivot={rep['min_pivot']:.3e}")
    assert rep["precision"] == 64 and rep["attempts"] == 1 and rep["lambda_used"] == orc["lam"]
    assert 0.0 < rep["min_pivot"] <= 1.0
    assert err < 1e-6
    np.testing.assert_array_equal(dd.cpu().numpy().astype(bool), orc["dead"])


@pytest.mark.parametrize("n", [96, 301, 640])
def test_f64_fold_ragged_and_padded(gpu, n):
    """n not a multiple of the 64 / 128 blocks, with padded rows of H, in f64."""
    rng = np.random.default_rng(n)
    X = rng.standard_normal((n, n // 2 + 3)) * np.exp(rng.standard_normal(n))[:, None]
    H = (X @ X.T).astype(np.float32)
    ld = n + 37
    Hp = np.full((n, ld), np.nan, np.float32)
    Hp[:, :n] = H
    view = _dev(Hp)[:, :n]
    U, hd, dd, rep = gpu.gptq_fold(view, 1e-5, precision="f64")
    torch.cuda.synchronize()
    orc = oracle.fold(H, 1e-5)
    assert rep["lambda_used"] == orc["lam"] and rep["precision"] == 64
    err = fold_rel_err(U.cpu().numpy(), orc["U"], np.sqrt(hd_diag(H, orc["dead"], orc["damp"])))
    say(f"f64 n={n} ld={ld}: relF={err:.2e}")
    assert err < 1e-6
    assert np.all(np.tril(U.cpu().numpy(), -1) == 0.0)


def test_f32_precision_is_the_pages_device_rule(gpu):
    """GPTQ_FOLD_F32 keeps the pages' device rule: on the stress workload a positive pivot is
    accepted at lambda = 1e-6, the reported smallest pivot is below the floor (the "auto"
    precision would have gone to f64), and the f32 error stays inside the envelope
    1e-5 / min_pivot that the floor was chosen from (the largest ratio seen over 3600 random
    rank-deficient Hessians was 5.7e-6)."""
    H, W, lam = workloads.make("stress", device="cuda")
    Hn = H.cpu().numpy()
    U, hd, dd, rep = gpu.gptq_fold(H, lam, precision="f32")
    torch.cuda.synchronize()
    say(f"stress f32: lambda={rep['lambda_used']} min_pivot={rep['min_pivot']:.3e}")
    assert rep["precision"] == 32 and rep["lambda_used"] == lam and rep["attempts"] == 1
    assert 0.0 < rep["min_pivot"] < PIVOT_FLOOR
    orc = oracle.fold(Hn, lam, retry=False)
    err = fold_rel_err(U.cpu().numpy(), orc["U"], np.sqrt(hd_diag(Hn, orc["dead"], orc["damp"])))
    say(f"stress f32: relF={err:.3e}, envelope {1e-5 / rep['min_pivot']:.3e}")
    assert err <= 1e-5 / rep["min_pivot"]


def test_auto_stays_f32_on_well_conditioned_layers(gpu):
    for name in ("tiny", "fixture"):
        H, W, lam = workloads.make(name, device="cuda")
        U, hd, dd, rep = gpu.gptq_fold(H, lam)
        assert rep["precision"] == 32 and rep["attempts"] == 1 and rep["min_pivot"] > PIVOT_FLOOR, rep


def test_workspace_per_precision(gpu):
    """The f32 precision runs in the smaller workspace its size query names; the other two
    refuse it before writing anything."""
    lib = gpu.load()
    n = 300
    f32_need = gpu.fold_workspace_size(n, "f32")
    assert 0 < f32_need < gpu.fold_workspace_size(n, "auto") == gpu.fold_workspace_size(n, "f64")
    rng = np.random.default_rng(9)
    X = rng.standard_normal((n, 2 * n))
    H = _dev((X @ X.T).astype(np.float32))
    ws = torch.empty(f32_need, dtype=torch.uint8, device="cuda")
    U = torch.full((n, n), 7.0, device="cuda")
    hd = torch.zeros(n, device="cuda")
    dd = torch.zeros(n, dtype=torch.uint8, device="cuda")
    _, _, _, rep = gpu.gptq_fold(H, 0.01, workspace=ws, out=(U, hd, dd), precision="f32")
    torch.cuda.synchronize()
    assert rep["status"] == 0 and rep["precision"] == 32
    U.fill_(7.0)
    for prec in ("auto", "f64"):
        with pytest.raises(ValueError):  # the binding checks the size before the call
            gpu.gptq_fold(H, 0.01, workspace=ws, out=(U, hd, dd), precision=prec)
    import ctypes
    rep = gpu.FoldReport()
    st = lib.gptq_fold_ex(ctypes.c_void_p(H.data_ptr()), n, n, 0.01, 0, ctypes.c_void_p(U.data_ptr()),
                          ctypes.c_void_p(hd.data_ptr()), ctypes.c_void_p(dd.data_ptr()),
                          ctypes.c_void_p(ws.data_ptr()), ws.numel(), None, ctypes.byref(rep))
    torch.cuda.synchronize()
    assert st == gpu.GPTQ_EWORKSPACE
    assert torch.all(U == 7.0)
