"""GPU parity at the method's layer sizes.  Where the oracle finishes in seconds it runs whole
(n = 4096; n = 8192 fold); at n = 17408, in the launch configuration the benchmark times, the
checks use outputs the oracle computes one by one (a trailing block of U, the first row of U,
sampled rows of the sweep) and properties that hold at any size."""
import threading

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import (FOLD_TOL, OUT_ERR_TOL, assert_sweep_bar, check_fold, check_sweep_isolated,
                    fold_rel_err, hd_diag, output_error, say)

pytestmark = pytest.mark.gpu


def _rows(rows, k, seed=0):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(rows, size=k, replace=False))


def test_attention_shaped_layer(gpu):
    say("attn n=4096 rows=4096")
    H, W, lam = workloads.make("attn", device="cuda")
    Hn, Wn = H.cpu().numpy(), W.cpu().numpy()
    (U, hdiag, dead, rep), orc, err = check_fold(gpu, H, lam, H_np=Hn)
    assert rep["n_dead"] == 20
    sel = _rows(Wn.shape[0], 256)
    st, (nib, rung, scale, E, lost, tab) = check_sweep_isolated(gpu, W, U, hdiag, dead, rows_sel=sel)
    assert_sweep_bar(st)
    # End to end on the sampled rows: the oracle's own fold and sweep at its own damping.
    of = orc if orc["lam"] == lam else oracle.fold(Hn, lam)
    lo, tb = oracle.ladder(Wn[sel], of["dead"])
    os_ = oracle.sweep(Wn[sel], of["U"], of["hdiag"], of["dead"], tb, lo, want_E=False)
    t_orc = oracle.output_error(Wn[sel], of["dead"], os_["code"], os_["scale"], Hn)
    t_gpu = output_error(Wn[sel], of["dead"], nib.cpu().numpy()[sel], scale.cpu().numpy()[sel], Hn)
    say(f"attn: tr(dW H dW^T) gpu={t_gpu:.6e} oracle={t_orc:.6e} rel={(t_gpu - t_orc) / t_orc:.2e}")
    assert abs(t_gpu - t_orc) <= OUT_ERR_TOL * t_orc


def test_ill_conditioned_retry_path(gpu):
    say("stress n=8192 rows=2048 lambda0=1e-6")
    H, W, lam = workloads.make("stress", device="cuda")
    Hn = H.cpu().numpy()
    (U, hdiag, dead, rep), orc, err = check_fold(gpu, H, lam, H_np=Hn)
    say(f"stress: lambda_gpu={rep['lambda_used']} attempts={rep['attempts']} n_dead={rep['n_dead']}")
    assert rep["attempts"] >= 2 and rep["lambda_used"] > lam, rep
    assert rep["n_dead"] == 164
    # The f64 oracle's own schedule from the same start ends no later than the f32 one.
    free = oracle.fold(Hn, lam)
    say(f"stress: lambda_oracle={free['lam']} attempts={free['attempts']}")
    assert free["lam"] <= rep["lambda_used"]
    sel = _rows(W.shape[0], 128, 1)
    st, (nib, rung, scale, E, lost, tab) = check_sweep_isolated(gpu, W, U, hdiag, dead, rows_sel=sel)
    assert_sweep_bar(st)
    # End to end on the sampled rows.  On this rank-deficient Hessian at small damping the
    # greedy rounding is chaotic: perturbing the oracle's own U by 2e-4 (relative Frobenius)
    # moves tr(dW H dW^T) by several percent either way, so the bar here is the pages' own
    # device-versus-host one: the GPU not worse than 1.05x the oracle, both at the GPU's damping
    # and free-running at its own.
    Wn = W.cpu().numpy()
    t_gpu = output_error(Wn[sel], free["dead"], nib.cpu().numpy()[sel], scale.cpu().numpy()[sel], Hn)
    for tag, f in (("oracle at lambda_gpu", orc), ("free-running oracle", free)):
        lo, tb = oracle.ladder(Wn[sel], f["dead"])
        os_ = oracle.sweep(Wn[sel], f["U"], f["hdiag"], f["dead"], tb, lo, want_E=False)
        t_orc = oracle.output_error(Wn[sel], f["dead"], os_["code"], os_["scale"], Hn)
        rel = (t_gpu - t_orc) / t_orc
        say(f"stress: tr(dW H dW^T) gpu={t_gpu:.6e} {tag}={t_orc:.6e} rel={rel:.2e}")
        assert t_gpu <= 1.05 * t_orc


def test_down_proj_full_size_sampled(gpu):
    """n = 17408, rows = 5120: U's trailing 3072 block against the oracle fold of H_d's trailing
    block (the same damping; the factor's block structure makes them equal), U's first row
    against LAPACK's H_d^-1 e_0 / sqrt(H_d^-1[0,0]), and 24 sampled rows of the sweep."""
    say("down n=17408 rows=5120")
    H, W, lam = workloads.make("down", device="cuda")
    n = H.shape[0]
    U, hdiag, dead, rep = gpu.gptq_fold(H, lam)
    torch.cuda.synchronize()
    say(f"down: lambda={rep['lambda_used']} attempts={rep['attempts']} base={rep['base']:.6e}")
    m = 3072
    Hb = H[n - m:, n - m:].contiguous().cpu().numpy()
    base_b = np.diag(Hb).astype(np.float64).mean()
    ob = oracle.fold(Hb, rep["damp"] / base_b, retry=False)
    assert ob["status"] == oracle.OK
    Ub = U[n - m:, n - m:].cpu().numpy()
    Dk = np.sqrt(hd_diag(Hb, ob["dead"], rep["damp"]))
    err_b = fold_rel_err(Ub, ob["U"], Dk)
    say(f"down: trailing {m} block relF(U D)={err_b:.3e}")
    assert err_b <= FOLD_TOL
    # First row: a closed form through one f64 solve (LAPACK).
    Hn = H.cpu().numpy().astype(np.float64)
    Hs = np.triu(Hn) + np.triu(Hn, 1).T
    del Hn
    Hs[np.diag_indices(n)] += rep["damp"]
    e0 = np.zeros(n)
    e0[0] = 1.0
    import scipy.linalg as sla
    x = sla.cho_solve(sla.cho_factor(Hs, lower=False, overwrite_a=False, check_finite=False), e0)
    row_ref = x / np.sqrt(x[0])
    D = np.sqrt(np.diag(Hs))
    del Hs
    row = U[0].cpu().numpy().astype(np.float64)
    err_r = float(np.linalg.norm((row - row_ref) * D) / np.linalg.norm(row_ref * D))
    say(f"down: first row relF(U D)={err_r:.3e}")
    assert err_r <= FOLD_TOL
    # Sweep: sampled rows against the oracle on the GPU's U.
    sel = _rows(W.shape[0], 24, 2)
    st, (nib, rung, scale, E, lost, tab) = check_sweep_isolated(gpu, W, U, hdiag, dead,
                                                                rows_sel=sel, want_E=True)
    assert st["code_hard"] == 0 and st["rung_hard"] == 0, st
    # Closed form at any size on the GPU's own outputs: dW = E U, so for every row
    # ||dW H_d||-weighted error equals ||e||^2; checked on the sampled rows in f64.
    Ud = U.cpu().numpy().astype(np.float64)
    Wn = W.cpu().numpy()[sel].astype(np.float64)
    code = oracle.unpack_nibbles(nib.cpu().numpy()[sel])
    dW = Wn - oracle.dequant(code, scale.cpu().numpy()[sel])
    Eg = E.cpu().numpy()[sel].astype(np.float64)
    rel = np.linalg.norm(Eg @ Ud - dW) / np.linalg.norm(dW)
    say(f"down: ||E U - dW|| / ||dW|| = {rel:.3e} (sampled rows), code agreement {st['code_agree']:.5f}")
    assert rel < 1e-4


def test_batched_round_on_streams(gpu):
    """11 independent n = 4096 groups folded and swept concurrently on 11 streams: each result
    equals the same group run alone, bit for bit; one group is also checked against the oracle."""
    say("batch 11 x n=4096 on streams")
    groups = []
    for k in range(11):
        H, W, lam = workloads.make("batch", k=k, device="cuda")
        groups.append((H, W, lam))
    torch.cuda.synchronize()

    def run(H, W, lam):
        U, hd, dd, rep = gpu.gptq_fold(H, lam)
        lost, tab = gpu.gptq_ladder(W, dd)
        nib, rung, scale, _ = gpu.gptq_sweep(W, U, hd, dd, tab, lost)
        return U, nib, rung, scale, rep

    solo = [run(*g) for g in groups]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in groups]
    outs = [None] * len(groups)
    errs = []

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                outs[i] = run(*groups[i])
                streams[i].synchronize()
        except Exception as e:  # surfaced below
            errs.append(e)

    th = [threading.Thread(target=worker, args=(i,)) for i in range(len(groups))]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    assert not errs, errs
    for i, (a, b) in enumerate(zip(solo, outs)):
        for x, y in zip(a[:4], b[:4]):
            assert torch.equal(x, y), f"group {i} differs between solo and concurrent runs"
    H, W, lam = groups[3]
    (U, hdiag, dead, rep), orc, err = check_fold(gpu, H, lam)
    st, _ = check_sweep_isolated(gpu, W, U, hdiag, dead, rows_sel=_rows(4096, 128, 3))
    assert_sweep_bar(st)
