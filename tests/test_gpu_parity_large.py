"""GPU parity at the method's layer sizes, whole: every entry of U against the oracle fold at
the GPU's damping, every row of the sweep in the oracle's tie-forced replay on the GPU's U,
and the layer-output error against the free-running oracle (its own fold and sweep) on
sampled rows.  The n = 17408 layer runs in the launch configuration the benchmark times."""
import threading

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import (OUT_ERR_TOL, assert_sweep_bar, check_fold, check_sweep_isolated,
                    output_error, say)

pytestmark = pytest.mark.gpu

# The "auto" fold stays in f32 while the smallest pivot of the equilibrated matrix is above this
# floor (include/gptq.h, GPTQ_FOLD_AUTO).
PIVOT_FLOOR = 1e-2


def _rows(rows, k, seed=0):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(rows, size=k, replace=False))


def _end_to_end(Hn, Wn, sel, of, nib, scale, tag):
    """tr(dW H dW^T) of the GPU's codes against the free-running oracle's (its own fold ``of``
    and its own sweep) on the rows ``sel``; two-sided 1%."""
    lo, tb = oracle.ladder(Wn[sel], of["dead"])
    os_ = oracle.sweep(Wn[sel], of["U"], of["hdiag"], of["dead"], tb, lo, want_E=False)
    t_orc = oracle.output_error(Wn[sel], of["dead"], os_["code"], os_["scale"], Hn)
    t_gpu = output_error(Wn[sel], of["dead"], nib.cpu().numpy()[sel], scale.cpu().numpy()[sel], Hn)
    rel = (t_gpu - t_orc) / t_orc
    say(f"{tag}: tr(dW H dW^T) on {len(sel)} rows gpu={t_gpu:.6e} oracle={t_orc:.6e} rel={rel:+.3e}")
    assert abs(t_gpu - t_orc) <= OUT_ERR_TOL * t_orc


def test_attention_shaped_layer(gpu):
    """n = 4096, all 4096 rows."""
    say("attn n=4096 rows=4096")
    H, W, lam = workloads.make("attn", device="cuda")
    Hn, Wn = H.cpu().numpy(), W.cpu().numpy()
    (U, hdiag, dead, rep), orc, err = check_fold(gpu, H, lam, H_np=Hn)
    assert rep["n_dead"] == 20
    assert rep["precision"] == 32 and rep["min_pivot"] > PIVOT_FLOOR, rep
    st, (nib, rung, scale, E, lost, tab) = check_sweep_isolated(gpu, W, U, hdiag, dead)
    assert_sweep_bar(st)
    assert orc["lam"] == lam
    _end_to_end(Hn, Wn, _rows(Wn.shape[0], 512), orc, nib, scale, "attn")


def test_ill_conditioned_retry_path(gpu):
    """The rank-deficient stress workload from lambda = 1e-6.  Its f32 factor has a pivot below
    the accuracy floor, so the fold runs in f64 with the host's pivot rule and reaches the
    damping the f64 oracle reaches from the same start; U meets the fold bar there (in f64 it is
    far inside it), and the layer-output error is within 1% of the free-running oracle's."""
    say("stress n=8192 rows=2048 lambda0=1e-6")
    H, W, lam = workloads.make("stress", device="cuda")
    Hn, Wn = H.cpu().numpy(), W.cpu().numpy()
    (U, hdiag, dead, rep), orc, err = check_fold(gpu, H, lam, H_np=Hn)
    free = oracle.fold(Hn, lam)
    say(f"stress: lambda_gpu={rep['lambda_used']} attempts={rep['attempts']} precision={rep['precision']} "
        f"min_pivot={rep['min_pivot']:.3e} lambda_oracle={free['lam']} attempts_oracle={free['attempts']}")
    assert rep["n_dead"] == 164
    assert rep["precision"] == 64 and rep["lambda_used"] == free["lam"], rep
    assert err <= 1e-6, err
    sel = _rows(W.shape[0], 256, 1)
    st, (nib, rung, scale, E, lost, tab) = check_sweep_isolated(gpu, W, U, hdiag, dead, rows_sel=sel)
    assert_sweep_bar(st)
    _end_to_end(Hn, Wn, sel, free, nib, scale, "stress")


def test_down_proj_full_size(gpu):
    """n = 17408, rows = 5120 (the benchmark's workload and launch configuration): the whole U
    against the oracle fold at the GPU's damping, all 5120 rows in the tie-forced replay, and
    the layer-output error on 256 sampled rows against the free-running oracle.  The fold
    stays on the f32 path (its smallest pivot is far above the floor)."""
    say("down n=17408 rows=5120")
    H, W, lam = workloads.make("down", device="cuda")
    Hn = H.cpu().numpy()
    (U, hdiag, dead, rep), orc, err = check_fold(gpu, H, lam, H_np=Hn)
    say(f"down: lambda={rep['lambda_used']} attempts={rep['attempts']} precision={rep['precision']} "
        f"min_pivot={rep['min_pivot']:.3e} relF(U D)={err:.3e}")
    assert rep["attempts"] == 1 and rep["precision"] == 32 and rep["min_pivot"] > PIVOT_FLOOR, rep
    assert orc["lam"] == lam
    st, (nib, rung, scale, E, lost, tab) = check_sweep_isolated(gpu, W, U, hdiag, dead, want_E=True)
    assert_sweep_bar(st)
    say(f"down: free-running code agreement {st['code_agree']:.6f}, replay {st['replay_agree']:.6f}")
    Wn = W.cpu().numpy()
    sel = _rows(Wn.shape[0], 256, 2)
    # dW = E U at any size, on the GPU's own outputs.
    Ud = U.cpu().numpy().astype(np.float64)
    code = oracle.unpack_nibbles(nib.cpu().numpy()[sel])
    dW = Wn[sel].astype(np.float64) - oracle.dequant(code, scale.cpu().numpy()[sel])
    Eg = E.cpu().numpy()[sel].astype(np.float64)
    rel = np.linalg.norm(Eg @ Ud - dW) / np.linalg.norm(dW)
    say(f"down: ||E U - dW|| / ||dW|| = {rel:.3e} on {len(sel)} rows")
    assert rel < 1e-4
    del Ud, Eg, dW
    _end_to_end(Hn, Wn, sel, orc, nib, scale, "down")


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
