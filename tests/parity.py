"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI binding, run the
oracle on the same inputs, and compare to the stated bars.

Bars (from the method's problem statement):
* fold: relative Frobenius error of U * D (columns scaled by D_k = sqrt(H_d,kk), i.e. the factor
  of the equilibrated inverse) <= 2e-3, with the oracle at the GPU's damping;
* sweep, isolated (oracle sweep on the GPU's U, hdiag, dead and ladder), tie-forced replay:
  0 hard disagreements (a code may differ only by one at a rounding tie
  |frac(|w/s|) - 0.5| < 1e-3; a rung only where the candidates' errors are within 1e-4
  relative or the nominal value sits within 1e-3 of a half-integer) and >= 99.9% of codes
  identical; the free-running agreement is reported;
* end to end: tr(dW H dW^T) within 1% of the oracle's (oracle fold at its own damping).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

FOLD_TOL = 2e-3
TIE_BAND = 1e-3
RUNG_BAND = 1e-4
CODE_AGREE = 0.999
OUT_ERR_TOL = 0.01


def say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def hd_diag(H: np.ndarray, dead: np.ndarray, damp: float) -> np.ndarray:
    d = np.where(dead, 1.0, np.diag(H).astype(np.float64))
    return d + damp


def fold_rel_err(U_gpu: np.ndarray, U_orc: np.ndarray, Dk: np.ndarray) -> float:
    a = U_gpu.astype(np.float64) * Dk[None, :]
    b = U_orc * Dk[None, :]
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def gpu_fold(pwq, H_dev, lam):
    U, hdiag, dead, rep = pwq.gptq_fold(H_dev, lam)
    torch.cuda.synchronize()
    return U, hdiag, dead, rep


def check_fold(pwq, H_dev, lam, H_np=None, nt=None):
    """Fold on the GPU and with the oracle at the GPU's damping; assert the bar; return both."""
    H_np = H_dev.cpu().numpy() if H_np is None else H_np
    U, hdiag, dead, rep = gpu_fold(pwq, H_dev, lam)
    orc = oracle.fold(H_np, rep["lambda_used"], retry=False, nt=nt)
    assert orc["status"] == oracle.OK, "oracle cannot factor at the GPU's damping"
    np.testing.assert_array_equal(dead.cpu().numpy().astype(bool), orc["dead"])
    np.testing.assert_array_equal(hdiag.cpu().numpy(), orc["hdiag"])
    np.testing.assert_allclose(rep["base"], orc["base"], rtol=1e-12)
    Ug = U.cpu().numpy()
    Dk = np.sqrt(hd_diag(H_np, orc["dead"], orc["damp"]))
    err = fold_rel_err(Ug, orc["U"], Dk)
    say(f"fold n={H_np.shape[0]} lambda_gpu={rep['lambda_used']} attempts={rep['attempts']} "
        f"relF(U D)={err:.3e}")
    assert err <= FOLD_TOL, err
    assert np.all(np.tril(Ug, -1) == 0.0)
    return (U, hdiag, dead, rep), orc, err


def check_sweep_isolated(pwq, W_dev, U, hdiag, dead, rows_sel=None, want_E=True, nt=None):
    """GPU ladder + sweep; oracle ladder (must match bit for bit) and oracle sweep on the GPU's
    U in free-running and tie-forced replay modes.  Returns a dict of statistics."""
    lost, tab = pwq.gptq_ladder(W_dev, dead)
    nib, rung, scale, E = pwq.gptq_sweep(W_dev, U, hdiag, dead, tab, lost, want_E=want_E)
    torch.cuda.synchronize()
    W = W_dev.cpu().numpy()
    d = dead.cpu().numpy().astype(bool)
    lost_o, tab_o = oracle.ladder(W, d)
    np.testing.assert_array_equal(lost.cpu().numpy(), lost_o)
    np.testing.assert_array_equal(tab.cpu().numpy(), tab_o)
    sel = np.arange(W.shape[0]) if rows_sel is None else np.asarray(rows_sel)
    code_g = oracle.unpack_nibbles(nib.cpu().numpy()[sel])
    rung_g = rung.cpu().numpy()[sel]
    scale_g = scale.cpu().numpy()[sel]
    Ud = U.cpu().numpy().astype(np.float64)
    hd = hdiag.cpu().numpy()
    free = oracle.sweep(W[sel], Ud, hd, d, tab_o[sel], lost_o[sel], nt=nt)
    rep = oracle.sweep(W[sel], Ud, hd, d, tab_o[sel], lost_o[sel], force_code=code_g,
                       force_rung=rung_g, tie_band=TIE_BAND, rung_band=RUNG_BAND, nt=nt)
    same = float((free["code"] == code_g).mean())
    same_rung = float((free["rung"] == rung_g).mean())
    total = code_g.size
    st = dict(rep["stats"], code_agree=same, rung_agree=same_rung, rows=len(sel),
              replay_agree=1.0 - (rep["stats"]["code_ties"] + rep["stats"]["code_hard"]) / total)
    # scales are TAB[rung] exactly
    np.testing.assert_array_equal(scale_g, np.take_along_axis(tab_o[sel], rung_g.astype(int), 1))
    if want_E:
        Eg = E.cpu().numpy()[sel].astype(np.float64)
        denom = np.linalg.norm(rep["E"])
        st["E_relF"] = float(np.linalg.norm(Eg - rep["E"]) / max(denom, 1e-300))
    say(f"sweep rows={len(sel)} n={W.shape[1]} {st}")
    return st, (nib, rung, scale, E, lost, tab)


def assert_sweep_bar(st):
    """0 hard disagreements, and >= 99.9% of codes identical in the tie-forced replay (the
    comparison where every disagreement is classified; a single tie flip in free-running mode
    sends the rest of its row down another, equally valid trajectory, so the free-running
    agreement is reported, not asserted)."""
    assert st["code_hard"] == 0, st
    assert st["rung_hard"] == 0, st
    assert st["replay_agree"] >= CODE_AGREE, st


def output_error(W_np, dead_np, nib, scale, H_np):
    code = oracle.unpack_nibbles(nib)
    return oracle.output_error(W_np, dead_np, code, scale, H_np)
