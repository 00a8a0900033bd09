"""GPU parity of the q2tp sweep ("placed" rule) against the oracle: the q2 ladder bit for bit;
the sweep isolated (oracle on the GPU's U, weights and ladder) in a tie-forced replay with 0
hard disagreements and >= 99.9% identical codes (a level may differ by one only where
w/s + 1.5 lies within 1e-3 of a half-integer; a rung only where the two rungs' errors are
within 1e-4 relative); E against the replay; the layer-output error within 1% of the
free-running oracle (its own fold).  Down_proj shape: 24 sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import CODE_AGREE, RUNG_BAND, TIE_BAND, check_fold, say


def check_q2(gpu, W, U, hdiag, dead, rows_sel=None, want_E=True):
    lost, tab = gpu.gptq_ladder_q2(W, dead)
    plane, rung, scale, E = gpu.gptq_sweep_q2(W, U, hdiag, dead, tab, want_E=want_E)
    torch.cuda.synchronize()
    Wn = W.cpu().numpy()
    d = dead.cpu().numpy().astype(bool)
    lost_o, tab_o = oracle.ladder_q2(Wn, d)
    assert np.array_equal(lost.cpu().numpy(), lost_o) and np.array_equal(tab.cpu().numpy(), tab_o)
    sel = np.arange(Wn.shape[0]) if rows_sel is None else np.asarray(rows_sel)
    code_g = oracle.unpack_q2(plane.cpu().numpy()[sel])
    rung_g = rung.cpu().numpy()[sel]
    Ud = U.cpu().numpy().astype(np.float64)
    hd = hdiag.cpu().numpy()
    free = oracle.sweep_q2(Wn[sel], Ud, hd, d, tab_o[sel])
    rep = oracle.sweep_q2(Wn[sel], Ud, hd, d, tab_o[sel], force_code=code_g, force_rung=rung_g,
                          tie_band=TIE_BAND, rung_band=RUNG_BAND)
    total = code_g.size
    st = dict(rep["stats"], code_agree=float((free["code"] == code_g).mean()),
              rung_agree=float((free["rung"] == rung_g).mean()),
              replay_agree=1.0 - (rep["stats"]["code_ties"] + rep["stats"]["code_hard"]) / total)
    assert np.array_equal(scale.cpu().numpy()[sel], np.take_along_axis(tab_o[sel], rung_g.astype(int), 1))
    if want_E:
        Eg = E.cpu().numpy()[sel].astype(np.float64)
        st["E_relF"] = float(np.linalg.norm(Eg - rep["E"]) / max(np.linalg.norm(rep["E"]), 1e-300))
        assert st["E_relF"] <= 1e-3, st
    say(f"q2 sweep rows={len(sel)} {st}")
    assert st["code_hard"] == 0 and st["rung_hard"] == 0, st
    assert st["replay_agree"] >= CODE_AGREE, st
    return plane, scale, st


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["tiny", "fixture"])
def test_q2_small_workloads(gpu, name):
    H, W, lam = workloads.make(name, device="cuda:0")
    (U, hdiag, dead, rep), orc, err = check_fold(gpu, H, lam)
    plane, scale, st = check_q2(gpu, W, U, hdiag, dead)
    Hn, Wn = H.cpu().numpy(), W.cpu().numpy()
    d = orc["dead"]
    lost_o, tab_o = oracle.ladder_q2(Wn, d)
    free = oracle.sweep_q2(Wn, orc["U"], orc["hdiag"], d, tab_o)
    def t(code, sc):
        Wz = Wn.astype(np.float64)
        Wz[:, d] = 0.0
        dW = Wz - oracle.dequant_q2(code, sc)
        dW[:, d] = 0.0
        Hs = oracle.symmetric_from_upper(Hn)
        return float(np.einsum("ij,jk,ik->", dW, Hs, dW))
    t_o = t(free["code"], free["scale"])
    t_g = t(oracle.unpack_q2(plane.cpu().numpy()), scale.cpu().numpy())
    say(f"q2 {name}: tr(dW H dW^T) gpu {t_g:.6e} oracle {t_o:.6e}")
    assert abs(t_g - t_o) <= 0.01 * t_o


@pytest.mark.gpu
@pytest.mark.parametrize("n,rows", [(32, 1), (160, 70), (288, 130)])
def test_q2_ragged(gpu, n, rows):
    H, W, lam = workloads.make("attn", device="cuda:0", n=n, rows=rows, T=1024)
    (U, hdiag, dead, rep), _, _ = check_fold(gpu, H, lam)
    check_q2(gpu, W, U, hdiag, dead)


@pytest.mark.gpu
def test_q2_zero_rows_and_groups(gpu):
    H, W, lam = workloads.make("tiny", device="cuda:0")
    W = W.clone()
    W[3] = 0.0            # an all-zero row
    W[5, 64:96] = 0.0     # an all-zero group
    U, hdiag, dead, rep = gpu.gptq_fold(H, lam)
    plane, scale, st = check_q2(gpu, W, U, hdiag, dead)
    assert np.all(scale.cpu().numpy()[3] == 0.0)


@pytest.mark.gpu
def test_q2_down_proj_sampled(gpu):
    H, W, lam = workloads.make("down", device="cuda:0")
    U, hdiag, dead, rep = gpu.gptq_fold(H, lam)
    torch.cuda.synchronize()
    sel = np.sort(np.random.default_rng(6).choice(W.shape[0], 24, replace=False))
    check_q2(gpu, W, U, hdiag, dead, rows_sel=sel, want_E=False)
