"""GPU parity of act-order GPTQ against the oracle: the channel order and dead mask (exact), the
permuted Hessian (exact: data movement), the fold of the permuted Hessian (the fold's bar), the
static rungs (exact: both sides sum the unit-weight error in f32 in column order), the codes in
a tie-forced replay of the oracle's act-order sweep on the GPU's U (0 hard disagreements,
>= 99.9% identical) and the end-to-end layer-output error within 1% of the free-running oracle.
Down_proj shape: 24 sampled rows (rows are independent given U)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import CODE_AGREE, TIE_BAND, check_fold, say


def run_gpu(gpu, H, W, lam):
    perm, dead = gpu.gptq_act_order_perm(H)
    Hp = gpu.gptq_permute_hessian(H, perm)
    torch.cuda.synchronize()
    return perm, dead, Hp


def check_order(perm, dead, Hp, H_np):
    hd = np.diag(H_np).astype(np.float32)
    p_o = oracle.act_order_perm(hd)
    assert np.array_equal(perm.cpu().numpy().astype(np.int64), p_o)
    assert np.array_equal(dead.cpu().numpy().astype(bool), ~(hd > 0))
    Hp_o = oracle.permute_sym(H_np, p_o)
    assert np.array_equal(Hp.cpu().numpy().astype(np.float64), Hp_o)
    return p_o


def check_sweep(gpu, W, Up, dead, perm, p_o, rows_sel=None, want_E=True):
    lost, tab = gpu.gptq_ladder(W, dead)
    nib, rung, scale, E = gpu.gptq_sweep_act_order(W, Up, dead, perm, tab, lost, want_E=want_E)
    torch.cuda.synchronize()
    Wn = W.cpu().numpy()
    d = dead.cpu().numpy().astype(bool)
    lost_o, tab_o = oracle.ladder(Wn, d)
    assert np.array_equal(lost.cpu().numpy(), lost_o) and np.array_equal(tab.cpu().numpy(), tab_o)
    sel = np.arange(Wn.shape[0]) if rows_sel is None else np.asarray(rows_sel)
    rung_o, scale_o = oracle.static_rungs(Wn[sel], d, tab_o[sel], lost_o[sel])
    assert np.array_equal(rung.cpu().numpy()[sel], rung_o), "static rungs differ"
    assert np.array_equal(scale.cpu().numpy()[sel], scale_o)
    code_g = oracle.unpack_nibbles(nib.cpu().numpy()[sel])
    Ud = Up.cpu().numpy().astype(np.float64)
    free = oracle.sweep_act_order(Wn[sel], Ud, d, p_o, tab_o[sel], lost_o[sel], rung=rung_o)
    rep = oracle.sweep_act_order(Wn[sel], Ud, d, p_o, tab_o[sel], lost_o[sel], rung=rung_o,
                                 force_code=code_g, tie_band=TIE_BAND)
    total = code_g.size
    st = dict(rep["stats"], code_agree=float((free["code"] == code_g).mean()),
              replay_agree=1.0 - (rep["stats"]["code_ties"] + rep["stats"]["code_hard"]) / total)
    if want_E:
        Eg = E.cpu().numpy()[sel].astype(np.float64)
        st["E_relF"] = float(np.linalg.norm(Eg - rep["E"]) / max(np.linalg.norm(rep["E"]), 1e-300))
    say(f"act-order sweep rows={len(sel)} {st}")
    assert st["code_hard"] == 0, st
    assert st["replay_agree"] >= CODE_AGREE, st
    return nib, scale, st


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["tiny", "fixture"])
def test_act_order_small_workloads(gpu, name):
    H, W, lam = workloads.make(name, device="cuda:0")
    H_np = H.cpu().numpy()
    perm, dead, Hp = run_gpu(gpu, H, W, lam)
    p_o = check_order(perm, dead, Hp, H_np)
    (Up, hdiag_p, dead_p, rep), orc, err = check_fold(gpu, Hp, lam)
    assert np.array_equal(dead_p.cpu().numpy(), dead.cpu().numpy()[p_o])
    nib, scale, st = check_sweep(gpu, W, Up, dead, perm, p_o)
    # End to end against the free-running oracle (its own fold and damping).
    Wn = W.cpu().numpy()
    d = dead.cpu().numpy().astype(bool)
    f_o = oracle.fold(oracle.permute_sym(H_np, p_o).astype(np.float32), lam)
    lost_o, tab_o = oracle.ladder(Wn, d)
    ao = oracle.sweep_act_order(Wn, f_o["U"], d, p_o, tab_o, lost_o)
    t_o = oracle.output_error(Wn, d, ao["code"], ao["scale"], H_np)
    t_g = oracle.output_error(Wn, d, oracle.unpack_nibbles(nib.cpu().numpy()), scale.cpu().numpy(), H_np)
    say(f"act-order {name}: tr(dW H dW^T) gpu {t_g:.6e} oracle {t_o:.6e}")
    assert abs(t_g - t_o) <= 0.01 * t_o
    # Plain sweep's error for context: act order should not be worse by much on these inputs.
    assert t_g > 0


@pytest.mark.gpu
@pytest.mark.parametrize("n,rows", [(96, 37), (288, 130)])
def test_act_order_ragged(gpu, n, rows):
    H, W, lam = workloads.make("attn", device="cuda:0", n=n, rows=rows, T=1024)
    H_np = H.cpu().numpy()
    perm, dead, Hp = run_gpu(gpu, H, W, lam)
    p_o = check_order(perm, dead, Hp, H_np)
    (Up, _, _, _), _, _ = check_fold(gpu, Hp, lam)
    check_sweep(gpu, W, Up, dead, perm, p_o)


@pytest.mark.gpu
def test_act_order_ties_and_special_diagonals(gpu):
    n = 64
    rng = np.random.default_rng(3)
    X = rng.standard_normal((n, 200)).astype(np.float32)
    H = X @ X.T
    d = np.diag(H).copy()
    d[[3, 9, 20]] = 5.0        # ties broken by index
    d[[30, 31]] = 0.0          # dead channels
    H[np.arange(n), np.arange(n)] = d
    H[30, :] = 0.0
    H[:, 30] = 0.0
    H[31, :] = 0.0
    H[:, 31] = 0.0
    Hd = torch.from_numpy(H).cuda()
    perm, dead, Hp = run_gpu(gpu, Hd, None, 0.01)
    check_order(perm, dead, Hp, H)


@pytest.mark.gpu
def test_act_order_down_proj_sampled(gpu):
    H, W, lam = workloads.make("down", device="cuda:0")
    perm, dead, Hp = run_gpu(gpu, H, W, lam)
    hd = np.diag(H.cpu().numpy()).astype(np.float32)
    p_o = oracle.act_order_perm(hd)
    assert np.array_equal(perm.cpu().numpy().astype(np.int64), p_o)
    # The permuted Hessian on a sample of entries.
    idx = np.random.default_rng(4).integers(0, H.shape[0], size=(2, 400))
    Hn = H.cpu().numpy()
    got = Hp.cpu().numpy()[idx[0], idx[1]]
    a, b = p_o[idx[0]], p_o[idx[1]]
    assert np.array_equal(got, Hn[np.minimum(a, b), np.maximum(a, b)])
    del Hn
    U, hdiag, dead_p, rep = gpu.gptq_fold(Hp, lam)
    torch.cuda.synchronize()
    sel = np.sort(np.random.default_rng(5).choice(W.shape[0], 24, replace=False))
    check_sweep(gpu, W, U, dead, perm, p_o, rows_sel=sel, want_E=False)


# --- act order with 2-bit codes (q2tp) ---------------------------------------------------------

def check_sweep_q2(gpu, W, Up, hdiag_p, dead, perm, p_o, rows_sel=None, want_E=True):
    """The q2tp act-order sweep: the q2 ladder bit for bit, the static rungs exactly (both sides
    sum the clipped-H_ii-weighted error in f32 in column order), the levels in a tie-forced
    replay of the oracle's static q2 sweep on the GPU's U (0 hard, >= 99.9% identical)."""
    lost, tab = gpu.gptq_ladder_q2(W, dead)
    plane, rung, scale, E = gpu.gptq_sweep_act_order_q2(W, Up, dead, hdiag_p, perm, tab, want_E=want_E)
    torch.cuda.synchronize()
    Wn = W.cpu().numpy()
    n = Wn.shape[1]
    d = dead.cpu().numpy().astype(bool)
    lost_o, tab_o = oracle.ladder_q2(Wn, d)
    assert np.array_equal(lost.cpu().numpy(), lost_o) and np.array_equal(tab.cpu().numpy(), tab_o)
    hd = np.empty(n, np.float32)
    hd[p_o] = hdiag_p.cpu().numpy()  # back to the original channel order
    sel = np.arange(Wn.shape[0]) if rows_sel is None else np.asarray(rows_sel)
    rung_o, scale_o = oracle.static_rungs_q2(Wn[sel], d, tab_o[sel], hd)
    assert np.array_equal(rung.cpu().numpy()[sel], rung_o), "static q2 rungs differ"
    assert np.array_equal(scale.cpu().numpy()[sel], scale_o)
    code_g = oracle.unpack_q2(plane.cpu().numpy()[sel])
    Ud = Up.cpu().numpy().astype(np.float64)
    free = oracle.sweep_act_order(Wn[sel], Ud, d, p_o, tab_o[sel], lost_o[sel], rung=rung_o, two_bit=True)
    rep = oracle.sweep_act_order(Wn[sel], Ud, d, p_o, tab_o[sel], lost_o[sel], rung=rung_o,
                                 force_code=code_g, tie_band=TIE_BAND, two_bit=True)
    total = code_g.size
    st = dict(rep["stats"], code_agree=float((free["code"] == code_g).mean()),
              replay_agree=1.0 - (rep["stats"]["code_ties"] + rep["stats"]["code_hard"]) / total)
    if want_E:
        Eg = E.cpu().numpy()[sel].astype(np.float64)
        st["E_relF"] = float(np.linalg.norm(Eg - rep["E"]) / max(np.linalg.norm(rep["E"]), 1e-300))
        assert st["E_relF"] <= 1e-3, st
    say(f"act-order q2 sweep rows={len(sel)} {st}")
    assert st["code_hard"] == 0, st
    assert st["replay_agree"] >= CODE_AGREE, st
    return plane, scale, st


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["tiny", "fixture"])
def test_act_order_q2_small_workloads(gpu, name):
    H, W, lam = workloads.make(name, device="cuda:0")
    H_np = H.cpu().numpy()
    perm, dead, Hp = run_gpu(gpu, H, W, lam)
    p_o = check_order(perm, dead, Hp, H_np)
    (Up, hdiag_p, dead_p, rep), orc, err = check_fold(gpu, Hp, lam)
    plane, scale, st = check_sweep_q2(gpu, W, Up, hdiag_p, dead, perm, p_o)
    # End to end against the free-running oracle (its own fold of the permuted Hessian).
    Wn = W.cpu().numpy()
    d = dead.cpu().numpy().astype(bool)
    f_o = oracle.fold(oracle.permute_sym(H_np, p_o).astype(np.float32), lam)
    lost_o, tab_o = oracle.ladder_q2(Wn, d)
    ao = oracle.sweep_act_order(Wn, f_o["U"], d, p_o, tab_o, lost_o, two_bit=True,
                                hdiag=np.diag(H_np).astype(np.float32))

    def t(code, sc):
        Wz = Wn.astype(np.float64)
        Wz[:, d] = 0.0
        dW = Wz - oracle.dequant_q2(code, sc)
        dW[:, d] = 0.0
        return float(np.einsum("ij,jk,ik->", dW, oracle.symmetric_from_upper(H_np), dW))

    t_o = t(ao["code"], ao["scale"])
    t_g = t(oracle.unpack_q2(plane.cpu().numpy()), scale.cpu().numpy())
    say(f"act-order q2 {name}: tr(dW H dW^T) gpu {t_g:.6e} oracle {t_o:.6e}")
    assert abs(t_g - t_o) <= 0.01 * t_o


@pytest.mark.gpu
@pytest.mark.parametrize("n,rows", [(96, 37), (288, 130)])
def test_act_order_q2_ragged(gpu, n, rows):
    H, W, lam = workloads.make("attn", device="cuda:0", n=n, rows=rows, T=1024)
    H_np = H.cpu().numpy()
    perm, dead, Hp = run_gpu(gpu, H, W, lam)
    p_o = check_order(perm, dead, Hp, H_np)
    (Up, hdiag_p, _, _), _, _ = check_fold(gpu, Hp, lam)
    check_sweep_q2(gpu, W, Up, hdiag_p, dead, perm, p_o)


@pytest.mark.gpu
def test_act_order_q2_down_proj_sampled(gpu):
    H, W, lam = workloads.make("down", device="cuda:0")
    perm, dead, Hp = run_gpu(gpu, H, W, lam)
    p_o = oracle.act_order_perm(np.diag(H.cpu().numpy()).astype(np.float32))
    assert np.array_equal(perm.cpu().numpy().astype(np.int64), p_o)
    U, hdiag_p, dead_p, rep = gpu.gptq_fold(Hp, lam)
    torch.cuda.synchronize()
    sel = np.sort(np.random.default_rng(6).choice(W.shape[0], 24, replace=False))
    check_sweep_q2(gpu, W, U, hdiag_p, dead, perm, p_o, rows_sel=sel, want_E=False)
