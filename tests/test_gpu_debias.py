"""GPU parity of the output debias (gptq_debias) against the oracle's f64 definition, on the
GPU's own codes (fold, ladder and sweep run first on the GPU).  Bar: the slope b within the
rounding bound of the f32 product W H (K = n terms, (n + 2) u |W| |H|, u = 2^-24) carried
through num / den; the new lo bit-identical to the oracle's wherever the oracle's value before
the f16 rounding lies farther than that bound from a rounding boundary, else within one f16
step; TAB and the scales exactly f32(2^(lo + c step)) of the GPU's lo.  At the down_proj shape
16 rows are checked."""
import numpy as np
import pytest
import torch

import oracle
import workloads

U32 = 2.0 ** -24


def f16_boundary_distance(v):
    """Distance of v to the nearest midpoint between two binary16 values."""
    ulp = oracle.f16_ulp(v)
    lo = np.floor(v / ulp) * ulp
    return abs(v - (lo + 0.5 * ulp))


def quantize_on_gpu(gpu, H, W, lam, two_bit=False):
    U, hdiag, dead, rep = gpu.gptq_fold(H, lam)
    if two_bit:
        lost, tab = gpu.gptq_ladder_q2(W, dead)
        codes, rung, scale, _ = gpu.gptq_sweep_q2(W, U, hdiag, dead, tab)
    else:
        lost, tab = gpu.gptq_ladder(W, dead)
        codes, rung, scale, _ = gpu.gptq_sweep(W, U, hdiag, dead, tab, lost)
    torch.cuda.synchronize()
    return dead, codes, rung, lost, scale


def check(gpu, H, W, lam, rows_sel=None, label="", two_bit=False):
    """The debias of the GPU's own codes (4-bit, or with ``two_bit`` the q2tp ones) against the
    oracle's definition, to the bars in the module docstring."""
    dead, nib, rung, lost, scale = quantize_on_gpu(gpu, H, W, lam, two_bit)
    lost0, scale0 = lost.cpu().numpy().copy(), scale.cpu().numpy().copy()
    debias = gpu.gptq_debias_q2 if two_bit else gpu.gptq_debias
    lost_g, tab_g, scale_g, slope_g = debias(W, H, dead, nib, rung, lost, scale)
    torch.cuda.synchronize()
    Wn, Hn = W.cpu().numpy(), H.cpu().numpy()
    dn = dead.cpu().numpy().astype(bool)
    code = (oracle.unpack_q2 if two_bit else oracle.unpack_nibbles)(nib.cpu().numpy())
    rg = rung.cpu().numpy()
    sel = np.arange(Wn.shape[0]) if rows_sel is None else np.asarray(rows_sel)
    orc = oracle.debias(Wn, Hn, dn, code, rg, lost0, scale0, rows=sel, two_bit=two_bit)
    # Rounding bound of b from the f32 product W H_s.
    n = Wn.shape[1]
    Wd = np.abs(Wn[sel].astype(np.float64))
    Wd[:, dn] = 0.0
    Hs = np.abs(oracle.symmetric_from_upper(Hn, dn))
    WH = Wd @ Hs
    Wq = np.abs((oracle.dequant_q2 if two_bit else oracle.dequant)(code[sel], scale0[sel]))
    Y = (np.where(dn, 0.0, Wn[sel].astype(np.float64))) @ oracle.symmetric_from_upper(Hn, dn)
    dN = (n + 2) * U32 * np.sum(Wq * WH, 1) + 2 * U32 * np.sum(np.abs(Wq * Y), 1)
    dD = (n + 2) * U32 * np.sum(Wd * WH, 1) + 2 * U32 * np.sum(np.abs(Wd * Y), 1)
    b_o, den = orc["b"], orc["den"]
    db = (dN + np.abs(b_o) * dD) / np.abs(den) * 1.01 + 1e-300
    b_g = slope_g.cpu().numpy()[sel]
    # A row with no weight outside dead columns has num = den = 0 and no slope: both sides
    # report NaN there (and keep lo, checked below).
    undef = np.isnan(b_o)
    assert np.array_equal(np.isnan(b_g), undef), f"{label}: undefined slopes differ"
    ok = ~undef
    assert np.all(np.abs(b_g[ok] - b_o[ok]) <= db[ok]), \
        f"{label}: slope off by {np.max(np.abs(b_g[ok] - b_o[ok]) / db[ok]):.2f} x bound"
    lo_g = lost_g.cpu().numpy()[sel, 0].astype(np.float64)
    ties = 0
    for k in range(len(sel)):
        if np.isnan(orc["v"][k]):
            assert lo_g[k] == lost0[sel[k], 0], f"{label}: row {sel[k]}: kept lo changed"
            continue
        dv = db[k] / abs(b_o[k]) / np.log(2.0) + 1e-12
        if f16_boundary_distance(orc["v"][k]) > dv:
            assert lo_g[k] == orc["lo"][k], f"{label}: row {sel[k]}: lo {lo_g[k]} vs {orc['lo'][k]}"
        else:
            ties += 1
            assert abs(lo_g[k] - orc["lo"][k]) <= oracle.f16_ulp(orc["lo"][k]), label
    # TAB and scales follow the GPU's lo exactly.
    st = lost_g.cpu().numpy()[sel, 1].astype(np.float64)
    if two_bit:
        tab_x = np.float32(np.exp2(lo_g[:, None] + (np.arange(32)[None, :] - 1) * st[:, None]))
        tab_x[:, 0] = 0.0
    else:
        tab_x = np.float32(np.exp2(lo_g[:, None] + np.arange(32)[None, :] * st[:, None]))
    assert np.array_equal(tab_g.cpu().numpy()[sel], tab_x)
    assert np.array_equal(scale_g.cpu().numpy()[sel],
                          np.take_along_axis(tab_x, rg[sel].astype(np.int64) & 31, 1))
    return ties, float(np.median(b_o[ok]))


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["tiny", "fixture"])
def test_debias_small_workloads(gpu, name):
    H, W, lam = workloads.make(name, device="cuda:0")
    ties, b = check(gpu, H, W, lam, label=name)
    assert 0.5 < b < 1.5


@pytest.mark.gpu
@pytest.mark.parametrize("n,rows", [(160, 70), (288, 129)])
def test_debias_ragged(gpu, n, rows):
    H, W, lam = workloads.make("attn", device="cuda:0", n=n, rows=rows, T=1024)
    check(gpu, H, W, lam, label=f"n={n} rows={rows}")


@pytest.mark.gpu
def test_debias_down_proj_sampled(gpu):
    H, W, lam = workloads.make("down", device="cuda:0")
    sel = np.sort(np.random.default_rng(13).choice(W.shape[0], 16, replace=False))
    check(gpu, H, W, lam, rows_sel=sel, label="down")


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["tiny", "fixture"])
def test_debias_q2_small_workloads(gpu, name):
    """The 2-bit debias (the pages' primary use) on the GPU's own q2tp codes."""
    H, W, lam = workloads.make(name, device="cuda:0")
    ties, b = check(gpu, H, W, lam, label=f"q2 {name}", two_bit=True)
    assert 0.5 < b < 1.5


@pytest.mark.gpu
@pytest.mark.parametrize("n,rows", [(160, 70), (288, 129)])
def test_debias_q2_ragged(gpu, n, rows):
    H, W, lam = workloads.make("attn", device="cuda:0", n=n, rows=rows, T=1024)
    check(gpu, H, W, lam, label=f"q2 n={n} rows={rows}", two_bit=True)


@pytest.mark.gpu
def test_debias_q2_down_proj_sampled(gpu):
    H, W, lam = workloads.make("down", device="cuda:0")
    sel = np.sort(np.random.default_rng(14).choice(W.shape[0], 16, replace=False))
    check(gpu, H, W, lam, rows_sel=sel, label="q2 down", two_bit=True)
