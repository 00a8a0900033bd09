"""GPU parity at sizes the oracle finishes in seconds: the HIP path through the C ABI against
the oracle, element by element, plus the closed-form and edge cases of the method."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import (assert_sweep_bar, check_fold, check_sweep_isolated, output_error, say,
                    OUT_ERR_TOL)

pytestmark = pytest.mark.gpu


def _dev(x):
    return torch.as_tensor(np.ascontiguousarray(x)).cuda()


@pytest.mark.parametrize("name", ["tiny", "fixture"])
def test_fold_and_sweep_small_workloads(gpu, name):
    say("case", name)
    H, W, lam = workloads.make(name)
    Hd, Wd = H.cuda(), W.cuda()
    (U, hdiag, dead, rep), orc, err = check_fold(gpu, Hd, lam)
    assert rep["attempts"] == 1 and rep["lambda_used"] == lam
    st, (nib, rung, scale, E, lost, tab) = check_sweep_isolated(gpu, Wd, U, hdiag, dead)
    assert_sweep_bar(st)
    assert st["E_relF"] < 1e-4
    # End to end against the free-running oracle (its own fold, its own damping).
    Hn, Wn = H.numpy(), W.numpy()
    of = oracle.fold(Hn, lam)
    lost_o, tab_o = oracle.ladder(Wn, of["dead"])
    os_ = oracle.sweep(Wn, of["U"], of["hdiag"], of["dead"], tab_o, lost_o, want_E=False)
    t_orc = oracle.output_error(Wn, of["dead"], os_["code"], os_["scale"], Hn)
    t_gpu = output_error(Wn, of["dead"], nib.cpu().numpy(), scale.cpu().numpy(), Hn)
    say(f"{name}: tr(dW H dW^T) gpu={t_gpu:.6e} oracle={t_orc:.6e} rel={(t_gpu - t_orc) / t_orc:.2e}")
    assert abs(t_gpu - t_orc) <= OUT_ERR_TOL * t_orc


@pytest.mark.parametrize("n,rows", [(32, 1), (160, 70), (288, 130), (384, 257)])
def test_ragged_shapes(gpu, n, rows):
    """n not a multiple of the 128 block, rows not a multiple of the 64/128 row tiles."""
    say("ragged", n, rows)
    rng = np.random.default_rng(n + rows)
    X = rng.standard_normal((n, 2 * n)) * np.exp(rng.standard_normal(n))[:, None]
    H = (X @ X.T).astype(np.float32)
    H[5 % n, :] = 0.0
    H[:, 5 % n] = 0.0
    W = (rng.standard_normal((rows, n)) * 0.02).astype(np.float32)
    (U, hdiag, dead, rep), orc, err = check_fold(gpu, _dev(H), 0.01, H_np=H)
    st, _ = check_sweep_isolated(gpu, _dev(W), U, hdiag, dead)
    assert_sweep_bar(st)


@pytest.mark.parametrize("n", [150, 301, 517])
def test_fold_n_not_multiple_of_4(gpu, n):
    """The fold for any n (the sweep needs whole 32-column groups): n that is not a multiple of
    4 takes the single-float build and make-U paths, and pads to the 128 block."""
    say("fold odd n", n)
    rng = np.random.default_rng(n)
    X = rng.standard_normal((n, n + 9)) * np.exp(0.5 * rng.standard_normal(n))[:, None]
    H = (X @ X.T).astype(np.float32)
    H[n // 3, :] = 0.0
    H[:, n // 3] = 0.0
    check_fold(gpu, _dev(H), 0.01, H_np=H)


@pytest.mark.parametrize("pad", [3, 4])
def test_fold_padded_leading_dimension(gpu, pad):
    """The fold of a row-padded H (ldh = n + pad, the padding NaN and never read) is bitwise the
    fold of the contiguous H, on the float4 build path (ldh % 4 == 0) and the single-float one."""
    n, lam = 300, 0.01
    say("fold ldh", n + pad)
    rng = np.random.default_rng(11)
    X = rng.standard_normal((n, n + 40)) * np.exp(0.7 * rng.standard_normal(n))[:, None]
    H = (X @ X.T).astype(np.float32)
    U0, hd0, dead0, rep0 = gpu.gptq_fold(_dev(H), lam)
    Hp = torch.full((n, n + pad), float("nan"), dtype=torch.float32, device="cuda")
    Hp[:, :n] = _dev(H)
    view = Hp[:, :n]
    assert view.stride(0) == n + pad
    U, hd, dead, rep = gpu.gptq_fold(view, lam)
    torch.cuda.synchronize()
    assert rep["status"] == gpu.GPTQ_OK and rep0["status"] == gpu.GPTQ_OK
    assert torch.equal(U, U0) and torch.equal(hd, hd0) and torch.equal(dead, dead0)


@pytest.mark.parametrize("n,rows", [(1184, 300), (2080, 77)])
def test_ragged_multi_panel(gpu, n, rows):
    """Several fold panels and sweep panels with ragged ends: n = 1184 pads to 1280 (outer
    fold panels of 256, sweep panels 512 + 512 + 160), n = 2080 pads to 2176 (fold panels of
    512 and a last one of 128; sweep panels 4 x 512 + 32); rows not a multiple of any tile."""
    say("ragged multi-panel", n, rows)
    rng = np.random.default_rng(7 * n + rows)
    X = rng.standard_normal((n, n + 64)) * np.exp(0.8 * rng.standard_normal(n))[:, None]
    H = (X @ X.T).astype(np.float32)
    for c in (3, n // 2, n - 1):
        H[c, :] = 0.0
        H[:, c] = 0.0
    W = (rng.standard_normal((rows, n)) * 0.02).astype(np.float32)
    (U, hdiag, dead, rep), orc, err = check_fold(gpu, _dev(H), 0.01, H_np=H)
    st, _ = check_sweep_isolated(gpu, _dev(W), U, hdiag, dead)
    assert_sweep_bar(st)


def test_identity_hessian_closed_form_and_rtn(gpu):
    n, rows, lam = 256, 96, 0.01
    say("identity hessian")
    U, hdiag, dead, rep = gpu.gptq_fold(_dev(np.eye(n, dtype=np.float32)), lam)
    Ug = U.cpu().numpy()
    np.testing.assert_allclose(Ug, np.eye(n) / np.sqrt(1 + lam), rtol=1e-6, atol=1e-7)
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((rows, n)) * 0.02).astype(np.float32)
    Wd = _dev(W)
    lost, tab = gpu.gptq_ladder(Wd, dead)
    nib, rung, scale, E = gpu.gptq_sweep(Wd, U, hdiag, dead, tab, lost, want_E=True)
    code = oracle.unpack_nibbles(nib.cpu().numpy()).astype(np.int16) - 8
    sc = np.repeat(scale.cpu().numpy(), 32, axis=1)
    # U is diagonal, so the feedback adds nothing and the codes are plain rounding at the
    # chosen scale, bit for bit.
    np.testing.assert_array_equal(code, np.clip(np.rint(W / sc), -8, 7).astype(np.int16))


def test_retry_and_degenerate_cases(gpu):
    say("retry cases")
    # [[1,1],[1,1]]: singular at 0.  The f32 attempt fails, the same damping fails in f64, and
    # 1e-4 factors in f64: the damping the f64 host fold reaches.
    U, hd, dd, rep = gpu.gptq_fold(_dev(np.array([[1, 1], [1, 1]], np.float32)), 0.0)
    orc = oracle.fold(np.array([[1, 1], [1, 1]], np.float32), 0.0)
    assert orc["lam"] == 1e-4
    assert rep["status"] == 0 and rep["lambda_used"] == orc["lam"], rep
    assert rep["attempts"] == 3 and rep["precision"] == 64, rep
    # The pages' f32 device rule alone reaches the same damping here.
    U, hd, dd, rep = gpu.gptq_fold(_dev(np.array([[1, 1], [1, 1]], np.float32)), 0.0, precision="f32")
    assert rep["status"] == 0 and rep["lambda_used"] == 1e-4 and rep["precision"] == 32, rep
    # [[1,20],[20,1]] cannot be damped into a factor below 10: U = I, DEGENERATE.
    U, hd, dd, rep = gpu.gptq_fold(_dev(np.array([[1, 20], [20, 1]], np.float32)), 0.01)
    assert rep["status"] == 4 and rep["degenerate"] == 1
    np.testing.assert_array_equal(U.cpu().numpy(), np.eye(2, dtype=np.float32))
    # A NaN off-diagonal fails every attempt.
    rng = np.random.default_rng(3)
    X = rng.standard_normal((64, 200))
    H = (X @ X.T).astype(np.float32)
    H[3, 40] = np.nan
    U, hd, dd, rep = gpu.gptq_fold(_dev(H), 0.01)
    assert rep["status"] == 4
    assert oracle.fold(H, 0.01)["status"] == oracle.DEGENERATE
    # Dead channels: zero, negative and NaN diagonals.
    H = (X @ X.T).astype(np.float32)
    H[7, :] = 0.0
    H[:, 7] = 0.0
    H[9, 9] = -2.0
    H[11, 11] = np.nan
    (U, hd, dd, rep), orc, err = check_fold(gpu, _dev(H), 0.01, H_np=H)
    assert rep["n_dead"] == 3


@pytest.mark.parametrize("precision", ["auto", "f64"])
def test_fold_reads_only_the_upper_triangle(gpu, precision):
    """Garbage below H's diagonal (NaN, inf, huge values) changes nothing: U is bit-identical to
    the fold of the symmetric matrix, in both arithmetics."""
    say(f"upper triangle only ({precision})")
    rng = np.random.default_rng(5)
    n = 300
    X = rng.standard_normal((n, 500)) * np.exp(rng.standard_normal(n))[:, None]
    H = (X @ X.T).astype(np.float32)
    Hg = H.copy()
    il = np.tril_indices(n, -1)
    junk = rng.choice(np.array([np.nan, np.inf, -np.inf, 1e30, -7.0], np.float32), size=il[0].size)
    Hg[il] = junk
    U0, hd0, dd0, r0 = gpu.gptq_fold(_dev(H), 0.01, precision=precision)
    U1, hd1, dd1, r1 = gpu.gptq_fold(_dev(Hg), 0.01, precision=precision)
    torch.cuda.synchronize()
    assert r0["status"] == r1["status"] == 0
    assert torch.equal(U0, U1) and torch.equal(hd0, hd1) and torch.equal(dd0, dd1)


def test_invalid_arguments_write_nothing(gpu):
    say("invalid arguments")
    lib = gpu.load()
    assert lib.gptq_fold_workspace_size(0) == 0
    H = _dev(np.eye(64, dtype=np.float32))
    U = torch.full((64, 64), 7.0, device="cuda")
    hd = torch.zeros(64, device="cuda")
    dd = torch.zeros(64, dtype=torch.uint8, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):  # the binding checks the size first
        gpu.gptq_fold(H, 0.01, workspace=ws, out=(U, hd, dd))
    import ctypes
    P = ctypes.c_void_p
    rep = gpu.FoldReport()
    st = lib.gptq_fold(P(H.data_ptr()), 64, 64, 0.01, P(U.data_ptr()), P(hd.data_ptr()),
                       P(dd.data_ptr()), P(ws.data_ptr()), ws.numel(), None, ctypes.byref(rep))
    torch.cuda.synchronize()
    assert st == gpu.GPTQ_EWORKSPACE
    assert torch.all(U == 7.0)
    with pytest.raises(ValueError):  # U of the wrong shape never reaches the library
        gpu.gptq_fold(H, 0.01, out=(torch.empty(64, 63, device="cuda"), hd, dd))
    W = torch.zeros(4, 48, device="cuda")  # n % 32 != 0
    with pytest.raises(gpu.GptqError):
        gpu.gptq_ladder(W, torch.zeros(48, dtype=torch.uint8, device="cuda"))


def test_repeat_runs_are_bitwise_identical(gpu):
    say("determinism")
    H, W, lam = workloads.make("tiny")
    Hd, Wd = H.cuda(), W.cuda()
    outs = []
    for _ in range(2):
        U, hd, dd, rep = gpu.gptq_fold(Hd, lam)
        lost, tab = gpu.gptq_ladder(Wd, dd)
        nib, rung, scale, E = gpu.gptq_sweep(Wd, U, hd, dd, tab, lost, want_E=True)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (U, nib, rung, scale, E)])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


def test_profile_counts_the_fold_bulk_updates(gpu):
    """The event timing behind the benchmark's roofline: at n = 2080 (padded to 2176, outer
    panels of 512) the f32 fold's bulk family is the Cholesky's trailing update beyond the next panel
    (3 launches) and the inverse's update of the rows below each panel (4 launches), with the
    flops of their definitions; every launch is timed."""
    n, lam = 2080, 0.01
    rng = np.random.default_rng(3)
    X = rng.standard_normal((n, n + 64))
    H = (X @ X.T).astype(np.float32)
    Hd = _dev(H)
    gpu.gptq_fold(Hd, lam, precision="f32")  # warm
    torch.cuda.synchronize()
    gpu.profile_collect()
    gpu.profile_enable(["fold_update"])
    try:
        gpu.gptq_fold(Hd, lam, precision="f32")
        torch.cuda.synchronize()
    finally:
        gpu.profile_enable([])
    fu = gpu.profile_collect()["fold_update"]
    np_, nb2 = 2176, 512
    launches, flops = 0, 0.0
    for kb in range(0, np_, nb2):
        w = min(nb2, np_ - kb)
        rest = np_ - kb - w
        if rest <= 0:
            continue
        rest2 = rest - min(nb2, rest)
        if rest2 > 0:
            launches += 1
            flops += w * rest2 * (rest2 + 1)  # lower triangle of a rank-w update
        launches += 1
        flops += 2.0 * w * rest * (kb + w)
    assert fu["launches"] == launches == 7
    assert fu["flops"] == pytest.approx(flops, rel=1e-12)
    tflops = fu["flops"] / (fu["ms"] * 1e-3) / 1e12
    say(f"fold_update at n={n}: {fu['launches']} launches, {fu['ms']:.3f} ms, {tflops:.1f} TFLOP/s")
    assert 0.0 < tflops < 157.3


@pytest.mark.parametrize("n,rows,want_e", [(256, 512, False), (256, 512, True), (1184, 300, False),
                                           (2080, 77, True)])
def test_sweep_inplace_matches_sweep(gpu, n, rows, want_e):
    """The in-place sweep gives gptq_sweep's codes, rungs, scales and residuals bit for bit
    (several 512-column panels and ragged rows included)."""
    say("sweep in place", n, rows, want_e)
    rng = np.random.default_rng(n + rows)
    X = rng.standard_normal((n, 2 * n)) * np.exp(rng.standard_normal(n))[:, None]
    H = (X @ X.T).astype(np.float32)
    W = (rng.standard_normal((rows, n)) * 0.02).astype(np.float32)
    U, hd, dd, rep = gpu.gptq_fold(_dev(H), 0.01)
    Wd = _dev(W)
    lost, tab = gpu.gptq_ladder(Wd, dd)
    a = gpu.gptq_sweep(Wd, U, hd, dd, tab, lost, want_E=want_e)
    Wi = Wd.clone()
    b = gpu.gptq_sweep_inplace(Wi, U, hd, dd, tab, lost, want_E=want_e)
    torch.cuda.synchronize()
    assert torch.equal(Wd, _dev(W))  # gptq_sweep leaves W alone
    for x, y in zip(a, b):
        if x is not None:
            assert torch.equal(x, y)


def test_misaligned_pointers_are_rejected(gpu):
    """Pointers the kernels read or write as float4 rows must be 16-byte aligned: a W, U, E or
    workspace four bytes off is refused with GPTQ_EINVAL before anything is written."""
    import ctypes
    lib = gpu.load()
    P = ctypes.c_void_p
    rows, n = 8, 64
    rng = np.random.default_rng(1)
    X = rng.standard_normal((n, 2 * n))
    Hd = _dev((X @ X.T).astype(np.float32))
    U, hd, dd, rep = gpu.gptq_fold(Hd, 0.01)
    Wbuf = _dev(np.concatenate([[0.0], (rng.standard_normal(rows * n) * 0.02)]).astype(np.float32))
    W_off = P(Wbuf.data_ptr() + 4)           # rows of W four bytes off
    W_ok = Wbuf[1:].clone()
    lost, tab = gpu.gptq_ladder(W_ok.view(rows, n), dd)
    nib = torch.full((rows, n // 2), 0xAB, dtype=torch.uint8, device="cuda")
    rung = torch.full((rows, n // 32), 0xCD, dtype=torch.uint8, device="cuda")
    scale = torch.full((rows, n // 32), 3.0, device="cuda")
    ws = torch.empty(lib.gptq_sweep_workspace_size(rows, n) + 64, dtype=torch.uint8, device="cuda")
    Ubuf = torch.empty(n * n + 4, device="cuda")
    Ubuf[1:n * n + 1].copy_(U.flatten())
    p = lambda t: P(t.data_ptr())
    args = lambda w, u, wsp: (w, u, p(hd), p(dd), p(tab), p(lost), rows, n, p(nib), p(rung),
                              p(scale), None, wsp, ws.numel() - 64, None)
    assert lib.gptq_sweep(*args(W_off, p(U), p(ws))) == gpu.GPTQ_EINVAL
    assert lib.gptq_sweep(*args(p(W_ok), P(Ubuf.data_ptr() + 4), p(ws))) == gpu.GPTQ_EINVAL
    assert lib.gptq_sweep(*args(p(W_ok), p(U), P(ws.data_ptr() + 4))) == gpu.GPTQ_EINVAL
    assert lib.gptq_sweep_inplace(*args(W_off, p(U), p(ws))) == gpu.GPTQ_EINVAL
    assert lib.gptq_sweep_q2(W_off, p(U), p(hd), p(dd), p(tab), rows, n, p(nib), p(rung), p(scale),
                             None, p(ws), ws.numel() - 64, None) == gpu.GPTQ_EINVAL
    assert lib.gptq_ladder(W_off, p(dd), rows, n, p(lost), p(tab), None) == gpu.GPTQ_EINVAL
    rep = gpu.FoldReport()
    wsf = torch.empty(gpu.fold_workspace_size(n) + 64, dtype=torch.uint8, device="cuda")
    Uo = torch.full((n, n), 7.0, device="cuda")
    assert lib.gptq_fold(p(Hd), n, n, 0.01, p(Uo), p(hd), p(dd), P(wsf.data_ptr() + 4),
                         wsf.numel() - 64, None, ctypes.byref(rep)) == gpu.GPTQ_EINVAL
    torch.cuda.synchronize()
    assert torch.all(nib == 0xAB) and torch.all(rung == 0xCD) and torch.all(scale == 3.0)
    assert torch.all(Uo == 7.0)
    # The same call with aligned pointers runs.
    assert lib.gptq_sweep(*args(p(W_ok), p(U), p(ws))) == gpu.GPTQ_OK
    torch.cuda.synchronize()


def test_calls_on_a_stream_that_is_not_current(gpu):
    """Every wrapper given stream= while another stream is current: its outputs and workspaces
    are allocated in that stream's order (the caching allocator churns on the current stream
    meanwhile), and the results equal those of the same calls on the current stream."""
    H, W, lam = workloads.make("fixture", device="cuda")

    def chain(stream):
        U, hd, dd, rep = gpu.gptq_fold(H, lam, stream=stream)
        lost, tab = gpu.gptq_ladder(W, dd, stream=stream)
        nib, rung, scale, E = gpu.gptq_sweep(W, U, hd, dd, tab, lost, want_E=True, stream=stream)
        lq, tq = gpu.gptq_ladder_q2(W, dd, stream=stream)
        plane, rq, sq, _ = gpu.gptq_sweep_q2(W, U, hd, dd, tq, stream=stream)
        lost_d, tab_d, scale_d, slope = gpu.gptq_debias(W, H, dd, nib, rung, lost.clone(), scale.clone(),
                                                        stream=stream)
        perm, dead_p = gpu.gptq_act_order_perm(H, stream=stream)
        return [U, hd, dd, lost, tab, nib, rung, scale, E, lq, tq, plane, rq, sq, lost_d, scale_d,
                perm, dead_p]

    ref = chain(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = chain(side)
    for _ in range(32):  # reuse of freed blocks on the current stream while side may still run
        torch.empty(1 << 22, device="cuda").fill_(float("nan"))
    side.synchronize()
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(got, ref)):
        assert torch.equal(a, b), f"output {i} differs on the side stream"
