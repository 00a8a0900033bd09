"""The library's launch schedules, checked on the CPU by its dry-run mode (include/gptq_check.h):
every kernel's reads and writes stay inside the buffers of the call, and no two launches on
different streams touch the same memory unordered.  The fold runs on three streams (serial
chain, Cholesky bulk update, inverse pipeline) and the sweep on two, so these checks cover the
event waits between them at the sizes the GPU runs, ragged sizes included."""
import ctypes

import pytest

import post_weight_quantization_amd as pwq

GPTQ_OK, GPTQ_ECHECK = pwq.GPTQ_OK, pwq.GPTQ_ECHECK
P = ctypes.c_void_p
BASE = 1 << 44          # fake device addresses: never dereferenced in a dry run
STRIDE = 1 << 38


def addrs(k):
    return [P(BASE + i * STRIDE) for i in range(k)]


@pytest.fixture(scope="module")
def lib():
    return pwq.load()


@pytest.mark.parametrize("lower", [False, True])
def test_gemm_tile_order_is_a_bijection(lib, lower):
    """Every workgroup of a tile GEMM launch gets a distinct tile and every tile is taken: square
    and ragged tile grids, grids narrower and wider than a super-tile, and the shapes the fold
    (lower trailing blocks at n = 17408) and the sweep (5120 rows) launch."""
    shapes = [(1, 1), (128, 128), (129, 4000), (1000, 100), (1024, 1024), (1152, 1152),
              (5120, 17408 - 512), (5120, 384), (17408 - 512, 17408 - 512), (17408 - 1024, 512),
              (3 * 128, 37 * 128), (9 * 128 + 5, 17 * 128 - 3)]
    shapes += [(m * 128, n * 128) for m in range(1, 20) for n in (1, 7, 8, 9, 23)]
    for M, N in shapes:
        assert pwq.check_tile_order(M, N, lower) == GPTQ_OK, (M, N, lower)
    if lower:
        for T in range(1, 140):
            assert pwq.check_tile_order(T * 128, 0 + 1, True) == GPTQ_OK, T
    assert pwq.check_tile_order(0, 5, lower) != GPTQ_OK


def test_checker_selftest(lib):
    assert pwq.check_selftest(0) == GPTQ_OK
    assert pwq.check_selftest(1) == GPTQ_ECHECK
    assert "race" in pwq.check_message()
    assert pwq.check_selftest(2) == GPTQ_OK
    assert pwq.check_selftest(3) == GPTQ_ECHECK
    assert "bounds" in pwq.check_message()


@pytest.mark.parametrize("n", [8, 96, 128, 256, 600, 1024, 2048, 2080, 4096, 8192, 17408])
@pytest.mark.parametrize("precision", ["auto", "f32", "f64"])
def test_fold_schedule(lib, n, precision):
    """Each precision's schedule with the workspace its size query asks for (the f32 one is
    smaller: the f64 one overlays the f32 matrices and adds an f64 inverse)."""
    H, U, hd, dead, ws = addrs(5)
    prec = pwq.FOLD_PRECISION[precision]
    need = lib.gptq_fold_workspace_size_ex(n, prec)
    rep = pwq.FoldReport()
    with pwq.check_mode():
        st = lib.gptq_fold_ex(H, n, n, 0.01, prec, U, hd, dead, ws, need, None, ctypes.byref(rep))
    assert st == GPTQ_OK, pwq.check_message()
    assert pwq.check_message() == ""
    assert rep.precision == (64 if precision == "f64" else 32)
    if precision == "f32":
        assert need < lib.gptq_fold_workspace_size(n)
    else:
        assert need == lib.gptq_fold_workspace_size(n)
        with pwq.check_mode():
            st = lib.gptq_fold_ex(H, n, n, 0.01, prec, U, hd, dead, ws,
                                  lib.gptq_fold_workspace_size_ex(n, 1), None, ctypes.byref(rep))
        assert st == pwq.GPTQ_EWORKSPACE


def test_fold_rejects_unknown_precision(lib):
    H, U, hd, dead, ws = addrs(5)
    rep = pwq.FoldReport()
    assert lib.gptq_fold_workspace_size_ex(64, 3) == 0
    with pwq.check_mode():
        st = lib.gptq_fold_ex(H, 64, 64, 0.01, 3, U, hd, dead, ws, 1 << 30, None, ctypes.byref(rep))
    assert st == pwq.GPTQ_EINVAL


def test_fold_schedule_padded_rows_of_h(lib):
    H, U, hd, dead, ws = addrs(5)
    n = 1000
    rep = pwq.FoldReport()
    with pwq.check_mode():
        st = lib.gptq_fold(H, n, 1024, 0.0, U, hd, dead, ws, lib.gptq_fold_workspace_size(n),
                           None, ctypes.byref(rep))
    assert st == GPTQ_OK, pwq.check_message()


@pytest.mark.parametrize("rows,n", [(16, 32), (37, 96), (512, 256), (100, 544), (300, 1056),
                                    (4096, 4096), (2048, 8192), (5120, 17408)])
@pytest.mark.parametrize("want_e", [False, True])
def test_sweep_schedule(lib, rows, n, want_e):
    W, U, hd, dead, tab, lost, nib, rung, scale, E, ws = addrs(11)
    need = lib.gptq_sweep_workspace_size(rows, n)
    with pwq.check_mode():
        st = lib.gptq_sweep(W, U, hd, dead, tab, lost, rows, n, nib, rung, scale,
                            E if want_e else None, ws, need, None)
    assert st == GPTQ_OK, pwq.check_message()


@pytest.mark.parametrize("rows,n", [(1, 32), (512, 256), (5120, 17408)])
def test_ladder_schedule(lib, rows, n):
    W, dead, lost, tab = addrs(4)
    with pwq.check_mode():
        st = lib.gptq_ladder(W, dead, rows, n, lost, tab, None)
    assert st == GPTQ_OK, pwq.check_message()


def test_undersized_buffers_are_caught(lib):
    """A caller's workspace is checked by size before anything runs; the dry run's own bounds
    check then sees every launch inside the buffers it was given."""
    H, U, hd, dead, ws = addrs(5)
    n = 512
    rep = pwq.FoldReport()
    with pwq.check_mode():
        st = lib.gptq_fold(H, n, n, 0.01, U, hd, dead, ws, lib.gptq_fold_workspace_size(n) - 1,
                           None, ctypes.byref(rep))
    assert st == pwq.GPTQ_EWORKSPACE


@pytest.mark.parametrize("n,t", [(4, 1), (200, 777), (4096, 8192), (17408, 32768)])
def test_gram_schedule(lib, n, t):
    H, X = addrs(2)
    with pwq.check_mode():
        st = lib.gptq_gram_add(H, n, n, X, t, n, None)
    assert st == GPTQ_OK, pwq.check_message()


@pytest.mark.parametrize("rows,n", [(1, 32), (70, 160), (5120, 17408)])
def test_debias_schedule(lib, rows, n):
    W, H, dead, nib, rung, lost, tab, scale, slope, ws = addrs(10)
    need = lib.gptq_debias_workspace_size(rows, n)
    with pwq.check_mode():
        st = lib.gptq_debias(W, H, n, dead, nib, rung, lost, tab, scale, slope, rows, n, ws,
                             need, None)
    assert st == GPTQ_OK, pwq.check_message()


@pytest.mark.parametrize("rows,n", [(1, 32), (37, 96), (300, 1056), (4096, 4096), (5120, 17408)])
@pytest.mark.parametrize("want_e", [False, True])
def test_act_order_schedule(lib, rows, n, want_e):
    W, U, dead, perm, tab, lost, nib, rung, scale, E, ws, H, Hp = addrs(13)
    need = lib.gptq_sweep_act_order_workspace_size(rows, n)
    with pwq.check_mode():
        st = lib.gptq_act_order_perm(H, n, n, perm, dead, None)
        assert st == GPTQ_OK, pwq.check_message()
        st = lib.gptq_permute_hessian(H, n, n, perm, Hp, None)
        assert st == GPTQ_OK, pwq.check_message()
        st = lib.gptq_sweep_act_order(W, U, dead, perm, tab, lost, rows, n, nib, rung, scale,
                                      E if want_e else None, ws, need, None)
    assert st == GPTQ_OK, pwq.check_message()


@pytest.mark.parametrize("rows,n", [(16, 32), (37, 96), (300, 1056), (5120, 17408)])
@pytest.mark.parametrize("want_e", [False, True])
def test_q2_schedule(lib, rows, n, want_e):
    W, U, hd, dead, tab, lost, plane, rung, scale, E, ws = addrs(11)
    need = lib.gptq_sweep_workspace_size(rows, n)
    with pwq.check_mode():
        st = lib.gptq_ladder_q2(W, dead, rows, n, lost, tab, None)
        assert st == GPTQ_OK, pwq.check_message()
        st = lib.gptq_sweep_q2(W, U, hd, dead, tab, rows, n, plane, rung, scale,
                               E if want_e else None, ws, need, None)
    assert st == GPTQ_OK, pwq.check_message()


@pytest.mark.parametrize("rows,n", [(16, 32), (37, 96), (300, 1056), (4096, 4096), (5120, 17408)])
@pytest.mark.parametrize("want_e", [False, True])
def test_sweep_inplace_schedule(lib, rows, n, want_e):
    """W is its own working copy: every launch stays inside W, the outputs and the panel
    workspace (none with E), and the helper stream's updates never race the chain's."""
    W, U, hd, dead, tab, lost, nib, rung, scale, E, ws = addrs(11)
    need = lib.gptq_sweep_inplace_workspace_size(rows, n)
    assert need < lib.gptq_sweep_workspace_size(rows, n)
    with pwq.check_mode():
        st = lib.gptq_sweep_inplace(W, U, hd, dead, tab, lost, rows, n, nib, rung, scale,
                                    E if want_e else None, None if want_e else ws,
                                    0 if want_e else need, None)
    assert st == GPTQ_OK, pwq.check_message()


@pytest.mark.parametrize("rows,n", [(16, 32), (300, 1056), (5120, 17408), (8192, 4096)])
@pytest.mark.parametrize("want_e", [False, True])
def test_sweep_inplace_noalloc_schedule(lib, rows, n, want_e):
    """The no-allocation sweep: one stream, the residual panels in the static scratch (a
    stand-in address in a dry run), every launch inside the call's buffers."""
    W, U, hd, dead, tab, lost, nib, rung, scale, E = addrs(10)
    with pwq.check_mode():
        st = lib.gptq_sweep_inplace_noalloc(W, U, hd, dead, tab, lost, rows, n, nib, rung, scale,
                                            E if want_e else None, None)
    assert st == GPTQ_OK, pwq.check_message()
    with pwq.check_mode():
        st = lib.gptq_sweep_inplace_noalloc(W, U, hd, dead, tab, lost, 8193, n, nib, rung, scale,
                                            None, None)
    assert st == pwq.GPTQ_ETOOBIG


@pytest.mark.parametrize("rows,n", [(1, 32), (37, 96), (300, 1056), (5120, 17408)])
@pytest.mark.parametrize("want_e", [False, True])
def test_act_order_q2_schedule(lib, rows, n, want_e):
    W, U, dead, hd, perm, tab, plane, rung, scale, E, ws = addrs(11)
    need = lib.gptq_sweep_act_order_workspace_size(rows, n)
    with pwq.check_mode():
        st = lib.gptq_sweep_act_order_q2(W, U, dead, hd, perm, tab, rows, n, plane, rung, scale,
                                         E if want_e else None, ws, need, None)
    assert st == GPTQ_OK, pwq.check_message()


@pytest.mark.parametrize("rows,n", [(1, 32), (70, 160), (5120, 17408)])
def test_debias_q2_schedule(lib, rows, n):
    W, H, dead, plane, rung, lost, tab, scale, slope, ws = addrs(10)
    need = lib.gptq_debias_workspace_size(rows, n)
    with pwq.check_mode():
        st = lib.gptq_debias_q2(W, H, n, dead, plane, rung, lost, tab, scale, slope, rows, n, ws,
                                need, None)
    assert st == GPTQ_OK, pwq.check_message()


PACKED = pwq.GPTQ_PACKED_UPPER


@pytest.mark.parametrize("n", [1, 8, 301, 4096, 17408])
@pytest.mark.parametrize("precision", ["auto", "f32", "f64"])
def test_fold_schedule_packed_hessian(lib, n, precision):
    """H as its packed upper triangle (n (n + 1) / 2 floats): every read of H lies inside it."""
    H, U, hd, dead, ws = addrs(5)
    prec = pwq.FOLD_PRECISION[precision]
    rep = pwq.FoldReport()
    with pwq.check_mode():
        st = lib.gptq_fold_ex(H, n, PACKED, 0.01, prec, U, hd, dead, ws,
                              lib.gptq_fold_workspace_size_ex(n, prec), None, ctypes.byref(rep))
    assert st == GPTQ_OK, pwq.check_message()


@pytest.mark.parametrize("n,t", [(4, 1), (200, 777), (17408, 32768)])
def test_gram_schedule_packed(lib, n, t):
    H, X = addrs(2)
    with pwq.check_mode():
        st = lib.gptq_gram_add(H, n, PACKED, X, t, n, None)
    assert st == GPTQ_OK, pwq.check_message()


@pytest.mark.parametrize("rows,n", [(1, 32), (5120, 17408)])
def test_debias_and_act_order_schedules_packed(lib, rows, n):
    W, H, dead, nib, rung, lost, tab, scale, slope, ws, perm, Hp = addrs(12)
    need = lib.gptq_debias_workspace_size(rows, n)
    with pwq.check_mode():
        st = lib.gptq_debias(W, H, PACKED, dead, nib, rung, lost, tab, scale, slope, rows, n, ws,
                             need, None)
    assert st == GPTQ_OK, pwq.check_message()
    with pwq.check_mode():
        st = lib.gptq_debias_q2(W, H, PACKED, dead, nib, rung, lost, tab, scale, slope, rows, n,
                                ws, need, None)
    assert st == GPTQ_OK, pwq.check_message()
    with pwq.check_mode():
        st = lib.gptq_act_order_perm(H, n, PACKED, perm, dead, None)
    assert st == GPTQ_OK, pwq.check_message()
    with pwq.check_mode():
        st = lib.gptq_permute_hessian(H, n, PACKED, perm, Hp, None)
    assert st == GPTQ_OK, pwq.check_message()


def test_hessian_leading_dimension_is_checked(lib):
    """ldh below n, or negative other than the packed marker, is refused before anything runs."""
    H, U, hd, dead, ws, X, perm, Hp = addrs(8)
    n = 64
    rep = pwq.FoldReport()
    for ldh in (n - 1, -2, 0):
        with pwq.check_mode():
            assert lib.gptq_fold(H, n, ldh, 0.01, U, hd, dead, ws, lib.gptq_fold_workspace_size(n),
                                 None, ctypes.byref(rep)) == pwq.GPTQ_EINVAL
            assert lib.gptq_gram_add(H, n, ldh, X, 16, n, None) == pwq.GPTQ_EINVAL
            assert lib.gptq_act_order_perm(H, n, ldh, perm, dead, None) == pwq.GPTQ_EINVAL
            assert lib.gptq_permute_hessian(H, n, ldh, perm, Hp, None) == pwq.GPTQ_EINVAL
