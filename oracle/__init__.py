"""CPU oracle of the GPTQ fold and the q4tp sweep (f64; plain C behind ctypes).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The product library never links, loads or calls
it, and this package imports nothing from the product package.

What each function follows (docs.rs source pages of the cortiq project):

* :func:`fold` -- "cortiq-cli 0.8.45 src/gptq.rs", ``gptq_fold_operator_par``: dead channels,
  damping ``lambda * mean(diag)``, the x10 retry, ``U`` = upper Cholesky factor of ``H_d^-1``,
  computed from that definition as ``J chol(J H_d J)^-1 J`` (see the C source).
* :func:`ladder` -- the per-row rung ladder; the pages take it from a converter whose rule is
  not printed, so the rule here is a stated reading (see the C source).
* :func:`sweep` -- "cortiq-cli 0.8.45 src/gptq.rs", ``gptq_quantize_q4tp``, and
  "cortiq-engine 0.8.41 src/gpu_wgpu/gptq_dev.rs", ``q4tp_group``: rung rule, rounding and
  column-by-column error feedback.
* :func:`gram` -- the device Hessian's accumulation ``H += X^T X`` over the rows (tokens) of an
  activation matrix ``X [t, n]`` ("cortiq-cli 0.8.45 src/gptq.rs": calibration's
  ``gram_add_dev`` and the test ``device_fold_and_sweep_match_host``, which accumulates
  ``h[i][j] += x[r][i] x[r][j]``), in f64 from the f32 inputs.
* :func:`debias` -- the output debias ("cortiq-cli 0.8.45 src/gptq.rs", ``q4tp_debias_hessian``
  and its GEMM form ``debias_gemm``): per row the slope ``b = (W^ H W^T)_rr / (W H W^T)_rr``
  removed through the row's f16 ``lo``.  The helper that applies ``b`` is not printed; the
  reading is ``lo <- f16(lo - log2 b)``, kept unless num and den are positive and finite.
* :func:`act_order_perm`, :func:`sweep_act_order` -- act-order GPTQ ("cortiq-cli 0.8.45
  src/gptq.rs", ``act_order_perm``, ``permute_sym``, ``gptq_quantize_q4tp_act_order``): channels
  in descending ``H_ii`` (total order, ties by index), the fold of ``H[perm][perm]``, static
  rungs chosen up front from the original tiles, columns eliminated in ``perm`` order.  The
  converter's rung choice is not printed; the reading is the sweep's rung rule on the
  dead-zeroed original tile with unit weights.
* :func:`static_rungs_q2` and :func:`sweep_act_order` with ``two_bit`` -- act order for q2tp
  ("cortiq-cli 0.8.45 src/gptq.rs", ``gptq_quantize_q2tp`` with ``perm``): the rungs fixed up
  front, 2-bit levels in elimination order.  The placement helper that fixes them is not
  printed; the reading is the sweep's full rung search on the dead-zeroed original tile with the
  clipped ``H_ii`` weights.  :func:`debias` with ``two_bit`` is ``q2tp_debias_hessian``.
* :func:`ladder_q2`, :func:`sweep_q2` -- the q2tp sweep with the "placed" rule ("cortiq-engine
  0.8.41 src/gpu_wgpu/gptq_dev.rs", ``q2tp_group``; "cortiq-cli 0.8.45 src/gptq.rs",
  ``sweep_q2tp``, ``gptq_quantize_q2tp``): 2-bit levels, a full search over rungs 1..31 by the
  clipped-``H_ii``-weighted error, rung 0 for an all-zero group.  The ladder placement is not
  printed; the ladder here is a stated reading (see the C source).
* :func:`output_error` -- the layer-output error ``tr(dW H dW^T)`` with the raw Hessian, the
  quantity the pages' device-versus-host test compares ("cortiq-cli 0.8.45 src/gptq.rs",
  test ``device_fold_and_sweep_match_host``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gptq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_gptq.so")
_lib = None

OK, FAILED, DEGENERATE = 0, 1, 4


def build() -> str:
    """Compile the oracle with gcc (no multiply-add contraction, OpenMP)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(
        ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
         "-Wall", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.orc_fold.argtypes = [P, i64, i64, ctypes.c_double, ctypes.c_int, ctypes.c_int,
                             P, P, P, P, ctypes.c_int]
    lib.orc_fold.restype = ctypes.c_int
    lib.orc_ladder.argtypes = [P, P, i64, i64, i64, P, P]
    lib.orc_ladder.restype = None
    lib.orc_sweep_static.argtypes = [P, i64, i64, P, P, ctypes.c_int, P, P, P, ctypes.c_double, P,
                                     ctypes.c_int]
    lib.orc_sweep_static.restype = ctypes.c_int
    lib.orc_ladder_q2.argtypes = [P, P, i64, i64, i64, P, P]
    lib.orc_ladder_q2.restype = None
    lib.orc_sweep_q2.argtypes = [P, i64, i64, i64, P, P, P, P, P, P, P, P, P, P,
                                 ctypes.c_double, ctypes.c_double, P, ctypes.c_int]
    lib.orc_sweep_q2.restype = ctypes.c_int
    lib.orc_sweep.argtypes = [P, i64, i64, i64, P, P, P, P, P, P, P, P, P, P, P, P,
                              ctypes.c_double, ctypes.c_double, P, ctypes.c_int]
    lib.orc_sweep.restype = ctypes.c_int
    lib.orc_f16_round.argtypes = [ctypes.c_double]
    lib.orc_f16_round.restype = ctypes.c_double
    lib.orc_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def threads(nt=None) -> int:
    return int(nt) if nt else int(_load().orc_max_threads())


def fold(H, lam, retry=True, route=0, nt=None):
    """Fold ``H`` (f32, ``n x ldh``; the upper triangle is read) at starting damping ``lam``.

    ``route`` 0 computes U = J chol(J H_d J)^-1 J (J the order reversal), the definition
    solved for U; route 1 does the same on the equilibrated matrix (a cross-check with other
    rounding).  Returns a dict with ``U`` (f64, upper),
    ``hdiag`` (f32), ``dead`` (bool), ``lam``, ``base``, ``damp``, ``attempts``, ``status``.
    """
    H = np.ascontiguousarray(H, dtype=np.float32)
    n = H.shape[0]
    U = np.empty((n, n), dtype=np.float64)
    hdiag = np.empty(n, dtype=np.float32)
    dead = np.empty(n, dtype=np.uint8)
    info = np.zeros(4, dtype=np.float64)
    st = _load().orc_fold(_ptr(H), n, H.shape[1], float(lam), int(bool(retry)), int(route),
                          _ptr(U), _ptr(hdiag), _ptr(dead), _ptr(info), threads(nt))
    return dict(U=U, hdiag=hdiag, dead=dead.astype(bool), lam=float(info[0]),
                base=float(info[1]), damp=float(info[2]), attempts=int(info[3]), status=st)


def ladder(W0, dead, gs=32):
    """Per-row ``lost`` (rows x 2: lo, step) and ``tab`` (rows x 32) from the dead-zeroed W0."""
    W0 = np.ascontiguousarray(W0, dtype=np.float32)
    rows, n = W0.shape
    d = np.ascontiguousarray(dead, dtype=np.uint8)
    lost = np.empty((rows, 2), dtype=np.float32)
    tab = np.empty((rows, 32), dtype=np.float32)
    _load().orc_ladder(_ptr(W0), _ptr(d), rows, n, gs, _ptr(lost), _ptr(tab))
    return lost, tab


def sweep(W0, U, hdiag, dead, tab, lost, gs=32, force_code=None, force_rung=None,
          tie_band=1e-3, rung_band=1e-4, want_E=True, want_Wc=False, nt=None):
    """Column-sequential q4tp sweep.  ``code`` holds ``q + 8`` one per byte (rows x n).

    With ``force_code`` / ``force_rung`` (another implementation's decisions) the sweep runs
    as a tie-forced replay and ``stats`` counts {code ties, code hard, rung ties, rung hard}.
    """
    W0 = np.ascontiguousarray(W0, dtype=np.float32)
    rows, n = W0.shape
    U = np.ascontiguousarray(U, dtype=np.float64)
    hdiag = np.ascontiguousarray(hdiag, dtype=np.float32)
    d = np.ascontiguousarray(dead, dtype=np.uint8)
    tab = np.ascontiguousarray(tab, dtype=np.float32)
    lost = np.ascontiguousarray(lost, dtype=np.float32)
    ng = n // gs
    code = np.empty((rows, n), dtype=np.uint8)
    rung = np.empty((rows, ng), dtype=np.uint8)
    scale = np.empty((rows, ng), dtype=np.float32)
    E = np.empty((rows, n), dtype=np.float64) if want_E else None
    Wc = np.empty((rows, n), dtype=np.float64) if want_Wc else None
    fc = None if force_code is None else np.ascontiguousarray(force_code, dtype=np.uint8)
    fr = None if force_rung is None else np.ascontiguousarray(force_rung, dtype=np.uint8)
    stats = np.zeros(4, dtype=np.int64)
    st = _load().orc_sweep(_ptr(W0), rows, n, gs, _ptr(U), _ptr(hdiag), _ptr(d), _ptr(tab),
                           _ptr(lost), _ptr(code), _ptr(rung), _ptr(scale), _ptr(E), _ptr(Wc),
                           _ptr(fc), _ptr(fr), float(tie_band), float(rung_band), _ptr(stats),
                           threads(nt))
    if st != OK:
        raise ValueError("oracle sweep rejected its arguments (n % gs, gs <= 64)")
    return dict(code=code, rung=rung, scale=scale, E=E, Wc=Wc,
                stats=dict(code_ties=int(stats[0]), code_hard=int(stats[1]),
                           rung_ties=int(stats[2]), rung_hard=int(stats[3])))


def f16_round(x: float) -> float:
    """Round to the nearest binary16 value (ties to even), returned as a float."""
    return float(_load().orc_f16_round(float(x)))


def pack_nibbles(code):
    """Nibble plane (rows x n/2 bytes): column 2m in the low nibble, 2m+1 in the high one."""
    code = np.asarray(code, dtype=np.uint8)
    return (code[:, 0::2] & 0x0F) | ((code[:, 1::2] & 0x0F) << 4)


def unpack_nibbles(nib):
    nib = np.asarray(nib, dtype=np.uint8)
    rows, half = nib.shape
    out = np.empty((rows, half * 2), dtype=np.uint8)
    out[:, 0::2] = nib & 0x0F
    out[:, 1::2] = nib >> 4
    return out


def dequant(code, scale, gs=32):
    """W_hat[r, j] = (code - 8) * scale[r, j // gs] in f64."""
    q = np.asarray(code, dtype=np.float64) - 8.0
    return q * np.repeat(np.asarray(scale, dtype=np.float64), gs, axis=1)


def output_error(W0, dead, code, scale, H, gs=32):
    """tr(dW H dW^T) with dW = W0 (dead columns zeroed) - W_hat and the raw Hessian H (f64).

    H is read from its upper triangle, as the fold reads it."""
    W = np.asarray(W0, dtype=np.float64).copy()
    W[:, np.asarray(dead, dtype=bool)] = 0.0
    dW = W - dequant(code, scale, gs)
    Hu = np.triu(np.asarray(H, dtype=np.float64))
    Hs = Hu + np.triu(Hu, 1).T
    return float(np.einsum("ij,ij->", dW @ Hs, dW))


def gram(X, H0=None):
    """H0 + X^T X in f64 for X [t, n] (tokens x channels): the definition, one library matmul.
    Also returns the elementwise magnitude |X|^T |X|, the scale of any summation's rounding."""
    X = np.asarray(X, dtype=np.float64)
    H = X.T @ X
    if H0 is not None:
        H = H + np.asarray(H0, dtype=np.float64)
    A = np.abs(X)
    return H, A.T @ A


def symmetric_from_upper(H, dead=None):
    """H read through its upper triangle, f64, dead channels' rows and columns zeroed."""
    H = np.asarray(H, dtype=np.float64)
    Hs = np.triu(H) + np.triu(H, 1).T
    if dead is not None:
        d = np.asarray(dead, dtype=bool)
        Hs[d, :] = 0.0
        Hs[:, d] = 0.0
    return Hs


def debias(W0, H, dead, code, rung, lost, scale, gs=32, rows=None, two_bit=False):
    """Output debias in f64.  ``code`` [rows, n] (0..15; with ``two_bit`` the q2tp levels 0..3),
    ``rung`` [rows, n/gs], ``lost`` [rows, 2] (lo, step), ``scale`` [rows, n/gs] the scales the
    codes were made with.  ``rows`` restricts the work to those row indices.  The new ladder is
    TAB[c] = 2^(lo + c step) (4-bit) or TAB[0] = 0, TAB[c] = 2^(lo + (c - 1) step) (2-bit, the
    q2tp ladder).  Returns dict(num, den, b, v = lo - log2 b before rounding (nan where lo is
    kept), lo, tab [rows, 32], scale)."""
    W0 = np.asarray(W0, dtype=np.float32)
    sel = np.arange(W0.shape[0]) if rows is None else np.asarray(rows)
    d = np.asarray(dead, dtype=bool)
    Wd = W0[sel].astype(np.float64)
    Wd[:, d] = 0.0
    dq = dequant_q2 if two_bit else dequant
    What = dq(np.asarray(code)[sel], np.asarray(scale)[sel], gs)
    Y = Wd @ symmetric_from_upper(H, d)          # H w for each row (H symmetric)
    num = np.sum(What * Y, axis=1)
    den = np.sum(Wd * Y, axis=1)
    lo = np.asarray(lost, dtype=np.float64)[sel, 0].copy()
    st = np.asarray(lost, dtype=np.float64)[sel, 1]
    with np.errstate(divide="ignore", invalid="ignore"):
        b = num / den
    v = np.full(len(sel), np.nan)
    for k in range(len(sel)):
        if num[k] > 0 and den[k] > 0 and np.isfinite(b[k]) and b[k] > 0:
            v[k] = lo[k] - np.log2(b[k])
            lo2 = f16_round(v[k])
            if np.isfinite(lo2):
                lo[k] = lo2
    if two_bit:
        tab = np.float32(np.exp2(lo[:, None] + (np.arange(32)[None, :] - 1) * st[:, None]))
        tab[:, 0] = 0.0
    else:
        tab = np.float32(np.exp2(lo[:, None] + np.arange(32)[None, :] * st[:, None]))
    rg = np.asarray(rung)[sel].astype(np.int64) & 31
    new_scale = np.take_along_axis(tab, rg, axis=1)
    return dict(num=num, den=den, b=b, v=v, lo=lo, tab=tab, scale=new_scale)


def f16_ulp(x: float) -> float:
    """Spacing of binary16 values at |x| (normal range)."""
    a = abs(float(x))
    if a < 2.0 ** -14:
        return 2.0 ** -24
    return 2.0 ** (np.floor(np.log2(a)) - 10)


def _total_key(x: np.float32) -> int:
    """The f32 total order as an integer (-NaN < -inf < ... < -0 < +0 < ... < +inf < +NaN)."""
    b = int(np.asarray(x, dtype=np.float32).view(np.int32))
    return b if b >= 0 else b ^ 0x7FFFFFFF


def act_order_perm(hdiag):
    """Channel order for act-order GPTQ: descending H_ii in the f32 total order, ties by
    ascending index."""
    h = np.asarray(hdiag, dtype=np.float32)
    return np.array(sorted(range(len(h)), key=lambda i: (-_total_key(h[i]), i)), dtype=np.int64)


def permute_sym(H, perm):
    """H[perm][perm] of the Hessian read through its upper triangle (f64)."""
    Hs = symmetric_from_upper(H)
    p = np.asarray(perm)
    return Hs[np.ix_(p, p)]


def static_rungs(W0, dead, tab, lost, gs=32):
    """The rung of every (row, group) chosen up front from the dead-zeroed original tile: the
    sweep's rung rule with unit weights and no error feedback (U = I)."""
    n = np.asarray(W0).shape[1]
    r = sweep(W0, np.eye(n), np.ones(n, np.float32), dead, tab, lost, gs=gs, want_E=False)
    return r["rung"], r["scale"]


def static_rungs_q2(W0, dead, tab, hdiag, gs=32):
    """The q2tp rung of every (row, group) chosen up front from the dead-zeroed original tile:
    the sweep's full search over rungs 1..31 by the max(H_ii, 0)-weighted error, with no error
    feedback (U = I); rung 0 for an all-zero tile."""
    n = np.asarray(W0).shape[1]
    r = sweep_q2(W0, np.eye(n), hdiag, dead, tab, gs=gs, want_E=False)
    return r["rung"], r["scale"]


def sweep_act_order(W0, Up, dead, perm, tab, lost, gs=32, rung=None, force_code=None,
                    tie_band=1e-3, want_E=True, nt=None, two_bit=False, hdiag=None):
    """Act-order sweep with static groups.  ``Up`` is the fold operator of H[perm][perm];
    ``dead`` (and ``hdiag``) are in original channel order.  4-bit (q4tp) by default: static
    rungs from :func:`static_rungs`, code = q + 8; ``two_bit``: q2tp, static rungs from
    :func:`static_rungs_q2` (needs ``hdiag``), code = the level 0..3.  Returns code (rows x n,
    original order), rung and scale (static), E (elimination order) and the tie statistics of a
    forced replay (force_code in original order)."""
    W0 = np.asarray(W0, dtype=np.float32)
    rows, n = W0.shape
    d = np.asarray(dead, dtype=bool)
    p = np.asarray(perm, dtype=np.int64)
    if rung is None:
        if two_bit:
            rung, scale = static_rungs_q2(W0, d, tab, hdiag, gs)
        else:
            rung, scale = static_rungs(W0, d, tab, lost, gs)
    else:
        rung = np.asarray(rung, dtype=np.uint8)
        scale = np.take_along_axis(np.asarray(tab, np.float32), rung.astype(np.int64) & 31, 1)
    Wd = W0.copy()
    Wd[:, d] = 0.0
    Wp = np.ascontiguousarray(Wd[:, p])
    sp = np.ascontiguousarray(np.repeat(scale, gs, axis=1)[:, p], dtype=np.float32)
    Upc = np.ascontiguousarray(Up, dtype=np.float64)
    code_p = np.empty((rows, n), dtype=np.uint8)
    E = np.empty((rows, n), dtype=np.float64) if want_E else None
    fc = None if force_code is None else np.ascontiguousarray(np.asarray(force_code)[:, p], dtype=np.uint8)
    stats = np.zeros(2, dtype=np.int64)
    _load().orc_sweep_static(_ptr(Wp), rows, n, _ptr(Upc), _ptr(sp), int(bool(two_bit)),
                             _ptr(code_p), _ptr(E), _ptr(fc), float(tie_band), _ptr(stats),
                             threads(nt))
    code = np.empty_like(code_p)
    code[:, p] = code_p
    return dict(code=code, rung=rung, scale=scale, E=E,
                stats=dict(code_ties=int(stats[0]), code_hard=int(stats[1])))


def ladder_q2(W0, dead, gs=32):
    """(lost [rows, 2], tab [rows, 32]) of the q2tp ladder (a stated reading), TAB[0] = 0."""
    W0 = np.ascontiguousarray(W0, dtype=np.float32)
    rows, n = W0.shape
    d = np.ascontiguousarray(dead, dtype=np.uint8)
    lost = np.empty((rows, 2), dtype=np.float32)
    tab = np.empty((rows, 32), dtype=np.float32)
    _load().orc_ladder_q2(_ptr(W0), _ptr(d), rows, n, gs, _ptr(lost), _ptr(tab))
    return lost, tab


def sweep_q2(W0, U, hdiag, dead, tab, gs=32, force_code=None, force_rung=None, tie_band=1e-3,
             rung_band=1e-4, want_E=True, nt=None):
    """Column-sequential q2tp sweep ("placed" rule).  ``code`` holds the 2-bit level 0..3 one
    per byte; the weights are max(H_ii, 0)."""
    W0 = np.ascontiguousarray(W0, dtype=np.float32)
    rows, n = W0.shape
    U = np.ascontiguousarray(U, dtype=np.float64)
    hw = np.ascontiguousarray(np.maximum(np.asarray(hdiag, dtype=np.float32), 0.0), dtype=np.float32)
    d = np.ascontiguousarray(dead, dtype=np.uint8)
    tab = np.ascontiguousarray(tab, dtype=np.float32)
    ng = n // gs
    code = np.empty((rows, n), dtype=np.uint8)
    rung = np.empty((rows, ng), dtype=np.uint8)
    scale = np.empty((rows, ng), dtype=np.float32)
    E = np.empty((rows, n), dtype=np.float64) if want_E else None
    fc = None if force_code is None else np.ascontiguousarray(force_code, dtype=np.uint8)
    fr = None if force_rung is None else np.ascontiguousarray(force_rung, dtype=np.uint8)
    stats = np.zeros(4, dtype=np.int64)
    st = _load().orc_sweep_q2(_ptr(W0), rows, n, gs, _ptr(U), _ptr(hw), _ptr(d), _ptr(tab),
                              _ptr(code), _ptr(rung), _ptr(scale), _ptr(E), _ptr(fc), _ptr(fr),
                              float(tie_band), float(rung_band), _ptr(stats), threads(nt))
    if st != OK:
        raise ValueError("oracle q2 sweep rejected its arguments")
    return dict(code=code, rung=rung, scale=scale, E=E,
                stats=dict(code_ties=int(stats[0]), code_hard=int(stats[1]),
                           rung_ties=int(stats[2]), rung_hard=int(stats[3])))


def pack_q2(code):
    """2-bit plane (rows x n/4 bytes): column 4m + i in bits 2i of byte m."""
    c = np.asarray(code, dtype=np.uint8) & 3
    return c[:, 0::4] | (c[:, 1::4] << 2) | (c[:, 2::4] << 4) | (c[:, 3::4] << 6)


def unpack_q2(plane):
    p = np.asarray(plane, dtype=np.uint8)
    rows, q = p.shape
    out = np.empty((rows, 4 * q), dtype=np.uint8)
    for i in range(4):
        out[:, i::4] = (p >> (2 * i)) & 3
    return out


def dequant_q2(code, scale, gs=32):
    """W_hat[r, j] = (code - 1.5) * scale[r, j // gs] in f64."""
    q = np.asarray(code, dtype=np.float64) - 1.5
    return q * np.repeat(np.asarray(scale, dtype=np.float64), gs, axis=1)

