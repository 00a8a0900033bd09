"""Python binding of libgptq_mi355x (ctypes): argument marshalling only.

Every step of the method runs in the library's HIP kernels; PyTorch supplies device memory
and the current stream.  There is no fallback: without the built library or a GPU the calls
raise.  Names follow the C ABI in ``include/gptq.h``:

* :func:`gptq_fold` -- H -> U, hdiag, dead, report
* :func:`gptq_ladder` -- W, dead -> lost, tab
* :func:`gptq_sweep` -- W, U, hdiag, dead, tab, lost -> nib, rung, scale, E
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgptq_mi355x.so")

GPTQ_OK, GPTQ_EINVAL, GPTQ_EWORKSPACE, GPTQ_EHIP, GPTQ_DEGENERATE, GPTQ_ECHECK, GPTQ_ETOOBIG = 0, 1, 2, 3, 4, 5, 6
GPTQ_PACKED_UPPER = -1  # ldh of a Hessian stored as its packed upper triangle

_lib = None


class GptqError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class FoldReport(ctypes.Structure):
    _fields_ = [("lambda_used", ctypes.c_double), ("base", ctypes.c_double),
                ("damp", ctypes.c_double), ("attempts", ctypes.c_int32),
                ("n_dead", ctypes.c_int32), ("degenerate", ctypes.c_int32),
                ("precision", ctypes.c_int32), ("min_pivot", ctypes.c_double)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


# Arithmetic of the fold (include/gptq.h, GPTQ_FOLD_*).
FOLD_PRECISION = {"auto": 0, "f32": 1, "f64": 2}
# Codecs of a round's members (GPTQ_CODEC_*).
CODEC = {"q4tp": 0, "q2tp": 1}


class RoundMember(ctypes.Structure):
    """gptq_member of include/gptq.h."""
    _fields_ = [("W", ctypes.c_void_p), ("rows", ctypes.c_int64), ("codec", ctypes.c_int32),
                ("pad", ctypes.c_int32), ("lost", ctypes.c_void_p), ("tab", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("rung", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class RoundGroup(ctypes.Structure):
    """gptq_group of include/gptq.h."""
    _fields_ = [("H", ctypes.c_void_p), ("n", ctypes.c_int64), ("ldh", ctypes.c_int64),
                ("lam", ctypes.c_double), ("precision", ctypes.c_int32),
                ("members", ctypes.c_int32), ("member", ctypes.POINTER(RoundMember)),
                ("hdiag", ctypes.c_void_p), ("dead", ctypes.c_void_p), ("report", FoldReport),
                ("status", ctypes.c_int32), ("pad", ctypes.c_int32)]


def load():
    """Load the in-tree library (built by ``build.build()``); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m post_weight_quantization_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    lib.gptq_fold_workspace_size.argtypes = [i64]
    lib.gptq_fold_workspace_size.restype = sz
    lib.gptq_fold_workspace_size_ex.argtypes = [i64, ctypes.c_int]
    lib.gptq_fold_workspace_size_ex.restype = sz
    lib.gptq_fold.argtypes = [P, i64, i64, ctypes.c_double, P, P, P, P, sz, P,
                              ctypes.POINTER(FoldReport)]
    lib.gptq_fold.restype = ctypes.c_int
    lib.gptq_fold_ex.argtypes = [P, i64, i64, ctypes.c_double, ctypes.c_int, P, P, P, P, sz, P,
                                 ctypes.POINTER(FoldReport)]
    lib.gptq_fold_ex.restype = ctypes.c_int
    lib.gptq_ladder.argtypes = [P, P, i64, i64, P, P, P]
    lib.gptq_ladder.restype = ctypes.c_int
    lib.gptq_sweep_workspace_size.argtypes = [i64, i64]
    lib.gptq_sweep_workspace_size.restype = sz
    lib.gptq_sweep.argtypes = [P, P, P, P, P, P, i64, i64, P, P, P, P, P, sz, P]
    lib.gptq_sweep.restype = ctypes.c_int
    lib.gptq_sweep_inplace_workspace_size.argtypes = [i64, i64]
    lib.gptq_sweep_inplace_workspace_size.restype = sz
    lib.gptq_sweep_inplace.argtypes = [P, P, P, P, P, P, i64, i64, P, P, P, P, P, sz, P]
    lib.gptq_sweep_inplace.restype = ctypes.c_int
    lib.gptq_sweep_inplace_noalloc.argtypes = [P, P, P, P, P, P, i64, i64, P, P, P, P, P]
    lib.gptq_sweep_inplace_noalloc.restype = ctypes.c_int
    lib.gptq_gram_add.argtypes = [P, i64, i64, P, i64, i64, P]
    lib.gptq_gram_add.restype = ctypes.c_int
    lib.gptq_debias_workspace_size.argtypes = [i64, i64]
    lib.gptq_debias_workspace_size.restype = sz
    lib.gptq_debias.argtypes = [P, P, i64, P, P, P, P, P, P, P, i64, i64, P, sz, P]
    lib.gptq_debias.restype = ctypes.c_int
    lib.gptq_act_order_perm.argtypes = [P, i64, i64, P, P, P]
    lib.gptq_act_order_perm.restype = ctypes.c_int
    lib.gptq_permute_hessian.argtypes = [P, i64, i64, P, P, P]
    lib.gptq_permute_hessian.restype = ctypes.c_int
    lib.gptq_sweep_act_order_workspace_size.argtypes = [i64, i64]
    lib.gptq_sweep_act_order_workspace_size.restype = sz
    lib.gptq_sweep_act_order.argtypes = [P, P, P, P, P, P, i64, i64, P, P, P, P, P, sz, P]
    lib.gptq_sweep_act_order.restype = ctypes.c_int
    lib.gptq_sweep_act_order_q2.argtypes = [P, P, P, P, P, P, i64, i64, P, P, P, P, P, sz, P]
    lib.gptq_sweep_act_order_q2.restype = ctypes.c_int
    lib.gptq_debias_q2.argtypes = [P, P, i64, P, P, P, P, P, P, P, i64, i64, P, sz, P]
    lib.gptq_debias_q2.restype = ctypes.c_int
    lib.gptq_ladder_q2.argtypes = [P, P, i64, i64, P, P, P]
    lib.gptq_ladder_q2.restype = ctypes.c_int
    lib.gptq_sweep_q2.argtypes = [P, P, P, P, P, i64, i64, P, P, P, P, P, sz, P]
    lib.gptq_sweep_q2.restype = ctypes.c_int
    lib.gptq_round_slot_size.argtypes = [ctypes.POINTER(RoundGroup), ctypes.c_int32]
    lib.gptq_round_slot_size.restype = sz
    lib.gptq_round_plan.argtypes = [ctypes.POINTER(RoundGroup), ctypes.c_int32, sz, ctypes.c_int32,
                                    ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.gptq_round_plan.restype = ctypes.c_int
    lib.gptq_round.argtypes = [ctypes.POINTER(RoundGroup), ctypes.c_int32, P, sz, ctypes.c_int32, P]
    lib.gptq_round.restype = ctypes.c_int
    lib.gptq_status_string.argtypes = [ctypes.c_int]
    lib.gptq_status_string.restype = ctypes.c_char_p
    lib.gptq_profile_enable.argtypes = [ctypes.c_uint]
    lib.gptq_profile_enable.restype = None
    lib.gptq_profile_collect.argtypes = [P, P, P, P, ctypes.c_int]
    lib.gptq_profile_collect.restype = ctypes.c_int
    lib.gptq_profile_family_count.restype = ctypes.c_int
    lib.gptq_profile_family_name.argtypes = [ctypes.c_int]
    lib.gptq_profile_family_name.restype = ctypes.c_char_p
    lib.gptq_check_mode.argtypes = [ctypes.c_int]
    lib.gptq_check_mode.restype = None
    lib.gptq_check_message.restype = ctypes.c_char_p
    lib.gptq_check_selftest.argtypes = [ctypes.c_int]
    lib.gptq_check_selftest.restype = ctypes.c_int
    lib.gptq_check_tile_order.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    lib.gptq_check_tile_order.restype = ctypes.c_int
    _lib = lib
    return lib


def require_native():
    """Raise unless the HIP library loads and a GPU is visible."""
    load()
    if not torch.cuda.is_available():
        raise RuntimeError("libgptq_mi355x needs a visible MI355X GPU")


def status_string(status: int) -> str:
    try:
        return load().gptq_status_string(int(status)).decode()
    except Exception:
        return "unknown"


def _dev(t: torch.Tensor, dtype, name, shape=None, align=1, device=None):
    """A contiguous device tensor's pointer, after checking its dtype, shape, device and the
    alignment (bytes) of its first element."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call's tensors on {device}")
    if align > 1 and t.data_ptr() % align:
        raise ValueError(f"{name} must be {align}-byte aligned")
    return ctypes.c_void_p(t.data_ptr())


def _dev_rows(t: torch.Tensor, dtype, name):
    """A 2-D device tensor whose rows may be padded: unit column stride, row stride >= width
    (the row stride is passed as the leading dimension)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")
    if t.dim() != 2 or (t.shape[0] > 1 and t.stride(1) != 1) or t.stride(0) < t.shape[1]:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return ctypes.c_void_p(t.data_ptr())


def _hessian(H: torch.Tensor, device=None):
    """(pointer, n, ldh) of a Hessian: a 2-D [n, n] tensor (rows may be padded) is passed as
    dense rows; a 1-D tensor of n (n + 1) / 2 floats as the packed upper triangle, row by row
    (ldh = GPTQ_PACKED_UPPER)."""
    if isinstance(H, torch.Tensor) and H.dim() == 1:
        P = H.numel()
        n = (math.isqrt(8 * P + 1) - 1) // 2
        if n < 1 or n * (n + 1) // 2 != P:
            raise ValueError("a packed H must hold n (n + 1) / 2 floats")
        return _dev(H, torch.float32, "H", device=device), n, GPTQ_PACKED_UPPER
    if not isinstance(H, torch.Tensor) or H.dim() != 2 or H.shape[0] != H.shape[1]:
        raise ValueError("H must be [n, n], or its packed upper triangle (1-D)")
    if device is not None and H.device != device:
        raise ValueError(f"H is on {H.device}, the call's tensors on {device}")
    return _dev_rows(H, torch.float32, "H"), H.shape[0], H.stride(0)


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream, device):
    """The stream a call is enqueued on, as a context for the tensors it allocates: PyTorch's
    caching allocator then reuses their memory only in that stream's order, after the call's
    kernels, never while they may still run."""
    s = torch.cuda.current_stream(device) if stream is None else stream
    return torch.cuda.stream(s)


def _workspace(workspace, need, device, name="workspace"):
    if workspace is None:
        return torch.empty(max(int(need), 1), dtype=torch.uint8, device=device)
    _dev(workspace, torch.uint8, name, align=256, device=device)
    if workspace.numel() < need:
        raise ValueError(f"{name} has {workspace.numel()} bytes, the call needs {need}")
    return workspace


def fold_workspace_size(n: int, precision: str = "auto") -> int:
    return int(load().gptq_fold_workspace_size_ex(int(n), FOLD_PRECISION[precision]))


def sweep_workspace_size(rows: int, n: int) -> int:
    return int(load().gptq_sweep_workspace_size(int(rows), int(n)))


def gptq_fold(H: torch.Tensor, lam: float, workspace: torch.Tensor | None = None, stream=None,
              out=None, check=True, precision: str = "auto"):
    """Fold H (f32 [n, n], upper triangle read, rows may be padded; or its packed upper
    triangle, 1-D).  ``precision`` is "auto" (f32, repeated in f64 where a pivot is at or below
    1e-2), "f32" or "f64".  Returns (U, hdiag, dead, report dict)."""
    lib = load()
    dev = H.device
    h_ptr, n, ldh = _hessian(H)
    prec = FOLD_PRECISION[precision]
    need = int(lib.gptq_fold_workspace_size_ex(n, prec))
    with _on(stream, dev):
        if out is None:
            U = torch.empty(n, n, dtype=torch.float32, device=dev)
            hdiag = torch.empty(n, dtype=torch.float32, device=dev)
            dead = torch.empty(n, dtype=torch.uint8, device=dev)
        else:
            U, hdiag, dead = out
        workspace = _workspace(workspace, need, dev)
    rep = FoldReport()
    st = lib.gptq_fold_ex(h_ptr, n, ldh, float(lam), prec,
                          _dev(U, torch.float32, "U", (n, n), device=dev),
                          _dev(hdiag, torch.float32, "hdiag", (n,), device=dev),
                          _dev(dead, torch.uint8, "dead", (n,), device=dev),
                          ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                          _stream(stream), ctypes.byref(rep))
    if check and st not in (GPTQ_OK, GPTQ_DEGENERATE):
        raise GptqError(st, "gptq_fold")
    r = rep.as_dict()
    r["status"] = st
    return U, hdiag, dead, r


def gptq_ladder(W: torch.Tensor, dead: torch.Tensor, stream=None, out=None):
    """Per-row (lo, step) and the 32 rung scales of the dead-zeroed W."""
    lib = load()
    rows, n = W.shape
    dev = W.device
    with _on(stream, dev):
        if out is None:
            lost = torch.empty(rows, 2, dtype=torch.float32, device=dev)
            tab = torch.empty(rows, 32, dtype=torch.float32, device=dev)
        else:
            lost, tab = out
    st = lib.gptq_ladder(_dev(W, torch.float32, "W", align=16), _dev(dead, torch.uint8, "dead", (n,), device=dev),
                         rows, n, _dev(lost, torch.float32, "lost", (rows, 2), device=dev),
                         _dev(tab, torch.float32, "tab", (rows, 32), device=dev), _stream(stream))
    if st != GPTQ_OK:
        raise GptqError(st, "gptq_ladder")
    return lost, tab


def gptq_sweep(W, U, hdiag, dead, tab, lost, want_E=False, workspace=None, stream=None,
               out=None):
    """The q4tp sweep.  Returns (nib [rows, n/2] u8, rung [rows, n/32] u8,
    scale [rows, n/32] f32, E [rows, n] f32 or None)."""
    lib = load()
    rows, n = W.shape
    dev = W.device
    need = int(lib.gptq_sweep_workspace_size(rows, n))
    with _on(stream, dev):
        if out is None:
            nib = torch.empty(rows, n // 2, dtype=torch.uint8, device=dev)
            rung = torch.empty(rows, n // 32, dtype=torch.uint8, device=dev)
            scale = torch.empty(rows, n // 32, dtype=torch.float32, device=dev)
            E = torch.empty(rows, n, dtype=torch.float32, device=dev) if want_E else None
        else:
            nib, rung, scale, E = out
        workspace = _workspace(workspace, need, dev)
    st = lib.gptq_sweep(_dev(W, torch.float32, "W", align=16),
                        _dev(U, torch.float32, "U", (n, n), 16, dev),
                        _dev(hdiag, torch.float32, "hdiag", (n,), device=dev),
                        _dev(dead, torch.uint8, "dead", (n,), device=dev),
                        _dev(tab, torch.float32, "tab", (rows, 32), 16, dev),
                        _dev(lost, torch.float32, "lost", (rows, 2), 8, dev),
                        rows, n, _dev(nib, torch.uint8, "nib", (rows, n // 2), 16, dev),
                        _dev(rung, torch.uint8, "rung", (rows, n // 32), device=dev),
                        _dev(scale, torch.float32, "scale", (rows, n // 32), device=dev),
                        None if E is None else _dev(E, torch.float32, "E", (rows, n), 16, dev),
                        ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                        _stream(stream))
    if st != GPTQ_OK:
        raise GptqError(st, "gptq_sweep")
    return nib, rung, scale, E


def gptq_sweep_inplace(W, U, hdiag, dead, tab, lost, want_E=False, workspace=None, stream=None,
                       out=None):
    """The q4tp sweep with W as its own working copy (W is overwritten).  Returns (nib, rung,
    scale, E or None), the same as :func:`gptq_sweep` on the original W."""
    lib = load()
    rows, n = W.shape
    dev = W.device
    with _on(stream, dev):
        if out is None:
            nib = torch.empty(rows, n // 2, dtype=torch.uint8, device=dev)
            rung = torch.empty(rows, n // 32, dtype=torch.uint8, device=dev)
            scale = torch.empty(rows, n // 32, dtype=torch.float32, device=dev)
            E = torch.empty(rows, n, dtype=torch.float32, device=dev) if want_E else None
        else:
            nib, rung, scale, E = out
        need = 0 if E is not None else int(lib.gptq_sweep_inplace_workspace_size(rows, n))
        if need:
            workspace = _workspace(workspace, need, dev)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if (need and workspace is not None) else None
    st = lib.gptq_sweep_inplace(_dev(W, torch.float32, "W", align=16),
                                _dev(U, torch.float32, "U", (n, n), 16, dev),
                                _dev(hdiag, torch.float32, "hdiag", (n,), device=dev),
                                _dev(dead, torch.uint8, "dead", (n,), device=dev),
                                _dev(tab, torch.float32, "tab", (rows, 32), 16, dev),
                                _dev(lost, torch.float32, "lost", (rows, 2), 8, dev),
                                rows, n, _dev(nib, torch.uint8, "nib", (rows, n // 2), device=dev),
                                _dev(rung, torch.uint8, "rung", (rows, n // 32), device=dev),
                                _dev(scale, torch.float32, "scale", (rows, n // 32), device=dev),
                                None if E is None else _dev(E, torch.float32, "E", (rows, n), 16, dev),
                                ws_ptr, workspace.numel() if ws_ptr is not None else 0,
                                _stream(stream))
    if st != GPTQ_OK:
        raise GptqError(st, "gptq_sweep_inplace")
    return nib, rung, scale, E


def gptq_gram_add(H: torch.Tensor, X: torch.Tensor, stream=None):
    """H (f32 [n, n], device; or its packed upper triangle, 1-D) += X^T X on its upper
    triangle, X f32 [t, n] (tokens x channels).  Returns H."""
    lib = load()
    h_ptr, n, ldh = _hessian(H)
    if X.dim() != 2 or X.shape[1] != n:
        raise ValueError("X must be [t, n] with n = H.shape[0]")
    if X.device != H.device:
        raise ValueError("X and H must be on one device")
    st = lib.gptq_gram_add(h_ptr, n, ldh,
                           _dev_rows(X, torch.float32, "X"), X.shape[0], X.stride(0), _stream(stream))
    if st != GPTQ_OK:
        raise GptqError(st, "gptq_gram_add")
    return H


def debias_workspace_size(rows: int, n: int) -> int:
    return int(load().gptq_debias_workspace_size(int(rows), int(n)))


def gptq_debias(W, H, dead, nib, rung, lost, scale, want_tab=True, want_slope=True,
                workspace=None, stream=None):
    """Output debias in place on (lost, scale).  Returns (lost, tab or None, scale,
    slope f64 [rows] or None)."""
    lib = load()
    rows, n = W.shape
    dev = W.device
    h_ptr, hn, ldh = _hessian(H, dev)
    if hn != n:
        raise ValueError(f"H has {hn} channels, W {n}")
    need = int(lib.gptq_debias_workspace_size(rows, n))
    with _on(stream, dev):
        tab = torch.empty(rows, 32, dtype=torch.float32, device=dev) if want_tab else None
        slope = torch.empty(rows, dtype=torch.float64, device=dev) if want_slope else None
        workspace = _workspace(workspace, need, dev)
    st = lib.gptq_debias(_dev(W, torch.float32, "W", align=16), h_ptr,
                         ldh, _dev(dead, torch.uint8, "dead", (n,), device=dev),
                         _dev(nib, torch.uint8, "nib", (rows, n // 2), 16, dev),
                         _dev(rung, torch.uint8, "rung", (rows, n // 32), device=dev),
                         _dev(lost, torch.float32, "lost", (rows, 2), 8, dev),
                         None if tab is None else _dev(tab, torch.float32, "tab", (rows, 32), 16, dev),
                         _dev(scale, torch.float32, "scale", (rows, n // 32), device=dev),
                         None if slope is None else _dev(slope, torch.float64, "slope", (rows,), device=dev),
                         rows, n, ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                         _stream(stream))
    if st != GPTQ_OK:
        raise GptqError(st, "gptq_debias")
    return lost, tab, scale, slope


def gptq_debias_q2(W, H, dead, plane, rung, lost, scale, want_tab=True, want_slope=True,
                   workspace=None, stream=None):
    """Output debias of 2-bit codes in place on (lost, scale).  Returns (lost, tab or None,
    scale, slope f64 [rows] or None)."""
    lib = load()
    rows, n = W.shape
    dev = W.device
    h_ptr, hn, ldh = _hessian(H, dev)
    if hn != n:
        raise ValueError(f"H has {hn} channels, W {n}")
    need = int(lib.gptq_debias_workspace_size(rows, n))
    with _on(stream, dev):
        tab = torch.empty(rows, 32, dtype=torch.float32, device=dev) if want_tab else None
        slope = torch.empty(rows, dtype=torch.float64, device=dev) if want_slope else None
        workspace = _workspace(workspace, need, dev)
    st = lib.gptq_debias_q2(_dev(W, torch.float32, "W", align=16), h_ptr,
                            ldh, _dev(dead, torch.uint8, "dead", (n,), device=dev),
                            _dev(plane, torch.uint8, "plane", (rows, n // 4), device=dev),
                            _dev(rung, torch.uint8, "rung", (rows, n // 32), device=dev),
                            _dev(lost, torch.float32, "lost", (rows, 2), 8, dev),
                            None if tab is None else _dev(tab, torch.float32, "tab", (rows, 32), 16, dev),
                            _dev(scale, torch.float32, "scale", (rows, n // 32), device=dev),
                            None if slope is None else _dev(slope, torch.float64, "slope", (rows,), device=dev),
                            rows, n, ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                            _stream(stream))
    if st != GPTQ_OK:
        raise GptqError(st, "gptq_debias_q2")
    return lost, tab, scale, slope


def gptq_sweep_act_order_q2(W, U, dead, hdiag, perm, tab, want_E=False, workspace=None,
                            stream=None):
    """Act-order q2tp sweep.  ``U`` and ``hdiag`` come from the fold of H[perm][perm] (hdiag
    in elimination order); ``dead`` in original order.  Returns (plane [rows, n/4], rung,
    scale, E or None); E in elimination order."""
    lib = load()
    rows, n = W.shape
    dev = W.device
    need = int(lib.gptq_sweep_act_order_workspace_size(rows, n))
    with _on(stream, dev):
        plane = torch.empty(rows, n // 4, dtype=torch.uint8, device=dev)
        rung = torch.empty(rows, n // 32, dtype=torch.uint8, device=dev)
        scale = torch.empty(rows, n // 32, dtype=torch.float32, device=dev)
        E = torch.empty(rows, n, dtype=torch.float32, device=dev) if want_E else None
        workspace = _workspace(workspace, need, dev)
    st = lib.gptq_sweep_act_order_q2(_dev(W, torch.float32, "W", align=16),
                                     _dev(U, torch.float32, "U", (n, n), 16, dev),
                                     _dev(dead, torch.uint8, "dead", (n,), device=dev),
                                     _dev(hdiag, torch.float32, "hdiag", (n,), device=dev),
                                     _dev(perm, torch.int32, "perm", (n,), device=dev),
                                     _dev(tab, torch.float32, "tab", (rows, 32), 16, dev),
                                     rows, n, _dev(plane, torch.uint8, "plane"),
                                     _dev(rung, torch.uint8, "rung"), _dev(scale, torch.float32, "scale"),
                                     None if E is None else _dev(E, torch.float32, "E"),
                                     ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                     _stream(stream))
    if st != GPTQ_OK:
        raise GptqError(st, "gptq_sweep_act_order_q2")
    return plane, rung, scale, E


def gptq_ladder_q2(W, dead, stream=None):
    """The q2tp ladder: (lost [rows, 2], tab [rows, 32]) with TAB[0] = 0."""
    lib = load()
    rows, n = W.shape
    dev = W.device
    with _on(stream, dev):
        lost = torch.empty(rows, 2, dtype=torch.float32, device=dev)
        tab = torch.empty(rows, 32, dtype=torch.float32, device=dev)
    st = lib.gptq_ladder_q2(_dev(W, torch.float32, "W", align=16),
                            _dev(dead, torch.uint8, "dead", (n,), device=dev), rows, n,
                            _dev(lost, torch.float32, "lost"), _dev(tab, torch.float32, "tab"),
                            _stream(stream))
    if st != GPTQ_OK:
        raise GptqError(st, "gptq_ladder_q2")
    return lost, tab


def gptq_sweep_q2(W, U, hdiag, dead, tab, want_E=False, workspace=None, stream=None):
    """The q2tp sweep ("placed" rule).  Returns (plane [rows, n/4] u8, rung, scale, E or None)."""
    lib = load()
    rows, n = W.shape
    dev = W.device
    need = int(lib.gptq_sweep_workspace_size(rows, n))
    with _on(stream, dev):
        plane = torch.empty(rows, n // 4, dtype=torch.uint8, device=dev)
        rung = torch.empty(rows, n // 32, dtype=torch.uint8, device=dev)
        scale = torch.empty(rows, n // 32, dtype=torch.float32, device=dev)
        E = torch.empty(rows, n, dtype=torch.float32, device=dev) if want_E else None
        workspace = _workspace(workspace, need, dev)
    st = lib.gptq_sweep_q2(_dev(W, torch.float32, "W", align=16),
                           _dev(U, torch.float32, "U", (n, n), 16, dev),
                           _dev(hdiag, torch.float32, "hdiag", (n,), device=dev),
                           _dev(dead, torch.uint8, "dead", (n,), device=dev),
                           _dev(tab, torch.float32, "tab", (rows, 32), 16, dev), rows, n,
                           _dev(plane, torch.uint8, "plane"), _dev(rung, torch.uint8, "rung"),
                           _dev(scale, torch.float32, "scale"),
                           None if E is None else _dev(E, torch.float32, "E"),
                           ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                           _stream(stream))
    if st != GPTQ_OK:
        raise GptqError(st, "gptq_sweep_q2")
    return plane, rung, scale, E


def sweep_act_order_workspace_size(rows: int, n: int) -> int:
    return int(load().gptq_sweep_act_order_workspace_size(int(rows), int(n)))


def gptq_act_order_perm(H, stream=None):
    """(perm i32 [n], dead u8 [n]) of act-order GPTQ from H's diagonal (H dense or packed)."""
    lib = load()
    dev = H.device
    h_ptr, n, ldh = _hessian(H)
    with _on(stream, dev):
        perm = torch.empty(n, dtype=torch.int32, device=dev)
        dead = torch.empty(n, dtype=torch.uint8, device=dev)
    st = lib.gptq_act_order_perm(h_ptr, n, ldh,
                                 _dev(perm, torch.int32, "perm"), _dev(dead, torch.uint8, "dead"),
                                 _stream(stream))
    if st != GPTQ_OK:
        raise GptqError(st, "gptq_act_order_perm")
    return perm, dead


def gptq_permute_hessian(H, perm, stream=None):
    """H[perm][perm] (f32 [n, n], full symmetric) from H's upper triangle (H dense or
    packed)."""
    lib = load()
    dev = H.device
    h_ptr, n, ldh = _hessian(H)
    with _on(stream, dev):
        Hp = torch.empty(n, n, dtype=torch.float32, device=dev)
    st = lib.gptq_permute_hessian(h_ptr, n, ldh,
                                  _dev(perm, torch.int32, "perm", (n,), device=dev),
                                  _dev(Hp, torch.float32, "Hp"), _stream(stream))
    if st != GPTQ_OK:
        raise GptqError(st, "gptq_permute_hessian")
    return Hp


def gptq_sweep_act_order(W, U, dead, perm, tab, lost, want_E=False, workspace=None, stream=None):
    """Act-order q4tp sweep.  Returns (nib, rung, scale, E or None); E in elimination order."""
    lib = load()
    rows, n = W.shape
    dev = W.device
    need = int(lib.gptq_sweep_act_order_workspace_size(rows, n))
    with _on(stream, dev):
        nib = torch.empty(rows, n // 2, dtype=torch.uint8, device=dev)
        rung = torch.empty(rows, n // 32, dtype=torch.uint8, device=dev)
        scale = torch.empty(rows, n // 32, dtype=torch.float32, device=dev)
        E = torch.empty(rows, n, dtype=torch.float32, device=dev) if want_E else None
        workspace = _workspace(workspace, need, dev)
    st = lib.gptq_sweep_act_order(_dev(W, torch.float32, "W", align=16),
                                  _dev(U, torch.float32, "U", (n, n), 16, dev),
                                  _dev(dead, torch.uint8, "dead", (n,), device=dev),
                                  _dev(perm, torch.int32, "perm", (n,), device=dev),
                                  _dev(tab, torch.float32, "tab", (rows, 32), 16, dev),
                                  _dev(lost, torch.float32, "lost", (rows, 2), 8, dev),
                                  rows, n, _dev(nib, torch.uint8, "nib"),
                                  _dev(rung, torch.uint8, "rung"), _dev(scale, torch.float32, "scale"),
                                  None if E is None else _dev(E, torch.float32, "E"),
                                  ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                  _stream(stream))
    if st != GPTQ_OK:
        raise GptqError(st, "gptq_sweep_act_order")
    return nib, rung, scale, E


PROFILE_FAMILIES = ["fold_update", "fold_panel", "fold_diag", "fold_build", "fold_make_u",
                    "sweep_group", "sweep_trail", "ladder", "fold_next", "sweep_next", "gram", "debias"]


def profile_enable(families=None):
    """Time the named kernel families (all when None; none for an empty list)."""
    if families is None:
        mask = (1 << len(PROFILE_FAMILIES)) - 1
    else:
        mask = 0
        for f in families:
            mask |= 1 << PROFILE_FAMILIES.index(f)
    load().gptq_profile_enable(mask)


def profile_collect():
    """{family: dict(ms, launches, flops, bytes)} for the launches since the last collect."""
    import numpy as np
    lib = load()
    nf = lib.gptq_profile_family_count()
    ms = np.zeros(nf)
    ln = np.zeros(nf, dtype=np.int64)
    fl = np.zeros(nf)
    by = np.zeros(nf)
    P = ctypes.c_void_p
    st = lib.gptq_profile_collect(P(ms.ctypes.data), P(ln.ctypes.data), P(fl.ctypes.data),
                                  P(by.ctypes.data), nf)
    if st != GPTQ_OK:
        raise GptqError(st, "gptq_profile_collect")
    return {lib.gptq_profile_family_name(f).decode(): dict(ms=float(ms[f]), launches=int(ln[f]),
                                                           flops=float(fl[f]), bytes=float(by[f]))
            for f in range(nf)}


class Round:
    """A batched round (include/gptq.h, gptq_round) with its outputs and workspace allocated
    once, so that run() can be repeated.  ``groups``: a sequence of dicts with "H" (f32 [n, n],
    rows may be padded, or its packed upper triangle, 1-D), "lam", optionally "precision"
    ("auto", "f32", "f64"), and "members": W [rows, n] tensors, or (W, codec) pairs with codec
    "q4tp" or "q2tp".  Without a workspace, the slots the library's plan would use (its largest
    gang, or its threads), within half of the free device memory, are allocated.  ``results``: per group a dict with hdiag, dead and, per member, (lost, tab,
    codes, rung, scale); run() adds the group's status and fold report."""

    def __init__(self, groups, max_concurrency: int = 0, workspace=None, stream=None):
        lib = load()
        if not groups:
            raise ValueError("a round needs at least one group")
        dev = groups[0]["H"].device
        G = len(groups)
        self.arr = (RoundGroup * G)()
        self.keep, self.results = [], []
        with _on(stream, dev):
            for i, g in enumerate(groups):
                h_ptr, n, ldh = _hessian(g["H"], dev)
                mem = list(g.get("members", ()))
                ms = (RoundMember * max(len(mem), 1))()
                outs = []
                for k, m in enumerate(mem):
                    W, codec = m if isinstance(m, tuple) else (m, "q4tp")
                    if W.dim() != 2 or W.shape[1] != n:
                        raise ValueError(f"group {i} member {k}: W must be [rows, {n}]")
                    rows = W.shape[0]
                    cb = n // 2 if codec == "q4tp" else n // 4
                    o = (torch.empty(rows, 2, dtype=torch.float32, device=dev),
                         torch.empty(rows, 32, dtype=torch.float32, device=dev),
                         torch.empty(rows, cb, dtype=torch.uint8, device=dev),
                         torch.empty(rows, n // 32, dtype=torch.uint8, device=dev),
                         torch.empty(rows, n // 32, dtype=torch.float32, device=dev))
                    ms[k] = RoundMember(_dev(W, torch.float32, "W", align=16, device=dev).value,
                                        rows, CODEC[codec], 0, *(t.data_ptr() for t in o))
                    outs.append(o)
                hdiag = torch.empty(n, dtype=torch.float32, device=dev)
                dead = torch.empty(n, dtype=torch.uint8, device=dev)
                self.arr[i] = RoundGroup(h_ptr.value, n, ldh, float(g["lam"]),
                                         FOLD_PRECISION[g.get("precision", "auto")], len(mem), ms,
                                         hdiag.data_ptr(), dead.data_ptr(), FoldReport(), 0, 0)
                self.keep.append((ms, g["H"], mem))
                self.results.append(dict(hdiag=hdiag, dead=dead, members=outs))
            self.slot_bytes = int(lib.gptq_round_slot_size(self.arr, G))
            if self.slot_bytes == 0:
                raise ValueError("a group of the round is invalid")
            if workspace is None:
                # The slots the library's plan uses with room for all of them, within half of
                # the device memory that is free.
                order = (ctypes.c_int32 * G)()
                conc = ctypes.c_int32(0)
                st = lib.gptq_round_plan(self.arr, G, ctypes.c_size_t(self.slot_bytes * G),
                                         int(max_concurrency), order, ctypes.byref(conc))
                if st != GPTQ_OK:
                    raise GptqError(st, "gptq_round_plan")
                free = torch.cuda.mem_get_info(dev)[0]
                k = max(1, min(conc.value, free // 2 // self.slot_bytes))
                workspace = torch.empty(self.slot_bytes * k, dtype=torch.uint8, device=dev)
            else:
                _dev(workspace, torch.uint8, "workspace", align=256, device=dev)
        self.workspace = workspace
        self.max_concurrency = int(max_concurrency)

    def plan(self):
        """(order, concurrency) of the round as the library schedules it."""
        G = len(self.arr)
        order = (ctypes.c_int32 * G)()
        conc = ctypes.c_int32(0)
        st = load().gptq_round_plan(self.arr, G, self.workspace.numel(), self.max_concurrency,
                                    order, ctypes.byref(conc))
        if st != GPTQ_OK:
            raise GptqError(st, "gptq_round_plan")
        return list(order), conc.value

    def run(self, stream=None) -> int:
        st = load().gptq_round(self.arr, len(self.arr), ctypes.c_void_p(self.workspace.data_ptr()),
                               self.workspace.numel(), self.max_concurrency, _stream(stream))
        for i, r in enumerate(self.results):
            r["status"] = int(self.arr[i].status)
            r["report"] = self.arr[i].report.as_dict()
        return int(st)


def gptq_round(groups, max_concurrency: int = 0, workspace=None, stream=None):
    """Run one batched round (see Round).  Returns (status, results)."""
    r = Round(groups, max_concurrency, workspace, stream)
    st = r.run(stream)
    return st, r.results


class check_mode:
    """Context manager: the library's calls run as dry runs of their schedule (no GPU; device
    pointers are never dereferenced) and return GPTQ_ECHECK when an access leaves its buffers
    or two launches on different streams race; see include/gptq_check.h."""

    def __enter__(self):
        load().gptq_check_mode(1)
        return self

    def __exit__(self, *exc):
        load().gptq_check_mode(0)
        return False


def check_message() -> str:
    return load().gptq_check_message().decode()


def check_selftest(which: int) -> int:
    return int(load().gptq_check_selftest(int(which)))


def check_tile_order(M: int, N: int, lower: bool) -> int:
    """Status of the host-side check of the tile GEMM's workgroup -> tile map for one shape."""
    return int(load().gptq_check_tile_order(int(M), int(N), 1 if lower else 0))


__all__ = ["check_mode", "check_message", "check_selftest", "check_tile_order", "gptq_gram_add", "gptq_debias",
           "gptq_act_order_perm", "gptq_permute_hessian", "gptq_sweep_act_order",
           "sweep_act_order_workspace_size", "gptq_ladder_q2", "gptq_sweep_q2",
           "gptq_sweep_act_order_q2", "gptq_debias_q2",
           "debias_workspace_size", "gptq_fold", "FOLD_PRECISION", "gptq_ladder", "gptq_sweep", "gptq_sweep_inplace", "fold_workspace_size",
           "sweep_workspace_size", "require_native", "load", "GptqError", "profile_enable",
           "profile_collect", "LIB_PATH", "gptq_round", "Round", "RoundGroup", "RoundMember", "CODEC"]
