"""The no-allocation entry point gptq_sweep_inplace_noalloc (include/gptq.h), for callers that
cannot allocate device memory: through the C ABI, against gptq_sweep_inplace (the same sweep
with a caller's workspace), bit for bit, on two calls in a row with the second one smaller,
so the static scratch is reused with stale contents from the first call."""
import ctypes

import numpy as np
import pytest
import torch

from parity import say

pytestmark = pytest.mark.gpu

P = ctypes.c_void_p


def _problem(gpu, n, rows, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, 2 * n)) * np.exp(rng.standard_normal(n))[:, None]
    H = torch.as_tensor((X @ X.T).astype(np.float32)).cuda()
    W = torch.as_tensor((rng.standard_normal((rows, n)) * 0.02).astype(np.float32)).cuda()
    U, hd, dd, rep = gpu.gptq_fold(H, 0.01)
    lost, tab = gpu.gptq_ladder(W, dd)
    return W, U, hd, dd, tab, lost


def _outputs(rows, n, want_e):
    nib = torch.full((rows, n // 2), 0x5A, dtype=torch.uint8, device="cuda")
    rung = torch.full((rows, n // 32), 0xEE, dtype=torch.uint8, device="cuda")
    scale = torch.full((rows, n // 32), -1.0, device="cuda")
    E = torch.full((rows, n), -2.0, device="cuda") if want_e else None
    return nib, rung, scale, E


def _noalloc(lib, W, U, hd, dd, tab, lost, outs):
    rows, n = W.shape
    nib, rung, scale, E = outs
    p = lambda t: None if t is None else P(t.data_ptr())
    return lib.gptq_sweep_inplace_noalloc(p(W), p(U), p(hd), p(dd), p(tab), p(lost), rows, n,
                                          p(nib), p(rung), p(scale), p(E),
                                          P(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("want_e", [False, True])
def test_noalloc_matches_inplace_sweep_on_two_calls(gpu, want_e):
    lib = gpu.load()
    for n, rows, seed in [(1184, 300, 1), (256, 77, 2)]:  # the second call is smaller
        say(f"no-alloc sweep n={n} rows={rows} E={want_e}")
        W, U, hd, dd, tab, lost = _problem(gpu, n, rows, seed)
        Wa, Wb = W.clone(), W.clone()
        ref = gpu.gptq_sweep_inplace(Wa, U, hd, dd, tab, lost, want_E=want_e)
        outs = _outputs(rows, n, want_e)
        st = _noalloc(lib, Wb, U, hd, dd, tab, lost, outs)
        torch.cuda.synchronize()
        assert st == gpu.GPTQ_OK, gpu.status_string(st)
        for x, y in zip(ref, outs):
            if x is not None:
                assert torch.equal(x, y)
        assert torch.equal(Wa, Wb)  # the same working-copy state too
        # and the same codes as the sweep that leaves W alone
        nib, rung, scale, _ = gpu.gptq_sweep(W, U, hd, dd, tab, lost)
        torch.cuda.synchronize()
        assert torch.equal(nib, outs[0]) and torch.equal(rung, outs[1]) and torch.equal(scale, outs[2])


def test_noalloc_rejects_more_rows_than_its_scratch(gpu):
    """Without E the residual panels need the static scratch, which holds 8192 rows: one more
    is refused with GPTQ_ETOOBIG and nothing is written; with E the scratch is not used."""
    lib = gpu.load()
    rows, n = 8193, 32
    W, U, hd, dd, tab, lost = _problem(gpu, n, rows, 3)
    outs = _outputs(rows, n, False)
    st = _noalloc(lib, W.clone(), U, hd, dd, tab, lost, outs)
    torch.cuda.synchronize()
    assert st == gpu.GPTQ_ETOOBIG and "8192" in gpu.status_string(st)
    assert torch.all(outs[0] == 0x5A) and torch.all(outs[1] == 0xEE) and torch.all(outs[2] == -1.0)
    outs = _outputs(rows, n, True)
    st = _noalloc(lib, W.clone(), U, hd, dd, tab, lost, outs)
    torch.cuda.synchronize()
    assert st == gpu.GPTQ_OK
    ref = gpu.gptq_sweep(W, U, hd, dd, tab, lost, want_E=True)
    torch.cuda.synchronize()
    for x, y in zip(ref, outs):
        assert torch.equal(x, y)
