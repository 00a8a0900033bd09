"""The packed upper-triangle Hessian (ldh = GPTQ_PACKED_UPPER), the pages' device layout (page
"cortiq-engine 0.8.41 src/gpu_wgpu/gptq_dev.rs", poff): every entry that reads or accumulates a
Hessian gives from the packed triangle exactly what it gives from the dense matrix, bit for bit,
and the packed accumulation and fold meet the oracle's bars directly."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from packing import pack_upper, unpack_upper
from parity import check_fold, say
from test_gpu_gram import check_upper

pytestmark = pytest.mark.gpu


def _same(a, b, label):
    assert torch.equal(a, b), f"{label}: packed and dense results differ"


@pytest.mark.parametrize("n,t", [(4, 1), (200, 777), (256, 2048), (1000, 333)])
def test_gram_packed_equals_dense(gpu, n, t):
    """Accumulation into the packed triangle: the same sums as into the dense upper triangle,
    on top of a nonzero start, and within the oracle's rounding bound."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(n * 7 + t)
    X = torch.randn(t, n, generator=g, device=dev)
    H0 = torch.triu(torch.randn(n, n, generator=g, device=dev))
    Hd = H0.clone()
    Hp = pack_upper(H0)
    gpu.gptq_gram_add(Hd, X)
    gpu.gptq_gram_add(Hp, X)
    torch.cuda.synchronize()
    _same(Hp, pack_upper(Hd), f"gram n={n} t={t}")
    check_upper(unpack_upper(Hp, n), H0, X, f"packed n={n} t={t}")


def test_gram_packed_at_down_proj_shape(gpu):
    """n = 17408 channels, 32768 tokens: the packed triangle (0.6 GB) equals the dense upper
    triangle (1.2 GB) entry for entry."""
    spec = workloads.SPECS["down"]
    n = spec.n
    X = workloads.activations(spec, T=32768, device="cuda:0")
    Hd = torch.zeros(n, n, device="cuda:0")
    Hp = torch.zeros(n * (n + 1) // 2, device="cuda:0")
    gpu.gptq_gram_add(Hd, X)
    gpu.gptq_gram_add(Hp, X)
    torch.cuda.synchronize()
    say(f"packed gram at n={n}: {Hp.numel() * 4 / 1e9:.2f} GB vs dense {Hd.numel() * 4 / 1e9:.2f} GB")
    for r0 in range(0, n, 2048):  # row blocks, so the packed copy of the dense triangle stays small
        r1 = min(n, r0 + 2048)
        for i in (r0, (r0 + r1) // 2, r1 - 1):
            off = i * (2 * n - i + 1) // 2
            _same(Hp[off:off + n - i], Hd[i, i:], f"row {i}")


@pytest.mark.parametrize("name", ["tiny", "fixture", "attn"])
def test_fold_packed_equals_dense(gpu, name):
    H, W, lam = workloads.make(name, device="cuda")
    Ud, hd_d, dd_d, rd = gpu.gptq_fold(H, lam)
    Up, hd_p, dd_p, rp = gpu.gptq_fold(pack_upper(H), lam)
    torch.cuda.synchronize()
    _same(Up, Ud, name)
    _same(hd_p, hd_d, name)
    _same(dd_p, dd_d, name)
    assert rp == rd


@pytest.mark.parametrize("n", [1, 7, 301, 640])
@pytest.mark.parametrize("precision", ["f32", "f64"])
def test_fold_packed_ragged_both_precisions(gpu, n, precision):
    """Sizes off every block and vector width (the dense fold takes its scalar build for n not a
    multiple of 4, the packed one always), in both arithmetics, on a rank-deficient Hessian."""
    rng = np.random.default_rng(1000 + n)
    X = rng.standard_normal((n, n // 2 + 3)) * np.exp(rng.standard_normal(n))[:, None]
    H = torch.as_tensor((X @ X.T).astype(np.float32)).cuda()
    Ud, hd_d, dd_d, rd = gpu.gptq_fold(H, 1e-4, precision=precision)
    Up, hd_p, dd_p, rp = gpu.gptq_fold(pack_upper(H), 1e-4, precision=precision)
    torch.cuda.synchronize()
    _same(Up, Ud, f"n={n} {precision}")
    _same(dd_p, dd_d, f"n={n}")
    assert rp == rd


def test_fold_packed_parity_with_oracle(gpu):
    """The fold of a packed Hessian against the oracle at the GPU's damping (the fold bar)."""
    H, W, lam = workloads.make("attn", device="cuda")
    check_fold(gpu, pack_upper(H), lam, H_np=H.cpu().numpy())


@pytest.mark.parametrize("two_bit", [False, True])
def test_debias_packed_equals_dense(gpu, two_bit):
    H, W, lam = workloads.make("fixture", device="cuda")
    U, hdiag, dead, _ = gpu.gptq_fold(H, lam)
    if two_bit:
        lost, tab = gpu.gptq_ladder_q2(W, dead)
        codes, rung, scale, _ = gpu.gptq_sweep_q2(W, U, hdiag, dead, tab)
        debias = gpu.gptq_debias_q2
    else:
        lost, tab = gpu.gptq_ladder(W, dead)
        codes, rung, scale, _ = gpu.gptq_sweep(W, U, hdiag, dead, tab, lost)
        debias = gpu.gptq_debias
    out_d = debias(W, H, dead, codes, rung, lost.clone(), scale.clone())
    out_p = debias(W, pack_upper(H), dead, codes, rung, lost.clone(), scale.clone())
    torch.cuda.synchronize()
    for a, b, what in zip(out_p, out_d, ("lost", "tab", "scale", "slope")):
        assert torch.equal(a, b) or (what == "slope" and torch.equal(torch.isnan(a), torch.isnan(b))
                                     and torch.equal(a[~torch.isnan(a)], b[~torch.isnan(b)])), what


@pytest.mark.parametrize("name", ["tiny", "attn"])
def test_act_order_packed_equals_dense(gpu, name):
    H, W, lam = workloads.make(name, device="cuda")
    Hpk = pack_upper(H)
    perm_d, dead_d = gpu.gptq_act_order_perm(H)
    perm_p, dead_p = gpu.gptq_act_order_perm(Hpk)
    torch.cuda.synchronize()
    _same(perm_p, perm_d, name)
    _same(dead_p, dead_d, name)
    _same(gpu.gptq_permute_hessian(Hpk, perm_d), gpu.gptq_permute_hessian(H, perm_d), name)
    np.testing.assert_array_equal(perm_d.cpu().numpy(),
                                  oracle.act_order_perm(np.diag(H.cpu().numpy())))


def test_packed_size_is_checked_by_the_binding(gpu):
    with pytest.raises(ValueError):
        gpu.gptq_fold(torch.zeros(11, device="cuda"), 0.01)  # not a triangular number
