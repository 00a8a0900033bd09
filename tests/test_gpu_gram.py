"""GPU parity of the device Hessian accumulation (gptq_gram_add) against the oracle's f64
definition.  Bar: every entry of the upper triangle within the worst-case rounding bound of an
f32 sum of t products in any order, (t + 2) u (|X|^T |X|)_ij with u = 2^-24; the lower
triangle untouched; repeated runs bit-identical.  At the down_proj shape (n = 17408,
t = 32768 tokens) sampled entries are checked one dot product at a time."""
import numpy as np
import pytest
import torch

import oracle
import workloads

U32 = 2.0 ** -24


def check_upper(Hg, H0, X, label):
    Hg = Hg.cpu().numpy().astype(np.float64)
    ref, mag = oracle.gram(X.cpu().numpy(), H0=None if H0 is None else H0.cpu().numpy())
    t = X.shape[0]
    base = np.abs(H0.cpu().numpy().astype(np.float64)) if H0 is not None else 0.0
    bound = (t + 2) * U32 * (mag + base) + 1e-30
    iu = np.triu_indices(Hg.shape[0])
    err = np.abs(Hg[iu] - ref[iu])
    worst = float(np.max(err / bound[iu]))
    assert worst <= 1.0, f"{label}: error {worst:.3f} x the rounding bound"
    return worst


def run(gpu, n, t, H0=None, seed=0, X=None):
    dev = torch.device("cuda:0")
    if X is None:
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        X = torch.randn(t, n, generator=g, device=dev, dtype=torch.float32)
    # A sentinel below the diagonal, which must stay untouched.
    upper = torch.triu(torch.ones(n, n, dtype=torch.bool, device=dev))
    H = torch.where(upper, torch.zeros(n, n, device=dev) if H0 is None else H0,
                    torch.full((n, n), -7.5, device=dev))
    Hin = H.clone()
    gpu.gptq_gram_add(H, X)
    torch.cuda.synchronize()
    low = torch.tril(torch.ones(n, n, dtype=torch.bool, device=dev), -1)
    assert torch.equal(H[low], Hin[low]), "lower triangle written"
    return H, X


@pytest.mark.gpu
@pytest.mark.parametrize("n,t", [(4, 1), (8, 33), (200, 777), (256, 2048), (384, 64)])
def test_gram_small_and_ragged(gpu, n, t):
    H, X = run(gpu, n, t, seed=n + t)
    check_upper(H, None, X, f"n={n} t={t}")


@pytest.mark.gpu
def test_gram_pages_fixture_and_accumulation(gpu):
    x = torch.from_numpy(workloads.pages_fixture_activations()).cuda()
    n = x.shape[1]
    H, _ = run(gpu, n, x.shape[0], X=x)
    check_upper(H, None, x, "fixture")
    assert not H[17, 17:].any() and not H[:17, 17].any()  # dead channel
    # A second window accumulates on top of the first.
    g = torch.Generator(device="cuda:0")
    g.manual_seed(5)
    x2 = torch.randn(300, n, generator=g, device="cuda:0")
    H1 = H.clone()
    gpu.gptq_gram_add(H, x2)
    torch.cuda.synchronize()
    H1l = torch.triu(H1)
    check_upper(H, H1l, x2, "second window")


@pytest.mark.gpu
def test_gram_workload_and_repeatability(gpu):
    spec = workloads.SPECS["tiny"]
    X = workloads.activations(spec, T=2048, device="cuda:0")
    H, _ = run(gpu, spec.n, X.shape[0], X=X)
    check_upper(H, None, X, "tiny workload")
    H2, _ = run(gpu, spec.n, X.shape[0], X=X)
    assert torch.equal(torch.triu(H), torch.triu(H2))


@pytest.mark.gpu
def test_gram_padded_leading_dimensions(gpu):
    """H and X with padded rows (ldh = n + 12, ldx = n + 8; the padding is NaN and neither read
    nor written): the upper triangle matches the contiguous call bitwise."""
    n, t = 200, 300
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(21)
    X = torch.randn(t, n, generator=g, device=dev)
    H0, _ = run(gpu, n, t, X=X)
    Xp = torch.full((t, n + 8), float("nan"), device=dev)
    Xp[:, :n] = X
    Hp = torch.full((n, n + 12), float("nan"), device=dev)
    Hp[:, :n] = torch.triu(torch.zeros(n, n, device=dev))
    gpu.gptq_gram_add(Hp[:, :n], Xp[:, :n])
    torch.cuda.synchronize()
    assert torch.equal(torch.triu(Hp[:, :n]), torch.triu(H0))
    assert torch.isnan(Hp[:, n:]).all()


@pytest.mark.gpu
def test_gram_zero_tokens_and_invalid(gpu):
    import ctypes
    H = torch.ones(64, 64, device="cuda:0")
    X = torch.ones(0, 64, device="cuda:0")
    gpu.gptq_gram_add(H, X)
    torch.cuda.synchronize()
    assert torch.equal(H, torch.ones_like(H))
    lib = gpu.load()
    Xb = torch.ones(10, 66, device="cuda:0")
    Hb = torch.ones(66, 66, device="cuda:0")
    st = lib.gptq_gram_add(ctypes.c_void_p(Hb.data_ptr()), 66, 66, ctypes.c_void_p(Xb.data_ptr()),
                           10, 66, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == gpu.GPTQ_EINVAL and torch.equal(Hb, torch.ones_like(Hb))


@pytest.mark.gpu
def test_gram_down_proj_shape_sampled(gpu):
    spec = workloads.SPECS["down"]
    X = workloads.activations(spec, device="cuda:0")
    n, t = spec.n, X.shape[0]
    H = torch.zeros(n, n, device="cuda:0")
    gpu.gptq_gram_add(H, X)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    i = rng.integers(0, n, 200)
    j = rng.integers(0, n, 200)
    i, j = np.minimum(i, j), np.maximum(i, j)
    i = np.concatenate([i, np.arange(0, n, 997)])
    j = np.concatenate([j, np.arange(0, n, 997)])
    cols = np.unique(np.concatenate([i, j]))
    Xc = X[:, torch.from_numpy(cols).cuda()].cpu().numpy().astype(np.float64)
    pos = {c: k for k, c in enumerate(cols)}
    got = H[torch.from_numpy(i).cuda(), torch.from_numpy(j).cuda()].cpu().numpy().astype(np.float64)
    worst = 0.0
    for a, b, gv in zip(i, j, got):
        xa, xb = Xc[:, pos[a]], Xc[:, pos[b]]
        ref = float(xa @ xb)
        bound = (t + 2) * U32 * float(np.abs(xa) @ np.abs(xb)) + 1e-30
        worst = max(worst, abs(gv - ref) / bound)
    assert worst <= 1.0, f"sampled error {worst:.3f} x bound"
    low = torch.tril(torch.ones(64, 64, dtype=torch.bool, device="cuda:0"), -1)
    assert not H[:64, :64][low].any()


@pytest.mark.gpu
def test_gram_bit_exact_at_down_proj_shape(gpu):
    """n = 17408 channels, t = 32768 tokens with integer activations in -2..2 and power-of-two
    channel scales: every product and partial sum of an entry is exact in f32 (the entry is
    2^(e_i + e_j) times an integer of magnitude at most 4 t < 2^24), so whatever the summation
    order the result is the definition h_ij = sum_r x_ri x_rj exactly.  Checked bit for bit
    against the f64 definition on whole 512 x 512 tiles: the first and last diagonal tiles, the
    corner tile, the edge tiles of the last tile row and column, and interior tiles."""
    n, t = 17408, 32768
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(1717)
    Xi = torch.randint(-2, 3, (t, n), generator=g, device=dev, dtype=torch.int32).float()
    e = torch.randint(-6, 7, (n,), generator=g, device=dev, dtype=torch.int32).float()
    X = Xi * torch.exp2(e)[None, :]
    del Xi
    H = torch.zeros(n, n, device=dev)
    gpu.gptq_gram_add(H, X)
    torch.cuda.synchronize()
    T = 512
    last = n - T
    tiles = [(0, 0), (last, last), (0, last), (T * 13, last), (T * 7, T * 21), (T * 16, T * 16),
             (T * 3, T * 30)]
    for i0, j0 in tiles:
        xi = X[:, i0:i0 + T].cpu().numpy().astype(np.float64)
        xj = X[:, j0:j0 + T].cpu().numpy().astype(np.float64)
        ref = xi.T @ xj
        got = H[i0:i0 + T, j0:j0 + T].cpu().numpy().astype(np.float64)
        up = np.add.outer(np.arange(i0, i0 + T), -np.arange(j0, j0 + T)) <= 0  # j >= i
        assert np.array_equal(got[up], ref[up]), f"tile ({i0}, {j0}) differs"
        if i0 != j0:
            assert up.all()
