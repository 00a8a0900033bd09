"""The batched round on the GPU (include/gptq.h, gptq_round): every group's results equal, bit for
bit, those of the separate calls (fold, ladder, sweep) on the same inputs, whatever the slots,
order and concurrency; a degenerate group and groups of mixed widths, precisions, layouts and
codecs in one round; and one group's layer-output error against the free-running oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from packing import pack_upper
from parity import OUT_ERR_TOL, output_error, say

pytestmark = pytest.mark.gpu


def separate(gpu, g):
    """The group through the separate entry points."""
    U, hd, dd, rep = gpu.gptq_fold(g["H"], g["lam"], precision=g.get("precision", "auto"),
                                   check=False)
    outs = []
    for m in g.get("members", ()):
        W, codec = m if isinstance(m, tuple) else (m, "q4tp")
        if codec == "q4tp":
            lost, tab = gpu.gptq_ladder(W, dd)
            codes, rung, scale, _ = gpu.gptq_sweep(W, U, hd, dd, tab, lost)
        else:
            lost, tab = gpu.gptq_ladder_q2(W, dd)
            codes, rung, scale, _ = gpu.gptq_sweep_q2(W, U, hd, dd, tab)
        outs.append((lost, tab, codes, rung, scale))
    torch.cuda.synchronize()
    return rep, hd, dd, outs


def assert_same(gpu, groups, results, label):
    for i, (g, r) in enumerate(zip(groups, results)):
        rep, hd, dd, outs = separate(gpu, g)
        assert r["status"] == rep["status"], (label, i, r["status"], rep["status"])
        want = {k: v for k, v in rep.items() if k != "status"}
        assert r["report"] == want, (label, i)
        assert torch.equal(r["hdiag"], hd) and torch.equal(r["dead"], dd), (label, i)
        for k, (a, b) in enumerate(zip(r["members"], outs)):
            for x, y, what in zip(a, b, ("lost", "tab", "codes", "rung", "scale")):
                assert torch.equal(x, y), f"{label}: group {i} member {k}: {what} differs"


@pytest.mark.parametrize("conc", [0, 1, 4, 11])
def test_batched_round_equals_separate_calls(gpu, conc):
    """The batched round of 11 attention-shaped groups (n 4096, W 4096 x 4096, distinct seeds):
    one gang of 11 (the default, and a cap of 11), gangs of 4, 4 and 3, and one group at a time
    on one slot."""
    groups = []
    for k in range(11):
        H, W, lam = workloads.make("batch", k=k, device="cuda")
        groups.append({"H": H, "lam": lam, "members": [W]})
    torch.cuda.synchronize()
    st, res = gpu.gptq_round(groups, max_concurrency=conc)
    torch.cuda.synchronize()
    assert st == gpu.GPTQ_OK
    say(f"round of 11 at concurrency {conc}: statuses {[r['status'] for r in res]}")
    assert_same(gpu, groups, res, f"batch conc={conc}")


def _rank_deficient(rng, n, t):
    X = rng.standard_normal((n, t)) * np.exp(rng.standard_normal(n))[:, None]
    return torch.as_tensor((X @ X.T).astype(np.float32)).cuda()


def test_mixed_round_on_a_side_stream(gpu):
    """Mixed widths (the widest first), f64 and packed groups, a q2tp member, a group with no
    members and one with two; the workspace holds two slots of three asked for; the round on a
    stream that is not the current one."""
    rng = np.random.default_rng(7)
    Ha, Wa, lam_a = workloads.make("attn", device="cuda")
    Ht, Wt, lam_t = workloads.make("tiny", device="cuda")
    Hr = _rank_deficient(rng, 1184, 500)
    W2 = (torch.randn(300, 2080, device="cuda") * 0.02).contiguous()
    H2 = _rank_deficient(rng, 2080, 3000)
    groups = [
        {"H": Ht, "lam": lam_t, "members": [Wt, (Wt[:100].contiguous(), "q2tp")]},
        {"H": Hr, "lam": 1e-5, "members": [(torch.randn(77, 1184, device="cuda") * 0.02).contiguous()]},
        {"H": pack_upper(Ha), "lam": lam_a, "members": [Wa[:640].contiguous()], "precision": "f32"},
        {"H": H2, "lam": 0.01, "members": [W2, (W2, "q2tp")], "precision": "f64"},
        {"H": _rank_deficient(rng, 300, 400), "lam": 0.01},
    ]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    ws = torch.empty(2 * _slot_size(gpu, groups), dtype=torch.uint8, device="cuda")
    st, res = gpu.gptq_round(groups, max_concurrency=3, workspace=ws, stream=side)
    side.synchronize()
    assert st == gpu.GPTQ_OK, [r["status"] for r in res]
    say("mixed round precisions " + str([r["report"]["precision"] for r in res]))
    assert res[3]["report"]["precision"] == 64
    assert_same(gpu, groups, res, "mixed")


def _slot_size(gpu, groups):
    """gptq_round_slot_size of the groups, through the binding's structures."""
    lib = gpu.load()
    arr = (gpu.RoundGroup * len(groups))()
    keep = []
    for i, g in enumerate(groups):
        h_ptr, n, ldh = gpu._hessian(g["H"])
        mem = list(g.get("members", ()))
        ms = (gpu.RoundMember * max(len(mem), 1))()
        for k, m in enumerate(mem):
            W, codec = m if isinstance(m, tuple) else (m, "q4tp")
            ms[k] = gpu.RoundMember(W.data_ptr(), W.shape[0], gpu.CODEC[codec], 0, 16, 16, 16, 16, 16)
        keep.append(ms)
        arr[i] = gpu.RoundGroup(h_ptr.value, n, ldh, float(g["lam"]),
                                gpu.FOLD_PRECISION[g.get("precision", "auto")], len(mem), ms,
                                None, None, gpu.FoldReport(), 0, 0)
    return int(lib.gptq_round_slot_size(arr, len(groups)))


def test_degenerate_group_in_a_round(gpu):
    """A Hessian no damping makes positive definite: the group reports GPTQ_DEGENERATE, its
    member is swept against U = I, as the separate calls do, and the round still returns OK."""
    n = 64
    H = torch.full((n, n), -0.9, device="cuda")
    H.fill_diagonal_(1.0)
    W = (torch.randn(48, n, device="cuda") * 0.02).contiguous()
    Ht, Wt, lam_t = workloads.make("tiny", device="cuda")
    groups = [{"H": H, "lam": 0.01, "members": [W]}, {"H": Ht, "lam": lam_t, "members": [Wt]}]
    st, res = gpu.gptq_round(groups, max_concurrency=2)
    torch.cuda.synchronize()
    assert st == gpu.GPTQ_OK
    assert res[0]["status"] == gpu.GPTQ_DEGENERATE and res[0]["report"]["degenerate"] == 1
    assert res[1]["status"] == gpu.GPTQ_OK
    assert_same(gpu, groups, res, "degenerate")


def test_round_group_against_the_oracle(gpu):
    """One group of a round against the free-running oracle: the layer-output error
    tr(dW H dW^T) within 1% (two-sided)."""
    groups = []
    for k in range(3):
        H, W, lam = workloads.make("batch", k=k, device="cuda")
        groups.append({"H": H, "lam": lam, "members": [W[:256].contiguous()]})
    st, res = gpu.gptq_round(groups)
    torch.cuda.synchronize()
    assert st == gpu.GPTQ_OK
    g, r = groups[2], res[2]
    Hn, Wn = g["H"].cpu().numpy(), g["members"][0].cpu().numpy()
    free = oracle.fold(Hn, g["lam"])
    assert r["report"]["lambda_used"] == free["lam"]
    lo, tb = oracle.ladder(Wn, free["dead"])
    os_ = oracle.sweep(Wn, free["U"], free["hdiag"], free["dead"], tb, lo, want_E=False)
    t_orc = oracle.output_error(Wn, free["dead"], os_["code"], os_["scale"], Hn)
    lost, tab, codes, rung, scale = r["members"][0]
    t_gpu = output_error(Wn, free["dead"], codes.cpu().numpy(), scale.cpu().numpy(), Hn)
    say(f"round group 2: output error rel {(t_gpu - t_orc) / t_orc:+.2e}")
    assert abs(t_gpu - t_orc) <= OUT_ERR_TOL * t_orc


def _full_rank(rng, n, t):
    X = rng.standard_normal((n, t))
    return torch.as_tensor((X @ X.T).astype(np.float32)).cuda()


def test_gang_with_failing_and_degenerate_groups(gpu):
    """A gang of five n = 1184 groups at lambda 1e-5: two rank-deficient Hessians (their f32
    attempt meets the pivot floor: folded again on their own, in f64), two full-rank ones (f32)
    and one that no damping makes positive definite (GPTQ_DEGENERATE, U = I); ragged members of
    77 rows.  Every status, report and output equals the separate calls'."""
    rng = np.random.default_rng(11)
    n = 1184
    Hdeg = torch.full((n, n), -0.9, device="cuda")
    Hdeg.fill_diagonal_(1.0)
    Hs = [_rank_deficient(rng, n, 500), _full_rank(rng, n, 5000), _rank_deficient(rng, n, 700),
          Hdeg, _full_rank(rng, n, 6000)]
    groups = [{"H": H, "lam": 1e-5, "members": [(torch.randn(77, n, device="cuda") * 0.02).contiguous()]}
              for H in Hs]
    torch.cuda.synchronize()
    r = gpu.Round(groups)
    assert r.plan()[1] == 5
    st = r.run()
    torch.cuda.synchronize()
    res = r.results
    assert st == gpu.GPTQ_OK, [x["status"] for x in res]
    precisions = [x["report"]["precision"] for x in res]
    say(f"gang of 5: statuses {[x['status'] for x in res]}, precisions {precisions}")
    assert precisions[0] == 64 and precisions[2] == 64 and precisions[1] == 32 and precisions[4] == 32
    assert res[3]["status"] == gpu.GPTQ_DEGENERATE
    assert_same(gpu, groups, res, "gang with failing groups")


def test_gang_of_mixed_layouts_and_codecs_on_a_side_stream(gpu):
    """A gang of three n = 640 groups whose Hessians come packed, dense and row-padded, each
    with two members (96 rows q4tp, 33 rows q2tp), on a stream that is not the current one; a
    second run of the same round gives the same results."""
    rng = np.random.default_rng(5)
    n = 640
    H0 = _full_rank(rng, n, 2000)
    H1 = _full_rank(rng, n, 3000)
    Hp = torch.zeros(n, 700, device="cuda")
    Hp[:, :n] = _full_rank(rng, n, 2500)
    Hp = Hp[:, :n]  # rows 700 floats apart
    groups = []
    for H in (pack_upper(H0), H1, Hp):
        W = (torch.randn(96, n, device="cuda") * 0.02).contiguous()
        W2 = (torch.randn(33, n, device="cuda") * 0.02).contiguous()
        groups.append({"H": H, "lam": 0.01, "members": [W, (W2, "q2tp")]})
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    r = gpu.Round(groups, stream=side)
    assert r.plan()[1] == 3
    for rep in range(2):
        st = r.run(stream=side)
        side.synchronize()
        assert st == gpu.GPTQ_OK, [x["status"] for x in r.results]
        assert_same(gpu, groups, r.results, f"mixed gang run {rep}")


def test_gangs_of_sixteen_at_a_ragged_width(gpu):
    """20 groups of the tiny workload's recipe (outliers, dead channels) at n = 288, which pads
    to 384 inside the fold, with 100-row members: gangs of 16 and 4, every result equal to the
    separate calls'."""
    groups = []
    for k in range(20):
        H, W, lam = workloads.make("tiny", k=k, device="cuda", n=288, rows=100)
        groups.append({"H": H, "lam": lam, "members": [W]})
    torch.cuda.synchronize()
    r = gpu.Round(groups, max_concurrency=16)
    assert r.plan()[1] == 16
    st = r.run()
    torch.cuda.synchronize()
    assert st == gpu.GPTQ_OK, [x["status"] for x in r.results]
    assert_same(gpu, groups, r.results, "gangs of 16 and 4")


@pytest.mark.parametrize("seed", range(8))
def test_random_gangs(gpu, seed):
    """Seeded random rounds of one shape (so one gang, or gangs of the cap): 2..12 groups, n a
    multiple of 32 in 64..1216, 1..3 members of random rows and codecs, lambda in {1e-6, 1e-4,
    1e-2}, "auto" or "f32", Hessians full rank or rank-deficient, dense, row-padded or packed.
    Every status, report and output equals the separate calls'."""
    rng = np.random.default_rng(1000 + seed)
    G = int(rng.integers(2, 13))
    n = 32 * int(rng.integers(2, 39))
    lam = float(rng.choice([1e-6, 1e-4, 1e-2]))
    precision = str(rng.choice(["auto", "f32"]))
    members = [(int(rng.integers(1, 301)), str(rng.choice(["q4tp", "q2tp"])))
               for _ in range(int(rng.integers(1, 4)))]
    cap = int(rng.choice([0, 3, 16]))
    groups = []
    for g in range(G):
        t = int(rng.integers(n // 3, 3 * n))
        X = rng.standard_normal((n, t)) * np.exp(rng.standard_normal(n))[:, None]
        H = torch.as_tensor((X @ X.T).astype(np.float32)).cuda()
        layout = int(rng.integers(0, 3))
        if layout == 1:
            Hp = torch.zeros(n, n + 8, device="cuda")
            Hp[:, :n] = H
            H = Hp[:, :n]
        elif layout == 2:
            H = pack_upper(H)
        ms = [((torch.randn(r, n, device="cuda") * 0.02).contiguous(), c) for r, c in members]
        groups.append({"H": H, "lam": lam, "precision": precision, "members": ms})
    torch.cuda.synchronize()
    say(f"random gang {seed}: G={G} n={n} lambda={lam} {precision} members={members} cap={cap}")
    r = gpu.Round(groups, max_concurrency=cap)
    st = r.run()
    torch.cuda.synchronize()
    assert st == gpu.GPTQ_OK, [x["status"] for x in r.results]
    assert_same(gpu, groups, r.results, f"random gang {seed}")
