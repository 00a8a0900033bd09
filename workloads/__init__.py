"""Seeded synthetic inputs (Hessians and weights) shaped like the layers the method targets.

This module only draws random numbers and forms ``H = X X^T`` from them: it holds none of the
method's arithmetic, and both the HIP path and the oracle consume the tensors it returns.

Workloads (``make(name, ...)``):

=========  =======  ======  ==========================================================  ========
name       n        rows    H = X X^T from X [n, T]                                     lambda
=========  =======  ======  ==========================================================  ========
tiny       256      512     T=2048, N(0,1); 4 channels x100; 2 channels zeroed (dead)   0.01
attn       4096     4096    T=8192; 1% of channels x exp(2 z); 0.5% dead                 0.01
down       17408    5120    T=32768; every channel x exp(1.490 z) (top 0.1% ~1e4 x the   0.01
                            median energy); no dead channels
batch[k]   4096     4096    as ``attn`` with group index k = 0..10                       0.01
stress     8192     2048    T=4096 (rank-deficient); 2% dead; 0.1% of channels x100      1e-6
fixture    160      48      the pages' device-versus-host test recipe (see below)       0.01
=========  =======  ======  ==========================================================  ========

Weights are N(0, sigma^2) with sigma = 0.02 (0.015 for ``down``).  Seeds: X from
``1000 c + 2 k``, W from ``1000 c + 2 k + 1``, channel picks from ``torch.randperm`` on the CPU
with ``1000 c + 100 + k`` (c = workload number 1..5, k = group index).  H accumulates over
T-chunks of 4096 columns in f32.  A random-number stream depends on the device it is drawn on,
so a workload drawn on the GPU and one drawn on the CPU differ; every comparison feeds the
same drawn tensors to both sides.

``fixture`` re-creates the calibration data of the test ``device_fold_and_sweep_match_host`` on
the page "cortiq-cli 0.8.45 src/gptq.rs" from its formulas: correlated activations from
modular hashes, channels with ``c % 41 == 3`` made 30x louder, channels 17 and 90 dead, and
weights from a multiplicative hash times 0.08.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Spec:
    name: str
    cfg: int          # workload number used in the seeds
    n: int            # input channels (Hessian size)
    rows: int         # output rows of W
    T: int            # calibration columns of X
    lam: float        # starting damping
    w_sigma: float
    outliers: int     # channels scaled by `outlier_scale` (or lognormal when < 0)
    outlier_scale: float
    lognormal_frac: float
    lognormal_sigma: float
    all_lognormal_sigma: float
    dead: int


SPECS = {
    "tiny": Spec("tiny", 1, 256, 512, 2048, 0.01, 0.02, 4, 100.0, 0.0, 0.0, 0.0, 2),
    "attn": Spec("attn", 2, 4096, 4096, 8192, 0.01, 0.02, 0, 1.0, 0.01, 2.0, 0.0, 20),
    "down": Spec("down", 3, 17408, 5120, 32768, 0.01, 0.015, 0, 1.0, 0.0, 0.0, 1.490, 0),
    "batch": Spec("batch", 4, 4096, 4096, 8192, 0.01, 0.02, 0, 1.0, 0.01, 2.0, 0.0, 20),
    "stress": Spec("stress", 5, 8192, 2048, 4096, 1e-6, 0.02, 8, 100.0, 0.0, 0.0, 0.0, 164),
}

CHUNK = 4096


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def channel_scales(spec: Spec, k: int = 0, n: int | None = None, device="cpu"):
    """Per-channel multipliers of X and the dead-channel mask (as a float 0/1 keep vector)."""
    n = spec.n if n is None else n
    gx = _gen(1000 * spec.cfg + 2 * k, device)
    scale = torch.ones(n, dtype=torch.float32, device=device)
    if spec.all_lognormal_sigma > 0:
        z = torch.randn(n, generator=gx, device=device, dtype=torch.float32)
        scale = torch.exp(spec.all_lognormal_sigma * z)
    perm = torch.randperm(n, generator=_gen(1000 * spec.cfg + 100 + k, "cpu"))
    pos = 0
    if spec.outliers:
        idx = perm[pos:pos + spec.outliers]
        scale[idx.to(device)] = spec.outlier_scale
        pos += spec.outliers
    if spec.lognormal_frac > 0:
        m = max(1, int(round(spec.lognormal_frac * n)))
        idx = perm[pos:pos + m].to(device)
        z = torch.randn(m, generator=gx, device=device, dtype=torch.float32)
        scale[idx] = torch.exp(spec.lognormal_sigma * z)
        pos += m
    keep = torch.ones(n, dtype=torch.float32, device=device)
    if spec.dead:
        idx = perm[pos:pos + spec.dead].to(device)
        keep[idx] = 0.0
    return scale, keep, gx


def hessian(spec: Spec, k: int = 0, n: int | None = None, T: int | None = None, device="cpu"):
    """H = X X^T (f32, n x n) with X [n, T] ~ N(0,1) scaled per channel, dead channels zero."""
    n = spec.n if n is None else n
    T = spec.T if T is None else T
    scale, keep, gx = channel_scales(spec, k, n, device)
    mult = (scale * keep).unsqueeze(1)
    H = torch.zeros(n, n, dtype=torch.float32, device=device)
    for t0 in range(0, T, CHUNK):
        tc = min(CHUNK, T - t0)
        X = torch.randn(n, tc, generator=gx, device=device, dtype=torch.float32) * mult
        H.addmm_(X, X.t())
        del X
    return H


def weights(spec: Spec, k: int = 0, rows: int | None = None, n: int | None = None,
            device="cpu"):
    rows = spec.rows if rows is None else rows
    n = spec.n if n is None else n
    gw = _gen(1000 * spec.cfg + 2 * k + 1, device)
    return torch.randn(rows, n, generator=gw, device=device, dtype=torch.float32) * spec.w_sigma


def make(name: str, k: int = 0, device="cpu", n: int | None = None, rows: int | None = None,
         T: int | None = None):
    """(H, W, lam) for a named workload; ``n``/``rows``/``T`` override the sizes (the channel
    picks and seeds stay those of the workload)."""
    if name == "fixture":
        H, W = fixture(device)
        return H, W, 0.01
    spec = SPECS[name]
    H = hessian(spec, k, n=n, T=T, device=device)
    W = weights(spec, k, rows=rows, n=n, device=device)
    return H, W, spec.lam


def _fixture_x():
    n, t = 160, 700
    ri = torch.arange(t).unsqueeze(1)
    ci = torch.arange(n).unsqueeze(0)
    f32 = torch.float32
    base = ((ri * 37 % 101).to(f32) - 50.0) / 29.0
    v = ((ri * 7919 + ci * 104729) % 1009).to(f32) / 1009.0 - 0.5
    loud = torch.where(ci % 41 == 3, torch.tensor(30.0), torch.tensor(1.0)).to(f32)
    x = (v + 0.3 * base) * loud
    x[:, [17, 90]] = 0.0
    return x


def pages_fixture_activations():
    """The activations x [700, 160] (tokens x channels, f32) of the pages' device-versus-host
    test, whose Hessian is sum over tokens of x_r^T x_r; channels 17 and 90 are dead."""
    return _fixture_x().numpy()


def activations(spec: Spec, k: int = 0, T: int | None = None, n: int | None = None,
                device="cpu", seed_offset: int = 7):
    """X [T, n] f32, tokens x channels, with the workload's channel energies and dead channels
    (the layout the Hessian accumulation takes; drawn from its own seed)."""
    n = spec.n if n is None else n
    T = spec.T if T is None else T
    scale, keep, _ = channel_scales(spec, k, n, device)
    g = _gen(1000 * spec.cfg + 2 * k + seed_offset, device)
    X = torch.randn(T, n, generator=g, device=device, dtype=torch.float32)
    return X * (scale * keep).unsqueeze(0)


def fixture(device="cpu"):
    """The pages' device-versus-host test data: n=160 channels, 48 rows, 700 samples
    (element formulas evaluated in f32, the Hessian summed in f64 then stored as f32)."""
    n, rows = 160, 48
    x = _fixture_x()
    f32 = torch.float32
    H = (x.double().t() @ x.double()).float()
    kk = torch.arange(rows * n, dtype=torch.int64)
    w = (((kk * 2654435761) % 2003).to(f32) / 2003.0 - 0.5) * 0.08
    W = w.reshape(rows, n)
    return H.to(device), W.to(device)


def lcg_fixture():
    """The pages' GPTQ-beats-RTN test data ("cortiq-cli 0.8.45 src/gptq.rs", test
    ``gptq_q4tp_beats_rtn_on_output_error``): a 64-bit linear congruential stream, 4 latent
    factors, channel 5 eight times louder.  Returns (H f32 [96, 96], W f32 [24, 96], X [400, 96])."""
    rows, cols, t = 24, 96, 400
    state = [12345]
    mask = (1 << 64) - 1

    def rnd():
        state[0] = (state[0] * 6364136223846793005 + 1442695040888963407) & mask
        return np.float32((state[0] >> 33) / float(1 << 31)) - np.float32(0.5)

    w = np.array([rnd() for _ in range(rows * cols)], dtype=np.float32).reshape(rows, cols)
    lat = np.array([rnd() for _ in range(t * 4)], dtype=np.float32).reshape(t, 4)
    mix = np.array([rnd() for _ in range(4 * cols)], dtype=np.float32).reshape(4, cols)
    x = np.zeros((t, cols), dtype=np.float32)
    for s in range(t):
        for c in range(cols):
            v = np.float32(0.2) * np.float32(rnd())
            for f in range(4):
                v = np.float32(v + lat[s, f] * mix[f, c])
            x[s, c] = v * np.float32(8.0) if c == 5 else v
    h = x.astype(np.float64).T @ x.astype(np.float64)
    return h.astype(np.float32), w, x


def sizes(name: str):
    if name == "fixture":
        return 160, 48
    s = SPECS[name]
    return s.n, s.rows


__all__ = ["SPECS", "Spec", "make", "hessian", "weights", "fixture", "lcg_fixture", "sizes",
           "channel_scales", "activations", "pages_fixture_activations"]
