#!/usr/bin/env python3
"""Benchmark of the GPTQ fold-and-quantize hot path on one MI355X.

One step = gptq_fold (H -> U) + gptq_ladder + gptq_sweep (W, U -> codes, scales) of one
Hessian group, inputs already resident in HBM.  The workload is the down_proj-shaped layer:
n = 17408 input channels, W [5120, 17408] f32, H = X X^T from X [17408, 32768] with lognormal
channel energies, lambda = 0.01, groups of 32 (synthetic, seeded; see workloads/).

Prints one JSON line: groups/s over the timed steps, the roofline of the dominant kernel (the
fold's trailing-update GEMM, timed live with HIP events on its own stream) and the CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense FP32 matrix peak
FP64_MFMA_PEAK_TFLOPS = 78.6    # MI355X dense FP64 matrix peak
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def sweep_bytes_k32(rows: int, n: int) -> float:
    """HBM bytes a sweep that updates the trailing columns once per group (K = 32) would move:
    trailing W read + write, U panel, group read, residual write + read, nibbles / rung / scale.
    The blocked sweep moves far less (the trailing W once per 512 columns), so the rate below is
    an equivalent, not a measured bandwidth; the sweep is bound by its MFMA work."""
    b = 0.0
    for g in range(n // 32):
        rest = n - 32 * (g + 1)
        b += 8.0 * rows * rest + 128.0 * rest
    return b + rows * n * 12.5 + 5.0 * rows * n / 32.0


def sweep_flops(rows: int, n: int) -> float:
    return rows * (n * n - 32.0 * n) + 51.0 * rows * n


def recorded_sweep_dram_bytes():
    """DRAM bytes of one sweep at n = 17408 from the committed counter summary (its sentence
    "Per sweep this is X GB of DRAM traffic"), or None."""
    import re
    try:
        txt = open(os.path.join(ROOT, "profiles", "sweep_hbm_traffic_n17408.md")).read()
    except OSError:
        return None
    m = re.search(r"Per sweep this is ([0-9.]+) GB of DRAM traffic", txt)
    return float(m.group(1)) * 1e9 if m else None


def recorded_traffic():
    """HBM bytes per launch of the fold's bulk update from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), or None when the kernel's sources
    have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "fold_update_traffic_n17408.md")
    try:
        rec = {}
        for line in open(path):
            k, sep, v = line.partition(":")
            if sep and k.strip() in ("traffic_bytes_per_launch", "kernel_sources_sha256",
                                     "kernel_sources"):
                rec[k.strip()] = v.strip()
        h = hashlib.sha256()
        for f in rec["kernel_sources"].split():
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != rec["kernel_sources_sha256"]:
            return None
        return float(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(H, U, hdiag, dead, W, lost, tab, n, rows, m_fold=8192, rows_sweep=1024):
    """The oracle on a bounded sample: the fold of the trailing m x m block of H and the sweep
    of `rows_sweep` rows at full width against the GPU's U, scaled to one whole group."""
    import numpy as np

    import oracle
    nt = oracle.threads()
    Hb = H[n - m_fold:, n - m_fold:].contiguous().cpu().numpy()
    t0 = time.perf_counter()
    f = oracle.fold(Hb, 0.01, nt=nt)
    t_fold = time.perf_counter() - t0
    Ud = U.cpu().numpy().astype(np.float64)
    sel = slice(0, rows_sweep)
    Wn = W[sel].cpu().numpy()
    t0 = time.perf_counter()
    oracle.sweep(Wn, Ud, hdiag.cpu().numpy(), dead.cpu().numpy().astype(bool),
                 tab[sel].cpu().numpy(), lost[sel].cpu().numpy(), want_E=False, nt=nt)
    t_sweep = time.perf_counter() - t0
    del Ud
    t_group = t_fold * (n / m_fold) ** 3 + t_sweep * rows / rows_sweep
    return {
        "value": 1.0 / t_group, "unit": "groups/s", "cores": nt, "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"fold of the trailing {m_fold}x{m_fold} block of H ({t_fold:.2f} s, scaled by "
                   f"(n/{m_fold})^3) + sweep of {rows_sweep} of {rows} rows at n={n} against the "
                   f"GPU's U ({t_sweep:.2f} s, scaled by rows); f64, {nt} threads; status "
                   f"{f['status']}"),
    }


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def all_configs(pwq, torch, dev):
    """One record per workload of the method's configurations: GPU fold / sweep times, the
    fold's damping, attempts and precision, parity figures against the oracle, and the oracle's
    own times on the host cores.  Printed as one JSON line ({"configs": [...]}) plus a table on
    stderr; the numbers behind the per-configuration table of the design notes."""
    import numpy as np

    import oracle
    import workloads
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import fold_rel_err, hd_diag, output_error

    nt = oracle.threads()
    recs = []

    def gpu_step_times(H, W, lam, reps):
        n, rows = H.shape[0], W.shape[0]
        ws_f = torch.empty(pwq.fold_workspace_size(n), dtype=torch.uint8, device=dev)
        ws_s = torch.empty(pwq.sweep_workspace_size(rows, n), dtype=torch.uint8, device=dev)
        U = torch.empty(n, n, device=dev)
        hd = torch.empty(n, device=dev)
        dd = torch.empty(n, dtype=torch.uint8, device=dev)
        lost = torch.empty(rows, 2, device=dev)
        tab = torch.empty(rows, 32, device=dev)
        out = (torch.empty(rows, n // 2, dtype=torch.uint8, device=dev),
               torch.empty(rows, n // 32, dtype=torch.uint8, device=dev),
               torch.empty(rows, n // 32, device=dev), None)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        tf, tsw = [], []
        for i in range(reps + 2):
            ev[0].record()
            _, _, _, rep = pwq.gptq_fold(H, lam, workspace=ws_f, out=(U, hd, dd))
            ev[1].record()
            pwq.gptq_ladder(W, dd, out=(lost, tab))
            pwq.gptq_sweep(W, U, hd, dd, tab, lost, workspace=ws_s, out=out)
            ev[2].record()
            torch.cuda.synchronize()
            if i >= 2:
                tf.append(ev[0].elapsed_time(ev[1]))
                tsw.append(ev[1].elapsed_time(ev[2]))
        return float(np.median(tf)), float(np.median(tsw)), rep, (U, hd, dd, lost, tab) + out[:3]

    for name in ("tiny", "attn", "down", "stress"):
        spec = workloads.SPECS[name]
        H, W, lam = workloads.make(name, device=dev)
        torch.cuda.synchronize()
        n, rows = spec.n, spec.rows
        log(f"config {name}: n={n} rows={rows}")
        t_fold, t_sweep, rep, (U, hd, dd, lost, tab, nib, rung, scale) = gpu_step_times(
            H, W, lam, 3 if name == "down" else 5)
        rec = dict(workload=name, n=n, rows=rows, lambda_start=lam, lambda_used=rep["lambda_used"],
                   attempts=rep["attempts"], precision=rep["precision"], min_pivot=rep["min_pivot"],
                   gpu_fold_ms=t_fold, gpu_sweep_ms=t_sweep,
                   gpu_groups_per_s=1e3 / (t_fold + t_sweep),
                   fold_tflops=2.0 * n ** 3 / 3.0 / (t_fold * 1e-3) / 1e12)
        rec["fold_frac_peak"] = rec["fold_tflops"] / (FP32_MFMA_PEAK_TFLOPS if rep["precision"] == 32
                                                      else FP64_MFMA_PEAK_TFLOPS)
        rec["sweep_tflops"] = sweep_flops(rows, n) / (t_sweep * 1e-3) / 1e12
        Hn, Wn = H.cpu().numpy(), W.cpu().numpy()
        if name != "down":
            # Parity and the oracle's own time on the whole workload.
            t0 = time.perf_counter()
            of = oracle.fold(Hn, lam, nt=nt)
            t_ofold = time.perf_counter() - t0
            Ug = U.cpu().numpy()
            og = of if of["lam"] == rep["lambda_used"] else oracle.fold(Hn, rep["lambda_used"], retry=False, nt=nt)
            rec["fold_relF"] = fold_rel_err(Ug, og["U"], np.sqrt(hd_diag(Hn, og["dead"], og["damp"])))
            rec["oracle_lambda"] = of["lam"]
            lo, tb = oracle.ladder(Wn, of["dead"])
            t0 = time.perf_counter()
            os_ = oracle.sweep(Wn, of["U"], of["hdiag"], of["dead"], tb, lo, want_E=False, nt=nt)
            t_osweep = time.perf_counter() - t0
            code_g = oracle.unpack_nibbles(nib.cpu().numpy())
            rp = oracle.sweep(Wn, Ug.astype(np.float64), hd.cpu().numpy(), dd.cpu().numpy().astype(bool),
                              tab.cpu().numpy(), lost.cpu().numpy(), force_code=code_g,
                              force_rung=rung.cpu().numpy(), want_E=False, nt=nt)
            st_ = rp["stats"]
            rec["sweep_hard"] = st_["code_hard"] + st_["rung_hard"]
            rec["sweep_replay_agree"] = 1.0 - (st_["code_ties"] + st_["code_hard"]) / code_g.size
            t_o = oracle.output_error(Wn, of["dead"], os_["code"], os_["scale"], Hn)
            t_g = output_error(Wn, of["dead"], nib.cpu().numpy(), scale.cpu().numpy(), Hn)
            rec["output_error_rel"] = (t_g - t_o) / t_o
            rec.update(oracle_fold_s=t_ofold, oracle_sweep_s=t_osweep,
                       oracle_groups_per_s=1.0 / (t_ofold + t_osweep), oracle_threads=nt)
            if name == "tiny":
                t0 = time.perf_counter()
                of1 = oracle.fold(Hn, lam, nt=1)
                oracle.sweep(Wn, of1["U"], of1["hdiag"], of1["dead"], tb, lo, want_E=False, nt=1)
                rec["oracle_1thread_s"] = time.perf_counter() - t0
        else:
            cb = cpu_baseline(H, U, hd, dd, W, lost, tab, n, rows)
            rec.update(oracle_groups_per_s=cb["value"], oracle_threads=nt, oracle_sample=cb["sample"],
                       parity="whole-layer parity: tests/test_gpu_parity_large.py::test_down_proj_full_size")
        rec["speedup_vs_oracle"] = rec["gpu_groups_per_s"] / rec["oracle_groups_per_s"]
        recs.append(rec)
        del H, W, U
        torch.cuda.empty_cache()
    # Config 4: 11 groups of the attention shape.  GPU: the library's round (gptq_round).
    # Oracle: the groups concurrently with the host threads split between them, as the pages'
    # host round runs them.
    spec = workloads.SPECS["batch"]
    groups = [workloads.make("batch", k=k, device=dev) for k in range(11)]
    rnd = pwq.Round([{"H": H, "lam": lam, "members": [W]} for H, W, lam in groups])
    torch.cuda.synchronize()
    rnd.run()
    torch.cuda.synchronize()
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        rnd.run()
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    t_round = float(np.median(ts))
    gpu_conc = rnd.plan()[1]
    del rnd
    conc = 4
    per = max(nt // conc, 1)
    host = [(H.cpu().numpy(), W.cpu().numpy(), lam) for H, W, lam in groups]

    def orc_group(k):
        Hn, Wn, lam = host[k]
        of = oracle.fold(Hn, lam, nt=per)
        lo, tb = oracle.ladder(Wn, of["dead"])
        oracle.sweep(Wn, of["U"], of["hdiag"], of["dead"], tb, lo, want_E=False, nt=per)

    import concurrent.futures as cf
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(conc) as ex:
        list(ex.map(orc_group, range(11)))
    t_orc = time.perf_counter() - t0
    recs.append(dict(workload="batch", n=spec.n, rows=spec.rows, groups=11,
                     gpu_round_ms=t_round * 1e3, gpu_groups_per_s=11 / t_round,
                     gpu_concurrency=gpu_conc,
                     oracle_round_s=t_orc, oracle_groups_per_s=11 / t_orc,
                     oracle_threads=nt, oracle_concurrency=f"{conc} groups at a time, {per} threads each",
                     speedup_vs_oracle=(11 / t_round) / (11 / t_orc)))
    out = {"cpu_model": cpu_model(), "host_threads": nt, "configs": recs}
    for r in recs:
        log(json.dumps(r))
    print(json.dumps(out), flush=True)


def round_only(pwq, torch, dev, steps, warmup):
    """The batched round of 11 groups of the attention shape (n 4096, W 4096 x 4096, distinct
    seeds) through gptq_round with its default plan; groups/s over the timed rounds."""
    import workloads
    groups = [workloads.make("batch", k=k, device=dev) for k in range(11)]
    rnd = pwq.Round([{"H": H, "lam": lam, "members": [W]} for H, W, lam in groups])
    torch.cuda.synchronize()
    for i in range(max(warmup, 1)):
        st = rnd.run()
        torch.cuda.synchronize()
        if st != pwq.GPTQ_OK:
            raise pwq.GptqError(st, "gptq_round")
        log(f"warmup round {i + 1} done")
    t0 = time.perf_counter()
    for _ in range(steps):
        rnd.run()
        torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"workload": "batch: 11 groups, n=4096, W[4096,4096] f32", "rounds": steps,
                      "ms_per_round": dt * 1e3, "groups_per_s": 11 / dt,
                      "slots": rnd.plan()[1]}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="down")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gram", action="store_true", help="skip the Hessian accumulation timing")
    ap.add_argument("--no-packed", action="store_true",
                    help="skip the timing of the fold from a packed Hessian")
    ap.add_argument("--no-debias", action="store_true", help="skip the output debias timing")
    ap.add_argument("--no-act-order", action="store_true", help="skip the act-order timing")
    ap.add_argument("--no-q2", action="store_true", help="skip the q2tp sweep timing")
    ap.add_argument("--no-rounds", action="store_true", help="skip the concurrent-group timings")
    ap.add_argument("--all-configs", action="store_true",
                    help="instead of the benchmark line: one record per configuration of the "
                         "method (GPU times, damping, parity, oracle times)")
    ap.add_argument("--round-only", action="store_true",
                    help="instead of the benchmark line: time only the batched round of 11 "
                         "attention-shaped groups (gptq_round, its default plan) and print one "
                         "record")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one plain 1 GiB device copy first (a known-size reference for "
                         "hardware traffic counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the fold and sweep of a Hessian group run on a single "
              "MI355X (groups are independent; see the multi-GPU notes in the design); run it "
              "with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import post_weight_quantization_amd as pwq
    import workloads

    pwq.require_native()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.all_configs:
        all_configs(pwq, torch, dev)
        return
    if args.round_only:
        round_only(pwq, torch, dev, args.steps, args.warmup)
        return
    spec = workloads.SPECS[args.workload]
    n, rows = spec.n, spec.rows
    log(f"generating workload {args.workload}: n={n} rows={rows} T={spec.T}")
    t0 = time.perf_counter()
    H, W, lam = workloads.make(args.workload, device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")

    if args.calib_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read + 1 GiB written")
        del src, dst

    U = torch.empty(n, n, dtype=torch.float32, device=dev)
    hdiag = torch.empty(n, dtype=torch.float32, device=dev)
    dead = torch.empty(n, dtype=torch.uint8, device=dev)
    lost = torch.empty(rows, 2, dtype=torch.float32, device=dev)
    tab = torch.empty(rows, 32, dtype=torch.float32, device=dev)
    nib = torch.empty(rows, n // 2, dtype=torch.uint8, device=dev)
    rung = torch.empty(rows, n // 32, dtype=torch.uint8, device=dev)
    scale = torch.empty(rows, n // 32, dtype=torch.float32, device=dev)
    ws_f = torch.empty(pwq.fold_workspace_size(n), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(pwq.sweep_workspace_size(rows, n), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    phase_ms = {"fold": 0.0, "ladder": 0.0, "sweep": 0.0}
    reports = []

    def step(record):
        if record:
            ev[0].record(stream)
        _, _, _, rep = pwq.gptq_fold(H, lam, workspace=ws_f, out=(U, hdiag, dead))
        if record:
            ev[1].record(stream)
        pwq.gptq_ladder(W, dead, out=(lost, tab))
        if record:
            ev[2].record(stream)
        pwq.gptq_sweep(W, U, hdiag, dead, tab, lost, workspace=ws_s,
                       out=(nib, rung, scale, None))
        if record:
            ev[3].record(stream)
        reports.append(rep)

    for i in range(args.warmup):
        step(False)
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")

    pwq.profile_enable(["fold_update"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(True)
        ev[3].synchronize()
        phase_ms["fold"] += ev[0].elapsed_time(ev[1])
        phase_ms["ladder"] += ev[1].elapsed_time(ev[2])
        phase_ms["sweep"] += ev[2].elapsed_time(ev[3])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    pwq.profile_enable([])
    prof = pwq.profile_collect()
    elapsed = t1 - t0
    K = args.steps
    log(f"timed {K} steps in {elapsed:.3f} s")

    fold_ms = phase_ms["fold"] / K
    sweep_ms = phase_ms["sweep"] / K
    ladder_ms = phase_ms["ladder"] / K
    fold_flops = 2.0 * n ** 3 / 3.0
    fu = prof["fold_update"]
    achieved = fu["flops"] / (fu["ms"] * 1e-3) / 1e12 if fu["ms"] > 0 else 0.0
    rep = reports[-1]
    result = {
        "metric": "Hessian groups/s + fold TFLOP/s (%FP32 MFMA peak) at n=17408; sweep GB/s",
        "value": K / elapsed,
        "unit": "groups/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: down_proj-shaped layer, n={n}, "
                               f"W[{rows},{n}] f32, H=X X^T from X[{n},{spec.T}]",
                   "n": n, "rows": rows, "lambda": lam, "group": 32},
        "roofline": {
            "kernel": "gemm_kernel<0> (the fold's bulk updates: Cholesky SYRK, then the inverse update, on one helper stream)",
            "bound": "mfma", "achieved": achieved, "peak": FP32_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / FP32_MFMA_PEAK_TFLOPS,
            "traffic": recorded_traffic(),
            "traffic_note": "HBM bytes per launch: rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 "
                            "(factors from a plain 1 GiB copy); null once the kernel changed",
            "launches": fu["launches"], "avg_launch_us": 1e3 * fu["ms"] / max(fu["launches"], 1),
            "flops_per_launch": fu["flops"] / max(fu["launches"], 1),
        },
        "detail": {
            "fold_ms": fold_ms, "ladder_ms": ladder_ms, "sweep_ms": sweep_ms,
            "fold_tflops": fold_flops / (fold_ms * 1e-3) / 1e12,
            "fold_frac_fp32_mfma": fold_flops / (fold_ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS,
            "sweep_k32_equivalent_rate_gbps": sweep_bytes_k32(rows, n) / (sweep_ms * 1e-3) / 1e9,
            "sweep_k32_equivalent_note": "not a bandwidth: the bytes a per-group (K = 32) sweep "
                                         "would move, over the time of this blocked (K = 512) "
                                         "sweep, which moves about 8x fewer; see sweep_roofline",
            "sweep_tflops": sweep_flops(rows, n) / (sweep_ms * 1e-3) / 1e12,
            "sweep_frac_fp32_mfma": sweep_flops(rows, n) / (sweep_ms * 1e-3) / 1e12
                                    / FP32_MFMA_PEAK_TFLOPS,
            "lambda_used": rep["lambda_used"], "attempts": rep["attempts"],
            "n_dead": rep["n_dead"], "fold_precision": rep["precision"],
            "fold_min_pivot": rep["min_pivot"],
        },
    }
    # The sweep's own roofline.  Reassociated into 512-column panels its trailing updates are
    # K = 512 products (MFMA-bound); the HBM target of a per-group sweep does not describe it.
    sweep_tf = sweep_flops(rows, n) / (sweep_ms * 1e-3) / 1e12
    dram = recorded_sweep_dram_bytes() if n == 17408 and rows == 5120 else None
    result["sweep_roofline"] = {
        "bound": "mfma", "achieved": sweep_tf, "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": sweep_tf / FP32_MFMA_PEAK_TFLOPS,
        "flops": sweep_flops(rows, n),
        "dram_bytes_counters": dram,
        "dram_gbps": dram / (sweep_ms * 1e-3) / 1e9 if dram else None,
        "dram_frac_hbm": dram / (sweep_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS if dram else None,
        "note": "flops rows (n^2 - 32 n) + 51 rows n over the whole sweep; DRAM bytes from the "
                "committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary at this workload",
    }
    # The device Hessian accumulation (a next-step row of the path, not part of the step):
    # H += X^T X for X [T, n] tokens x channels at the same shape, timed alone on the stream.
    if not args.no_gram:
        Xg = workloads.activations(spec, device=dev)
        Hg = torch.zeros(n, n, dtype=torch.float32, device=dev)
        pwq.gptq_gram_add(Hg, Xg)
        torch.cuda.synchronize()
        reps = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            pwq.gptq_gram_add(Hg, Xg)
        e1.record(stream)
        e1.synchronize()
        gram_ms = e0.elapsed_time(e1) / reps
        gram_flops = float(n) * (n + 1) * Xg.shape[0]
        result["detail"]["gram_ms"] = gram_ms
        result["detail"]["gram_tflops"] = gram_flops / (gram_ms * 1e-3) / 1e12
        result["detail"]["gram_frac_fp32_mfma"] = result["detail"]["gram_tflops"] / FP32_MFMA_PEAK_TFLOPS
        result["detail"]["gram_shape"] = f"H[{n},{n}] += X^T X, X[{Xg.shape[0]},{n}]"
        del Hg
        # The same accumulation into the packed upper triangle (half the bytes of H).
        Hpk = torch.zeros(n * (n + 1) // 2, dtype=torch.float32, device=dev)
        pwq.gptq_gram_add(Hpk, Xg)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            pwq.gptq_gram_add(Hpk, Xg)
        e1.record(stream)
        e1.synchronize()
        result["detail"]["gram_packed_ms"] = e0.elapsed_time(e1) / reps
        del Xg, Hpk
    # The fold of the same Hessian handed over as its packed upper triangle.
    if not args.no_packed:
        iu = torch.triu_indices(n, n, device=dev)
        Hpk = H[iu[0], iu[1]].contiguous()
        del iu
        pwq.gptq_fold(Hpk, lam, workspace=ws_f, out=(U, hdiag, dead))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(2):
            pwq.gptq_fold(Hpk, lam, workspace=ws_f, out=(U, hdiag, dead))
        e1.record(stream)
        e1.synchronize()
        result["detail"]["fold_packed_ms"] = e0.elapsed_time(e1) / 2
        del Hpk
    # Concurrent groups (the batched round): G independent groups through the library's round
    # (gptq_round's default plan: groups of one shape run as one gang, in lockstep), outputs and
    # workspace allocated once; groups/s over whole rounds.
    def concurrent_round(name, G, rounds):
        groups_ = []
        for kk in range(G):
            Hg_, Wg_, lam_g = workloads.make(name, k=kk, device=dev)
            groups_.append({"H": Hg_, "lam": lam_g, "members": [Wg_]})
        rnd = pwq.Round(groups_)
        torch.cuda.synchronize()
        st_ = rnd.run()
        torch.cuda.synchronize()
        if st_ != pwq.GPTQ_OK:
            raise pwq.GptqError(st_, "gptq_round")
        t0_ = time.perf_counter()
        for _ in range(rounds):
            rnd.run()
            torch.cuda.synchronize()
        dt_ = (time.perf_counter() - t0_) / rounds
        conc_ = rnd.plan()[1]
        del rnd, groups_
        torch.cuda.empty_cache()
        return G / dt_, dt_ * 1e3, conc_

    if not args.no_rounds:
        gps, ms, conc = concurrent_round("batch", 11, 3)
        result["detail"]["batched_round_11x4096_groups_per_s"] = gps
        result["detail"]["batched_round_11x4096_ms"] = ms
        result["detail"]["batched_round_concurrency"] = conc
        gps2, ms2, _ = concurrent_round("down", 2, 2)
        result["detail"]["concurrent_2x17408_groups_per_s"] = gps2
        result["detail"]["concurrent_2x17408_ms_per_pair"] = ms2
    # The q2tp sweep ("placed" rule) on the step's U (a next-step row, not part of the step).
    if not args.no_q2:
        lost_q, tab_q = pwq.gptq_ladder_q2(W, dead)
        out_q = pwq.gptq_sweep_q2(W, U, hdiag, dead, tab_q, workspace=ws_s)
        torch.cuda.synchronize()
        reps = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            pwq.gptq_sweep_q2(W, U, hdiag, dead, tab_q, workspace=ws_s)
        e1.record(stream)
        e1.synchronize()
        result["detail"]["q2_sweep_ms"] = e0.elapsed_time(e1) / reps
        # ... and the 2-bit output debias of those codes.
        if not args.no_debias:
            ws_dq = torch.empty(pwq.debias_workspace_size(rows, n), dtype=torch.uint8, device=dev)
            plane_q, rung_q, scale_q, _ = out_q
            lost_dq, scale_dq = lost_q.clone(), scale_q.clone()
            pwq.gptq_debias_q2(W, H, dead, plane_q, rung_q, lost_dq, scale_dq, workspace=ws_dq)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                lost_dq.copy_(lost_q)
                scale_dq.copy_(scale_q)
                pwq.gptq_debias_q2(W, H, dead, plane_q, rung_q, lost_dq, scale_dq, workspace=ws_dq)
            e1.record(stream)
            e1.synchronize()
            result["detail"]["debias_q2_ms"] = e0.elapsed_time(e1) / reps
            del ws_dq, lost_dq, scale_dq
        del out_q
    # Act-order GPTQ on the same layer (a next-step row, not part of the step): channel order,
    # permuted Hessian, fold of it, ladder and the static-group sweep, timed as one group.
    if not args.no_act_order:
        ws_a = torch.empty(pwq.sweep_act_order_workspace_size(rows, n), dtype=torch.uint8,
                           device=dev)

        def ao_step(two_bit):
            perm_a, dead_a = pwq.gptq_act_order_perm(H)
            Hp_a = pwq.gptq_permute_hessian(H, perm_a)
            Ua, hd_a, _, rep_a = pwq.gptq_fold(Hp_a, lam, workspace=ws_f)
            del Hp_a
            if two_bit:
                _, tab_a = pwq.gptq_ladder_q2(W, dead_a)
                pwq.gptq_sweep_act_order_q2(W, Ua, dead_a, hd_a, perm_a, tab_a, workspace=ws_a)
            else:
                lost_a, tab_a = pwq.gptq_ladder(W, dead_a)
                pwq.gptq_sweep_act_order(W, Ua, dead_a, perm_a, tab_a, lost_a, workspace=ws_a)
            return rep_a

        for two_bit, key in ((False, "act_order"), (True, "act_order_q2")):
            ao_step(two_bit)
            torch.cuda.synchronize()
            reps = 2
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                rep_a = ao_step(two_bit)
            e1.record(stream)
            e1.synchronize()
            result["detail"][f"{key}_ms"] = e0.elapsed_time(e1) / reps
            result["detail"][f"{key}_groups_per_s"] = 1e3 / result["detail"][f"{key}_ms"]
            result["detail"][f"{key}_lambda_used"] = rep_a["lambda_used"]
        del ws_a
    # The output debias on the step's codes (a next-step row of the path, not part of the step):
    # symmetrised H, the product W H and the per-row slopes, timed alone on the stream.
    if not args.no_debias:
        ws_d = torch.empty(pwq.debias_workspace_size(rows, n), dtype=torch.uint8, device=dev)
        lost_d, scale_d = lost.clone(), scale.clone()
        pwq.gptq_debias(W, H, dead, nib, rung, lost_d, scale_d, workspace=ws_d)
        torch.cuda.synchronize()
        reps = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            lost_d.copy_(lost)
            scale_d.copy_(scale)
            pwq.gptq_debias(W, H, dead, nib, rung, lost_d, scale_d, workspace=ws_d)
        e1.record(stream)
        e1.synchronize()
        debias_ms = e0.elapsed_time(e1) / reps
        result["detail"]["debias_ms"] = debias_ms
        result["detail"]["debias_gemm_tflops_whole_call"] = 2.0 * rows * n * n / (debias_ms * 1e-3) / 1e12
        del ws_d, lost_d, scale_d
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        result["cpu_baseline"] = cpu_baseline(H, U, hdiag, dead, W, lost, tab, n, rows)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
