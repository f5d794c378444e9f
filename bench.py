"""Benchmark of the owner-side Muon step (+ AdamW tail) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = muon_owner_step over the workload's whole bucket of matrices plus
adamw_tail_step over its packed fp32 tail, inputs already resident in HBM.
Prints one JSON line.  `value` is Newton-Schulz TFLOP/s with the nominal count
4 m^2 n + 2 m^3 per iteration and matrix (m = short side), from the wall time
of K steps; `roofline` is the dominant kernel's algorithmic throughput from
HIP events recorded around every launch of a second timed pass of the same K
steps (event markers would otherwise add gaps to the first); `cpu_baseline` is
the fp64 oracle timed on the host on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Muon owner-step ms + Newton–Schulz TFLOP/s (% bf16 MFMA peak), 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3         # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
PEAK_F64_TFLOPS = 78.6          # MI355X fp64 (vector FMA)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="large_single",
                    help="Muon workload (default large_single: 28672x8192, 8192x28672 and a "
                         "128256x4096 head, the largest configuration that fits one GPU)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-phase-timing", action="store_true",
                    help="skip the second, event-instrumented pass (no phases, no roofline object)")
    ap.add_argument("--profile-only", action="store_true",
                    help="warmup + timed steps only, no oracle leg (for profilers)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the step, time the library's plain copy kernel over "
                         "MIB mebibytes (HBM ceiling; byte-counter calibration)")
    ap.add_argument("--optimizer", default="muon", choices=["muon", "shampoo", "soap"],
                    help="shampoo: time the Shampoo owner step instead (workload "
                         "shampoo_decoder_layer_h2048 unless --workload names another Shampoo one); "
                         "soap: the SOAP owner step (workload soap_decoder_layer_h2048)")
    ap.add_argument("--graph", action="store_true",
                    help="capture the Muon step (the allocation-free entry point) once in a HIP graph and "
                         "time its replays (for launch-bound buckets); no per-phase timing")
    ap.add_argument("--adamw-sweep", action="store_true",
                    help="instead of the step, time adamw_tail_step over n = 2^24 .. 2^28 "
                         "fp32 elements (28 bytes moved per element) and print one JSON line per n")
    return ap.parse_args()


def adamw_sweep(args):
    """HBM throughput of the AdamW tail kernel at sizes where it is bandwidth-bound
    (the workloads' own tails are a few thousand elements and launch-bound)."""
    import torch
    import matrix_optimizers_amd as mo
    from matrix_optimizers_amd import workloads as wlmod
    a = wlmod.AdamWHP()
    for e in range(24, 29):
        n = 1 << e
        gen = torch.Generator(device="cuda").manual_seed(e)
        p = torch.randn(n, device="cuda", generator=gen) * 0.02
        g = torch.randn(n, device="cuda", generator=gen) * 1e-3
        m = torch.randn(n, device="cuda", generator=gen) * 1e-3
        v = (torch.randn(n, device="cuda", generator=gen) * 1e-3) ** 2
        for w in range(max(args.warmup, 1)):
            mo.adamw_tail_step(p, g, m, v, w + 1, lr=a.lr, beta1=a.beta1, beta2=a.beta2, eps=a.eps,
                               weight_decay=a.weight_decay)
        torch.cuda.synchronize()
        mo.profile_read()
        mo.profile_enable(True)
        for k in range(args.steps):
            mo.adamw_tail_step(p, g, m, v, k + 10, lr=a.lr, beta1=a.beta1, beta2=a.beta2, eps=a.eps,
                               weight_decay=a.weight_decay)
        torch.cuda.synchronize()
        mo.profile_enable(False)
        tot, cnt = mo.profile_read()["adamw"]
        per = tot / cnt
        gbs = 28.0 * n / (per * 1e-3) / 1e9
        print(json.dumps({"metric": "AdamW tail HBM throughput", "n": n, "bytes_per_launch": 28 * n,
                          "avg_ms": round(per, 5), "GBps": round(gbs, 1),
                          "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}), flush=True)
        del p, g, m, v


def copy_calibration(args):
    """Times mo_device_copy over a buffer of known size: the measured HBM copy
    ceiling, and the reference transfer for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    import matrix_optimizers_amd as mo
    nbytes = args.copy_calibration << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(max(args.warmup, 1)):
        mo.device_copy(dst, src)
    torch.cuda.synchronize()
    mo.profile_read()
    mo.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        mo.device_copy(dst, src)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    mo.profile_enable(False)
    tot, cnt = mo.profile_read()["copy"]
    assert torch.equal(dst, src)
    per = tot / cnt
    out = {"metric": "device copy bandwidth (read + write)", "bytes_per_launch": 2 * nbytes,
           "avg_ms": round(per, 5), "GBps": round(2 * nbytes / (per * 1e-3) / 1e9, 1),
           "wall_ms_per_launch": round((t1 - t0) * 1e3 / args.steps, 5), "peak_GBps": PEAK_HBM_GBS}
    print(json.dumps(out), flush=True)


def timed_steps(fn, steps):
    """Wall ms per step over `steps` calls, synchronized on both sides."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def event_timed_steps(fn, steps, per_step=None):
    """The same steps with every library launch bracketed by HIP events on its
    stream; returns ({phase: (total ms, launches)}, wall ms per step).  With a
    list `per_step`, it also receives each step's duration in ms from events
    recorded on the current stream (the launch stream) between steps."""
    import torch
    import matrix_optimizers_amd as mo
    mo.profile_read()               # drop anything recorded before
    mo.profile_enable(True)
    if per_step is None:
        ms = timed_steps(fn, steps)
    else:
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs[0].record()
        for k in range(steps):
            fn()
            evs[k + 1].record()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        per_step.extend(evs[k].elapsed_time(evs[k + 1]) for k in range(steps))
    mo.profile_enable(False)
    return mo.profile_read(), ms


def machine_info(query_smi=True):
    """ROCm / HIP version, gfx target and the shader clock and package power that
    rocm-smi reports right after the timed region (best effort: None where a tool
    is missing).  With query_smi False (--profile-only runs) no subprocess is
    started: under a profiler every child process initialises the GPU too, and
    rocm-smi, a script, would then be started by exec from such a child."""
    import subprocess
    import torch
    info = {"hip": getattr(torch.version, "hip", None), "torch": torch.__version__}
    try:
        info["gfx"] = torch.cuda.get_device_properties(0).gcnArchName
    except Exception:
        info["gfx"] = None
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    if not query_smi:
        info["sclk_after_run"] = info["power_after_run"] = None
        return info
    try:
        out = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                             timeout=20).stdout
        d = json.loads(out)
        card = next(iter(d.values()))
        info["sclk_after_run"] = card.get("sclk clock speed:")
        info["mclk_after_run"] = card.get("mclk clock speed:")
    except Exception:
        info["sclk_after_run"] = None
    try:   # package power and its cap, as rocm-smi names them
        out = subprocess.run(["rocm-smi", "--showpower", "--showmaxpower", "--json"], capture_output=True,
                             text=True, timeout=20).stdout
        card = next(iter(json.loads(out).values()))
        info["power_after_run"] = {k: v for k, v in card.items() if "ower" in k} or None
    except Exception:
        info["power_after_run"] = None
    return info


def algorithmic_flops(spec_rows, spec_cols, steps):
    """Per phase, one launch: Gram m^2 n (one triangle), Poly m^3 (one triangle),
    Update 2 m^2 n (dense)."""
    m, n = min(spec_rows, spec_cols), max(spec_rows, spec_cols)
    return {"gram": float(m) * m * n, "poly": float(m) ** 3, "update": 2.0 * m * m * n}


# copies of X0 the momentum kernel writes beyond the one the step needs (its transpose)
MOMENTUM_EXTRA_COPIES = 1

CPU_BUDGET_S = 20.0          # oracle work per bench run
ORACLE_TFLOPS_GUESS = 0.5    # fp64 numpy on the measuring machine's host, for sizing the sample only


def cpu_baseline(wl, args):
    """The fp64 oracle on a bounded sample of the workload: one matrix of each
    distinct shape, smallest first, while the estimated time stays within
    CPU_BUDGET_S (at least one matrix; if even the smallest would overrun, it
    runs with fewer Newton-Schulz steps), plus the AdamW tail."""
    import dataclasses
    import numpy as np
    from matrix_optimizers_amd import workloads as wlmod
    from oracle import adamw as oadamw
    from oracle import muon as omuon
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    seen, shapes = set(), []
    for i, s in enumerate(wl.matrices):
        if (s.rows, s.cols) not in seen:
            seen.add((s.rows, s.cols))
            shapes.append(i)
    per = lambda i, k: wlmod.ns_flops_nominal(wl.matrices[i].rows, wl.matrices[i].cols, k)
    shapes.sort(key=lambda i: per(i, wl.hp.ns_steps))
    sample, est = [], 0.0
    for i in shapes:
        t = per(i, wl.hp.ns_steps) / (ORACLE_TFLOPS_GUESS * 1e12)
        if sample and est + t > CPU_BUDGET_S:
            break
        sample.append(i)
        est += t
    hp = wl.hp
    if est > CPU_BUDGET_S and hp.ns_steps > 1:
        k = max(1, int(hp.ns_steps * CPU_BUDGET_S / est))
        hp = dataclasses.replace(hp, ns_steps=k)
    inputs = [wlmod.matrix_inputs(wl, i) for i in sample]
    tail = wlmod.tail_inputs(wl.seed, wl.tail_numel) if wl.tail_numel else None
    flops = sum(per(i, hp.ns_steps) for i in sample)

    def run_sample():
        t0 = time.perf_counter()
        for x in inputs:
            omuon.muon_step(x.W, x.G, x.M, hp)
        if tail is not None:
            a = wl.adamw
            oadamw.adamw_step(tail.p, tail.g, tail.m, tail.v, a.step, a.lr, a.beta1, a.beta2, a.eps,
                              a.weight_decay)
        return time.perf_counter() - t0

    dt = run_sample()
    single = None
    if wl.key in SINGLE_CORE_WORKLOADS:   # the small buckets: the same sample on one core as well
        try:
            import threadpoolctl
            with threadpoolctl.threadpool_limits(limits=1):
                dt1 = run_sample()
            single = {"value": flops / dt1 / 1e12, "unit": "TFLOP/s", "cores": 1, "seconds": round(dt1, 2),
                      "note": "the same sample with the BLAS pool limited to one thread"}
        except Exception as e:   # no BLAS pool control: say so instead of guessing
            single = {"value": None, "note": f"not measured: {type(e).__name__}"}
    desc = ", ".join(f"{wl.matrices[i].rows}x{wl.matrices[i].cols}" for i in sample)
    if len(sample) == len(shapes) and hp.ns_steps == wl.hp.ns_steps:
        what = f"one whole matrix of each distinct shape ({desc}), full step"
    else:
        what = (f"{len(sample)} whole matrix{'es' if len(sample) > 1 else ''} of the bucket ({desc}): "
                f"momentum, normalisation and {hp.ns_steps} of the {wl.hp.ns_steps} Newton-Schulz steps")
    total = sum(wlmod.ns_flops_nominal(m.rows, m.cols, wl.hp.ns_steps) for m in wl.matrices)
    out = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
           "sample": what
                     + (f" + the {wl.tail_numel}-element AdamW tail" if wl.tail_numel else "")
                     + f"; fp64 numpy, {dt:.2f} s; rate = nominal NS flops of what ran / time",
           "projected_full_step_s": round(dt * total / flops, 1),
           "projection_note": "the whole bucket at the sample's rate (a projection, not a measurement)",
           "host": host_cpu()}
    if single is not None:
        out["single_core"] = single
    return out


# Buckets small enough to time the oracle sample on one core too.
SINGLE_CORE_WORKLOADS = ("single_256x512_f32", "decoder_layer_h2048")


def host_cpu():
    """The host's CPU model and the CPUs this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "usable_cpus": usable, "os_cpu_count": os.cpu_count()}


SHAMPOO_METRIC = "Shampoo owner-step ms + fp32 TFLOP/s (algorithmic, % fp32 MFMA peak), 1 MI355X"


def shampoo_cpu_baseline(wl):
    """The fp64 oracle's Shampoo step on the workload's smallest matrix (its
    coupled Newton roots are 8 m^3 flops per step and side, plain matmuls)."""
    import numpy as np
    from matrix_optimizers_amd import workloads as wlmod
    from oracle import shampoo as osh
    try:
        import threadpoolctl
        cores = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    i = min(range(len(wl.matrices)), key=lambda k: wl.matrices[k].rows * wl.matrices[k].cols)
    W, G, L, R = wlmod.shampoo_inputs(wl, i)
    hp = wl.hp
    r, c = G.shape
    t0 = time.perf_counter()
    osh.shampoo_step(W, G, L, R, hp.lr, hp.weight_decay, "newton", hp.root_iters)
    dt = time.perf_counter() - t0
    f = wlmod.shampoo_flops_algorithmic(r, c, hp.root_iters)
    flops = sum(f.values())
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"one {r}x{c} matrix of the bucket, {hp.root_iters} coupled Newton steps per root, "
                      f"fp64 numpy, {dt:.2f} s (same algorithmic flop count as the GPU line)"}


def shampoo_main(args):
    import torch
    import matrix_optimizers_amd as mo
    from matrix_optimizers_amd import workloads as wlmod
    key = args.workload if args.workload in wlmod.SHAMPOO_WORKLOADS else "shampoo_decoder_layer_h2048"
    wl = wlmod.SHAMPOO_WORKLOADS[key]
    hp = wl.hp
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] shampoo workload {wl.key}: {len(wl.matrices)} matrices", file=sys.stderr, flush=True)
    mats = []
    for i, sp in enumerate(wl.matrices):
        W = wlmod.torch_normal(wl.seed, i, wlmod.ROLE_W, (sp.rows, sp.cols), wl.w_std, wl.w_dtype, dev)
        G = wlmod.torch_normal(wl.seed, i, wlmod.ROLE_G, (sp.rows, sp.cols), wl.g_std, wl.g_dtype, dev)
        L = torch.eye(sp.rows, device=dev) * hp.eps
        R = torch.eye(sp.cols, device=dev) * hp.eps
        mats.append((W, G, L, R))
    step = mo.ShampooOwnerStep(mats, lr=hp.lr, weight_decay=hp.weight_decay, root_iters=hp.root_iters)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done; timing {args.steps} steps", file=sys.stderr, flush=True)
    ms = timed_steps(step, args.steps)       # no per-launch events (see main)
    print(f"[bench] {ms:.3f} ms/step", file=sys.stderr, flush=True)
    prof = {}
    if not args.no_phase_timing:
        prof, _ = event_timed_steps(step, args.steps)
    flops = {"stats": 0.0, "root": 0.0, "left": 0.0, "right": 0.0}
    for sp in wl.matrices:
        for k, v in wlmod.shampoo_flops_algorithmic(sp.rows, sp.cols, hp.root_iters).items():
            flops[k] += v
    total = sum(flops.values())
    tflops = total / (ms * 1e-3) / 1e12
    per_launch = {name: {"avg_ms": round(tot / cnt, 5), "launches": int(cnt), "ms_per_step": round(tot / args.steps, 5)}
                  for name, (tot, cnt) in prof.items() if cnt}
    out = {
        "metric": SHAMPOO_METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.key, "matrices": len(wl.matrices),
                   "shapes": sorted({f"{s.rows}x{s.cols}" for s in wl.matrices}),
                   "root_iters": hp.root_iters, "eps": hp.eps, "w_dtype": wl.w_dtype,
                   "g_dtype": wl.g_dtype, "parallelism": "none (one owner's bucket)"},
        "pct_peak": round(100.0 * tflops / PEAK_F32_TFLOPS, 2),
        "phases": per_launch,
    }
    phase_of = {"stats": "sh_stats", "root": "sh_root", "left": "sh_left", "right": "sh_right"}
    timed = {k: per_launch[v] for k, v in phase_of.items() if v in per_launch}
    if timed:
        dom = max(timed, key=lambda k: timed[k]["ms_per_step"])
        launches = timed[dom]["launches"] / args.steps
        achieved = flops[dom] / (timed[dom]["ms_per_step"] * 1e-3) / 1e12
        # HBM bytes per launch of this role from the committed rocprofv3 summary,
        # only if it was taken on the current kernel sources
        from matrix_optimizers_amd import profiling
        tr = profiling.read_traffic(os.path.join(ROOT, "profiles"), wl.key, f"sh_gemm[{dom}]")
        out["roofline"] = {"kernel": f"sh_gemm_f32 ({phase_of[dom]})", "bound": "mfma",
                           "achieved": round(achieved, 2), "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(achieved / PEAK_F32_TFLOPS, 4),
                           "traffic": None if tr is None else round(tr["read_bytes"] + tr["write_bytes"]),
                           "algorithmic_per_launch": f"{flops[dom] / launches:.4e} flop (mean over "
                                                     f"{launches:.0f} launches per step)"}
        if tr is not None:
            out["roofline"]["traffic_detail"] = {
                "read_bytes": round(tr["read_bytes"]), "write_bytes": round(tr["write_bytes"]),
                "profile": tr["source"], "profile_avg_ms": round(tr["avg_ns"] / 1e6, 5)}
    if not args.no_cpu_baseline and not args.profile_only:
        print("[bench] cpu_baseline (fp64 oracle on host)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = shampoo_cpu_baseline(wl)
    print(json.dumps(out), flush=True)


SOAP_METRIC = "SOAP owner-step ms (fp64 blocked-Jacobi eigensolver + fp32 products), 1 MI355X"


def soap_cpu_baseline(wl):
    """The fp64 oracle's SOAP step (numpy eigh for the eigenbases) on the
    workload's smallest matrix, timed on the host."""
    import numpy as np
    from matrix_optimizers_amd import workloads as wlmod
    from oracle import soap as osoap
    try:
        import threadpoolctl
        cores = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    i = min(range(len(wl.matrices)), key=lambda k: wl.matrices[k].rows * wl.matrices[k].cols)
    sp = wl.matrices[i]
    hp = wl.hp
    W = wlmod.normal(wl.seed, i, wlmod.ROLE_W, (sp.rows, sp.cols), wl.w_std, wl.w_dtype).astype(np.float64)
    G = wlmod.normal(wl.seed, i, wlmod.ROLE_G, (sp.rows, sp.cols), wl.g_std, wl.g_dtype).astype(np.float64)
    L = hp.stat_eps * np.eye(sp.rows)
    R = hp.stat_eps * np.eye(sp.cols)
    Z = np.zeros_like(W)
    t0 = time.perf_counter()
    osoap.soap_step(W, G, L, R, Z, Z, 1, hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay)
    dt = time.perf_counter() - t0
    # the same matrix's share of the GPU step, in the GPU's own work units
    return {"value": round(dt * 1e3, 1), "unit": "ms per matrix step", "cores": int(cores), "kind": "oracle",
            "sample": f"one {sp.rows}x{sp.cols} matrix of the bucket (two numpy fp64 eigh, six products), "
                      f"{dt:.2f} s; the GPU line is the whole {len(wl.matrices)}-matrix bucket"}


def soap_main(args):
    import torch
    import matrix_optimizers_amd as mo
    from matrix_optimizers_amd import workloads as wlmod
    key = args.workload if args.workload in wlmod.SOAP_WORKLOADS else "soap_decoder_layer_h2048"
    wl = wlmod.SOAP_WORKLOADS[key]
    hp = wl.hp
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] soap workload {wl.key}: {len(wl.matrices)} matrices", file=sys.stderr, flush=True)
    # A warm state, as SOAP runs in training: statistics summed over ten earlier
    # gradients (drawn and multiplied with torch on the device), first and
    # second moments drawn, step counter from 10.  From eps I instead, each
    # 5632-sided statistic would carry a 3584-fold eigenvalue eps whose
    # eigenspace the Jacobi sweeps keep turning.
    mats = []
    for i, sp in enumerate(wl.matrices):
        W = wlmod.torch_normal(wl.seed, i, wlmod.ROLE_W, (sp.rows, sp.cols), wl.w_std, wl.w_dtype, dev)
        G = wlmod.torch_normal(wl.seed, i, wlmod.ROLE_G, (sp.rows, sp.cols), wl.g_std, wl.g_dtype, dev)
        L = torch.eye(sp.rows, device=dev) * hp.stat_eps
        R = torch.eye(sp.cols, device=dev) * hp.stat_eps
        for h in range(10):
            Gp = wlmod.torch_normal(wl.seed, i, 100 + h, (sp.rows, sp.cols), wl.g_std, wl.g_dtype, dev)
            L += Gp @ Gp.T
            R += Gp.T @ Gp
        M = wlmod.torch_normal(wl.seed, i, wlmod.ROLE_M, (sp.rows, sp.cols), wl.g_std, wlmod.F32, dev)
        V = wlmod.torch_normal(wl.seed, i, 200, (sp.rows, sp.cols), wl.g_std, wlmod.F32, dev) ** 2
        mats.append((W, G, L, R, M, V))
    torch.cuda.synchronize()
    step = mo.SoapOwnerStep(mats, lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2, eps=hp.eps,
                            weight_decay=hp.weight_decay, sweeps=hp.sweeps)
    counter = {"t": 9}

    def one():
        counter["t"] += 1
        step(counter["t"])
    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done; timing {args.steps} steps", file=sys.stderr, flush=True)
    ms = timed_steps(one, args.steps)
    print(f"[bench] {ms:.3f} ms/step", file=sys.stderr, flush=True)
    prof = {}
    if not args.no_phase_timing:
        prof, _ = event_timed_steps(one, args.steps)
    per_launch = {name: {"avg_ms": round(tot / cnt, 5), "launches": int(cnt), "ms_per_step": round(tot / args.steps, 5)}
                  for name, (tot, cnt) in prof.items() if cnt}
    jac = {"apply": 0.0, "etile": 0.0, "solve": 0.0}
    prod = 0.0
    for sp in wl.matrices:
        prod += wlmod.soap_product_flops(sp.rows, sp.cols)
        for m in (sp.rows, sp.cols):
            f = wlmod.soap_jacobi_flops(m, hp.sweeps)
            for key in jac:
                jac[key] += f[key]
    out = {
        "metric": SOAP_METRIC, "value": round(ms, 3), "unit": "ms/step", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f64+f32",
        "data": "synthetic",
        "config": {"workload": wl.key, "matrices": len(wl.matrices),
                   "shapes": sorted({f"{s.rows}x{s.cols}" for s in wl.matrices}),
                   "sweeps": hp.sweeps, "stat_eps": hp.stat_eps, "w_dtype": wl.w_dtype,
                   "state": "warm: statistics of 10 earlier gradients, M and V drawn, t from 10",
                   "g_dtype": wl.g_dtype, "parallelism": "none (one owner's bucket)"},
        "flops_per_step": {"jacobi_apply_f64": jac["apply"], "jacobi_etile_f32": jac["etile"],
                           "jacobi_solve_f64": jac["solve"], "products_f32": prod,
                           "note": "Jacobi counts are the work of every round as if no pair had converged; "
                                   "pairs converged to fp64 resolution are skipped in late sweeps"},
        "phases": per_launch,
    }
    if not args.no_phase_timing:
        # The Jacobi kernels' rate, from a pass of two sweeps: the decoder-layer
        # sides are far from converged after two, so no pair is skipped and every
        # counted flop is executed (late sweeps of the full step skip converged
        # pairs, which a rate over the whole step would count as done).
        probe = mo.SoapOwnerStep(mats, lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2, eps=hp.eps,
                                 weight_decay=hp.weight_decay, sweeps=2)
        probe(10)
        torch.cuda.synchronize()
        p2, _ = event_timed_steps(lambda: probe(10), 1)
        f2 = {"apply": 0.0, "etile": 0.0}
        for sp in wl.matrices:
            for m in (sp.rows, sp.cols):
                f = wlmod.soap_jacobi_flops(m, 2)
                f2["apply"] += f["apply"]
                f2["etile"] += f["etile"]
        # One launch per round applies the rotations: the A tiles on fp64 MFMA,
        # the E items on fp32 MFMA.  Its roofline is the MFMA time, each product
        # at its own peak (the flop-weighted peak below); the HBM rate of the
        # bytes it must move (the upper blocks of A in fp64 and E in fp32, read
        # and written once per round) is reported beside.
        tot, cnt = p2.get("so_apply", (0.0, 0))
        if cnt:
            nbytes = 0.0
            for sp in wl.matrices:
                for m in (sp.rows, sp.cols):
                    b = wlmod.soap_jacobi_bytes(m, 2)
                    nbytes += b["per_round"] * b["rounds"]
            t_s = tot * 1e-3
            flops = f2["apply"] + f2["etile"]
            t_min = f2["apply"] / (PEAK_F64_TFLOPS * 1e12) + f2["etile"] / (PEAK_F32_TFLOPS * 1e12)
            peak = flops / t_min / 1e12
            achieved = flops / t_s / 1e12
            gbs = nbytes / t_s / 1e9
            # HBM bytes per launch from the committed rocprofv3 summary (a mean over
            # the whole step's launches), only if taken on the current sources
            from matrix_optimizers_amd import profiling
            tr = profiling.read_traffic(os.path.join(ROOT, "profiles"), wl.key, "so_rotate_tiles")
            ex = profiling.read_executed(os.path.join(ROOT, "profiles"), wl.key, "so_rotate_tiles")
            out["roofline"] = {
                "kernel": "so_jac_rotate_kernel", "bound": "mfma", "achieved": round(achieved, 2),
                "peak": round(peak, 2), "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": None if tr is None else round(tr["read_bytes"] + tr["write_bytes"]),
                "algorithmic_per_launch": f"{flops / cnt:.4e} flop ({f2['apply'] / cnt:.3e} fp64 for A, "
                                          f"{f2['etile'] / cnt:.3e} fp32 for E), mean over the {cnt} launches "
                                          f"of a two-sweep pass, avg {tot / cnt:.3f} ms",
                "peak_note": f"flop-weighted: the A products at the fp64 peak ({PEAK_F64_TFLOPS}) and the E "
                             f"products at the fp32 peak ({PEAK_F32_TFLOPS}) take {t_min / cnt * 1e3:.3f} ms "
                             f"per launch",
                "hbm_GBps": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                "hbm_bytes_per_launch": f"{nbytes / cnt:.4e} B (upper blocks of A in fp64 and E in fp32, "
                                        f"read and written once per round)"}
            if ex is not None:
                out["roofline"]["executed"] = {"mfma_busy": ex["mfma_busy"], "clock_ghz": ex["clock_ghz"],
                                               "profile": ex["source"],
                                               "note": "MFMA-busy share of SIMD cycles and shader clock from "
                                                       "the counter profile, mean over a whole step"}
            if tr is not None:
                out["roofline"]["traffic_detail"] = {
                    "read_bytes": round(tr["read_bytes"]), "write_bytes": round(tr["write_bytes"]),
                    "profile": tr["source"], "profile_avg_ms": round(tr["avg_ns"] / 1e6, 5),
                    "note": "mean over the launches of a whole step, converged late sweeps included"}
    if not args.profile_only:
        # The same bucket with the eigensolver warm-started from the previous
        # step's bases (warm_start=1 from the second call on): one untimed cold
        # call, then the timed steps, each warm.  Every step draws a fresh
        # gradient (on the device, inside the timed step), as in training: with
        # one gradient repeated, successive statistics would differ by the same
        # G G^T and the bases would barely move.
        wstep = mo.SoapOwnerStep(mats, lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2, eps=hp.eps,
                                 weight_decay=hp.weight_decay, sweeps=hp.sweeps, warm_start=True)
        wcount = {"t": counter["t"]}
        wgen = torch.Generator(device=dev)
        wgen.manual_seed(wl.seed + 4242)

        def wone():
            wcount["t"] += 1
            for m in mats:
                m[1].copy_(torch.randn(m[1].shape, device=dev, generator=wgen) * wl.g_std)
            wstep(wcount["t"])
        wone()
        torch.cuda.synchronize()
        wms = timed_steps(wone, args.steps)
        print(f"[bench] warm start: {wms:.3f} ms/step", file=sys.stderr, flush=True)
        warm = {"ms_per_step": round(wms, 3),
                "note": "eigensolver started from the previous step's eigenbases (warm_start=1), the same "
                        "eigendecomposition by fewer rotating sweeps; a fresh gradient each step (drawn on "
                        "the device inside the timed step); state carried on from the steps above"}
        if not args.no_phase_timing:
            wprof, _ = event_timed_steps(wone, args.steps)
            warm["phases"] = {name: round(tot / args.steps, 3) for name, (tot, cnt) in wprof.items()
                              if cnt and name in ("so_warm", "so_solve", "so_apply", "so_products")}
            warm["phases_unit"] = "ms per step"
        warm["rotating_pairs_after"] = wstep.rotating_pairs()
        out["warm_start"] = warm
    if not args.no_cpu_baseline and not args.profile_only:
        print("[bench] cpu_baseline (fp64 oracle on host)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = soap_cpu_baseline(wl)
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the owner step issues no collectives, and the "
              f"benchmark measures one owner's share (--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    import torch
    import matrix_optimizers_amd as mo
    from matrix_optimizers_amd import workloads as wlmod

    if args.copy_calibration:
        return copy_calibration(args)
    if args.adamw_sweep:
        return adamw_sweep(args)
    if args.optimizer == "shampoo":
        return shampoo_main(args)
    if args.optimizer == "soap":
        return soap_main(args)
    wl = wlmod.get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hp = wl.hp
    print(f"[bench] workload {wl.key}: {len(wl.matrices)} matrices, tail {wl.tail_numel}",
          file=sys.stderr, flush=True)
    mats = [wlmod.torch_matrix_inputs(wl, i, dev) for i in range(len(wl.matrices))]
    step = mo.MuonOwnerStep(mats, lr=hp.lr, weight_decay=hp.weight_decay, momentum=hp.momentum,
                            nesterov=hp.nesterov, ns_steps=hp.ns_steps,
                            ns_coefficients=(hp.ns_a, hp.ns_b, hp.ns_c), eps=hp.eps,
                            adjust_lr_fn=hp.lr_adjust, ns_dtype=hp.ns_dtype)
    tail = wlmod.torch_tail_inputs(wl.seed, wl.tail_numel, dev) if wl.tail_numel else None
    a = wl.adamw
    t_count = [a.step]

    muon = step
    if args.graph:
        # The allocation-free entry point uploads its work list through kernel
        # arguments, so the whole step is capturable; each replay is one step
        # on the same tensors.  The first call (outside the capture) loads the
        # code objects and takes the static array's address.
        kw = dict(lr=hp.lr, weight_decay=hp.weight_decay, momentum=hp.momentum, nesterov=hp.nesterov,
                  ns_steps=hp.ns_steps, ns_coefficients=(hp.ns_a, hp.ns_b, hp.ns_c), eps=hp.eps,
                  adjust_lr_fn=hp.lr_adjust, ns_dtype=hp.ns_dtype)
        need = mo.workspace_bytes([mo.tensor_descriptor(*m) for m in mats], mo.hparams(**kw))
        if need > mo.NOALLOC_SCRATCH_BYTES:
            print(f"bench.py --graph: workload {wl.key} needs {need >> 20} MiB of workspace, more than "
                  f"the allocation-free step's {mo.NOALLOC_SCRATCH_BYTES >> 20} MiB", file=sys.stderr)
            sys.exit(2)
        mo.muon_owner_step_noalloc(mats, **kw)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            mo.muon_owner_step_noalloc(mats, **kw)
        muon = graph.replay
        args.no_phase_timing = True

    def one_step():
        muon()
        if tail is not None:
            mo.adamw_tail_step(*tail, t_count[0], lr=a.lr, beta1=a.beta1, beta2=a.beta2,
                               eps=a.eps, weight_decay=a.weight_decay)
            t_count[0] += 1

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done; timing {args.steps} steps", file=sys.stderr, flush=True)

    # The wall time comes from a timed region without per-launch events: each
    # event record is a marker packet that leaves a gap between dependent
    # kernels (about 120 us per step on the decoder bucket).  The per-phase
    # launch durations (and the roofline) come from HIP events on the launch
    # stream over a second timed region of the same K steps right after.
    ms = timed_steps(one_step, args.steps)
    print(f"[bench] {ms:.3f} ms/step", file=sys.stderr, flush=True)
    prof = None
    per_step = []
    if not args.no_phase_timing:
        prof, ms_events = event_timed_steps(one_step, args.steps, per_step)
        print(f"[bench] {ms_events:.3f} ms/step with per-launch events", file=sys.stderr, flush=True)

    nominal = sum(wlmod.ns_flops_nominal(s.rows, s.cols, hp.ns_steps) for s in wl.matrices)
    algo = sum(wlmod.ns_flops_algorithmic(s.rows, s.cols, hp.ns_steps) for s in wl.matrices)
    tflops = nominal / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if hp.ns_dtype == "bf16" else PEAK_F32_TFLOPS
    out = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": hp.ns_dtype, "data": "synthetic",
        "config": {"workload": wl.key, "matrices": len(wl.matrices),
                   "shapes": sorted({f"{s.rows}x{s.cols}" for s in wl.matrices}),
                   "tail_elems": wl.tail_numel, "ns_steps": hp.ns_steps,
                   "w_dtype": wl.w_dtype, "g_dtype": wl.g_dtype, "momentum_dtype": "f32",
                   "parallelism": "none (one owner's bucket)",
                   "launch": "HIP graph replay of muon_owner_step_noalloc" if args.graph else "eager launches"},
        "ns_tflops_nominal": round(tflops, 3),
        "ns_tflops_algorithmic": round(algo / (ms * 1e-3) / 1e12, 3),
        "pct_peak_nominal": round(100.0 * tflops / peak, 2),
    }
    if prof is not None:
        out["ms_per_step_with_launch_events"] = round(ms_events, 4)
        srt = sorted(per_step)
        out["step_ms_events"] = {"median": round(srt[len(srt) // 2] if len(srt) % 2 else
                                                 0.5 * (srt[len(srt) // 2 - 1] + srt[len(srt) // 2]), 4),
                                 "min": round(srt[0], 4), "max": round(srt[-1], 4),
                                 "note": "per-step durations from events between steps, in the pass with "
                                         "per-launch events"}
        per_launch = {}
        flops_launch = {"gram": 0.0, "poly": 0.0, "update": 0.0, "update_last": 0.0}
        for s in wl.matrices:
            f = algorithmic_flops(s.rows, s.cols, hp.ns_steps)
            f["update_last"] = f["update"]
            for k in flops_launch:
                flops_launch[k] += f[k]
        for name, (tot, cnt) in prof.items():
            if cnt:
                per_launch[name] = {"avg_ms": round(tot / cnt, 5), "launches": int(cnt),
                                    "ms_per_step": round(tot / args.steps, 5)}
        out["phases"] = per_launch
        gemm = {k: v for k, v in per_launch.items() if k in flops_launch}
        if gemm:
            dom = max(gemm, key=lambda k: gemm[k]["ms_per_step"])
            achieved = flops_launch[dom] / (gemm[dom]["avg_ms"] * 1e-3) / 1e12
            # HBM bytes per launch from the committed rocprofv3 counter summary,
            # only if it was taken on the current kernel sources
            from matrix_optimizers_amd import profiling
            tr = profiling.read_traffic(os.path.join(ROOT, "profiles"), wl.key,
                                        f"{dom}[{hp.ns_dtype}]")
            out["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                               "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                               "traffic": None if tr is None else round(tr["read_bytes"] + tr["write_bytes"]),
                               "algorithmic_per_launch": f"{flops_launch[dom]:.4e} flop"}
            if tr is not None:
                out["roofline"]["traffic_detail"] = {
                    "read_bytes": round(tr["read_bytes"]), "write_bytes": round(tr["write_bytes"]),
                    "profile": tr["source"], "profile_avg_ms": round(tr["avg_ns"] / 1e6, 5)}
            # executed utilisation from the committed counter summary (same sources):
            # the matrix cores' busy share at the clock the part actually ran
            ex = profiling.read_executed(os.path.join(ROOT, "profiles"), wl.key, f"{dom}[{hp.ns_dtype}]")
            if ex is not None:
                out["roofline"]["executed"] = {
                    "mfma_busy_per_simd_cycle": ex["mfma_busy"], "shader_clock_ghz": ex["clock_ghz"],
                    "peak_at_that_clock_TFLOPs": round(peak * ex["clock_ghz"] / 2.4, 1),
                    "profile": ex["source"]}
        if "momentum" in per_launch:
            # momentum kernel, algorithmic bytes: read G (2 or 4) + M (4), write
            # M' (4) + X0 once in the NS dtype (2 or 4): 12 B/elem for bf16 G and
            # NS dtype.  The kernel also writes X0's transpose (moved bytes).
            es_g = 2 if wl.g_dtype == "bf16" else 4
            es_x = 2 if hp.ns_dtype == "bf16" else 4
            elems = sum(s.rows * s.cols for s in wl.matrices)
            algo_b = elems * (es_g + 8 + es_x)
            moved_b = elems * (es_g + 8 + es_x * (1 + MOMENTUM_EXTRA_COPIES))
            t = per_launch["momentum"]["avg_ms"] * 1e-3
            gbs = algo_b / t / 1e9
            out["momentum_kernel"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                      "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                      "algorithmic_per_launch": f"{algo_b} B ({es_g + 8 + es_x} B/elem)",
                                      "moved_GBps": round(moved_b / t / 1e9, 1),
                                      "moved_per_launch": f"{moved_b} B"}
    out["machine"] = machine_info(query_smi=not args.profile_only)
    if not args.no_cpu_baseline and not args.profile_only:
        print("[bench] cpu_baseline (fp64 oracle on host)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
