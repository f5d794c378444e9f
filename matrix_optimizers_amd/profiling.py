"""Summaries of rocprofv3 output for the committed profiles, and the HBM
traffic figure bench.py reports.

    python -m matrix_optimizers_amd.profiling summarize TRACE_DIR COUNTER_DIR \\
        COPY_DIR OUT.md --command "..." --workload NAME

TRACE_DIR holds a ``--kernel-trace --stats -f csv`` run; COUNTER_DIR holds one
subdirectory per ``--pmc`` pass (FETCH_SIZE/, WRITE_SIZE/) of the same command;
COPY_DIR holds the same two passes over ``bench.py --copy-calibration`` (the
library's plain copy of a known number of bytes), which fixes the factor
between each counter and true bytes.  The summary states the per-kernel
durations, per-launch HBM bytes, and the SHA-256 of the kernel sources (of the
workload's optimizer) the counters were taken on; bench.py reports the traffic
only while that hash still matches the sources.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
from collections import defaultdict
from typing import Dict, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# What decides each optimizer's kernels and their memory traffic: the device
# code and the host code that builds its work lists (tile order); the upload
# and timing helpers (host_common.*) do not.  A summary is stamped with the
# hash of its own optimizer's sources, so that a change to one optimizer's
# kernels leaves the others' summaries standing.
FAMILY_SOURCES = {
    "muon": ["csrc/ns_kernels.hip", "csrc/tail_kernels.hip", "csrc/device_common.h", "csrc/mo_worklist.h",
             "csrc/gemm_core.h", "csrc/gemm_core8.h", "csrc/tile_dispatch.h", "csrc/host.cpp"],
    "shampoo": ["csrc/shampoo_kernels.hip", "csrc/sh_worklist.h", "csrc/shampoo.cpp", "csrc/device_common.h",
                "csrc/mo_worklist.h", "csrc/gemm_core.h", "csrc/tile_dispatch.h"],
    "soap": ["csrc/soap_kernels.hip", "csrc/so_worklist.h", "csrc/soap.cpp", "csrc/device_common.h",
             "csrc/mo_worklist.h"],
}


def family_of(workload: str) -> str:
    """The optimizer a profiled workload runs: SOAP and Shampoo workloads carry
    the optimizer's name as a prefix, every other workload is a Muon bucket."""
    for fam in ("soap", "shampoo"):
        if workload.startswith(fam + "_"):
            return fam
    return "muon"


def sources_sha256(family: str) -> str:
    h = hashlib.sha256()
    for rel in FAMILY_SOURCES[family]:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


SH_KERNELS = (("sh_gemm_f32", "sh_gemm"), ("sh_layout_kernel", "sh_layout"), ("sh_sumsq_kernel", "sh_sumsq"),
              ("sh_norm_kernel", "sh_norm"), ("sh_init_kernel", "sh_init"),
              # SOAP step
              ("so_jac_rotate_kernel", "so_rotate_tiles"),
              ("so_jac_solve_kernel", "so_solve"), ("so_gemm_kernel", "so_gemm"), ("so_prep_kernel", "so_prep"),
              ("so_eig_init_kernel", "so_eig_init"), ("so_norm_rows_kernel", "so_norm_rows"),
              ("so_norm_final_kernel", "so_norm_final"), ("so_eig_sort_kernel", "so_sort"),
              ("so_eig_gather_kernel", "so_gather"))


def short_name(kernel: str) -> Optional[str]:
    """Library kernel -> phase name (None for kernels that are not ours)."""
    for key, name in SH_KERNELS:
        if key in kernel:
            return name
    m = re.search(r"\b(gram|poly|update_last|update)_(bf16|f32)\b", kernel)
    if m:
        return f"{m.group(1)}[{m.group(2)}]"
    for key, name in (("momentum_kernel", "momentum"), ("norm_kernel", "norm"),
                      ("apply_kernel", "apply"), ("adamw", "adamw")):
        if key in kernel:
            return name
    if kernel.startswith("(anonymous namespace)::copy_kernel") or "::copy_kernel(" in kernel:
        return "copy"
    return None


def shampoo_roles(names):
    """The Shampoo GEMM launches of a dispatch sequence, by role: in each step
    (which starts with the layout launch) the first GEMM launch forms the
    statistics, the last two are the left and right products, the others
    are coupled Newton (root) products.  Returns one name per entry."""
    out = list(names)
    step = []
    def close():
        for n, i in enumerate(step):
            out[i] = ("sh_gemm[stats]" if n == 0 else "sh_gemm[right]" if n == len(step) - 1
                      else "sh_gemm[left]" if n == len(step) - 2 else "sh_gemm[root]")
    for i, n in enumerate(names):
        if n == "sh_layout":
            close()
            step = []
        elif n == "sh_gemm":
            step.append(i)
    close()
    return out


def _ordered(rows, key):
    rows = sorted(rows, key=lambda r: float(r[key]))
    names = shampoo_roles([short_name(r["Kernel_Name"]) for r in rows])
    return list(zip(rows, names))


def kernel_stats(trace_dir: str) -> Dict[str, dict]:
    """Per-phase calls / total / average (ns) from the kernel trace."""
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    out: Dict[str, dict] = defaultdict(lambda: {"calls": 0, "total_ns": 0.0})
    for f in files:
        for r, name in _ordered(list(csv.DictReader(open(f))), "Start_Timestamp"):
            if name is None:
                continue
            d = out[name]
            d["calls"] += 1
            d["total_ns"] += float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    for d in out.values():
        d["avg_ns"] = d["total_ns"] / d["calls"]
    return dict(out)


def counter_means(pass_dir: str, counter: str) -> Dict[str, float]:
    """Mean value of `counter` per dispatch, per phase."""
    vals: Dict[str, list] = defaultdict(list)
    for f in glob.glob(os.path.join(pass_dir, "**", "*counter_collection.csv"), recursive=True):
        rows = [r for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]
        for r, name in _ordered(rows, "Dispatch_Id"):
            if name is not None:
                vals[name].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def copy_factor(copy_dir: str, counter: str, copied_bytes: int) -> float:
    """True bytes per counter unit, from the copy kernel: it reads and writes
    copied_bytes each."""
    m = counter_means(os.path.join(copy_dir), counter).get("copy")
    if not m:
        raise RuntimeError(f"no copy-kernel {counter} samples in {copy_dir}")
    return copied_bytes / m


def summarize(trace_dir, counter_dir, copy_dirs, out_md, command, workload, copied_mib=1024, note=""):
    stats = kernel_stats(trace_dir)
    copied = copied_mib << 20
    fetch = counter_means(os.path.join(counter_dir, "FETCH_SIZE"), "FETCH_SIZE")
    write = counter_means(os.path.join(counter_dir, "WRITE_SIZE"), "WRITE_SIZE")
    ff = copy_factor(copy_dirs["FETCH_SIZE"], "FETCH_SIZE", copied)
    wf = copy_factor(copy_dirs["WRITE_SIZE"], "WRITE_SIZE", copied)
    lines = [f"# rocprofv3 summary: {workload}", "",
             "Commands (run from the repository root on one MI355X):", "",
             "```", command, "```", "",
             f"Kernel sources SHA-256 ({family_of(workload)}): `{sources_sha256(family_of(workload))}`", ""] + ([note, ""] if note else []) + [
             f"Byte-counter calibration with the library's copy kernel ({copied_mib} MiB read + written): "
             f"FETCH_SIZE x {ff:.4g} B, WRITE_SIZE x {wf:.4g} B.", "",
             "| phase | launches | avg (us) | total (ms) | HBM read / launch (MB) | HBM write / launch (MB) |",
             "|---|---|---|---|---|---|"]
    for name, d in sorted(stats.items(), key=lambda kv: -kv[1]["total_ns"]):
        rd = fetch.get(name)
        wr = write.get(name)
        lines.append(f"| {name} | {d['calls']} | {d['avg_ns'] / 1e3:.2f} | {d['total_ns'] / 1e6:.3f} | "
                     f"{'' if rd is None else f'{rd * ff / 1e6:.1f}'} | "
                     f"{'' if wr is None else f'{wr * wf / 1e6:.1f}'} |")
    lines += ["", "Machine-readable (bench.py reads these lines):", ""]
    for name, d in sorted(stats.items()):
        rd, wr = fetch.get(name), write.get(name)
        if rd is not None and wr is not None:
            lines.append(f"traffic {workload} {name} {rd * ff:.0f} {wr * wf:.0f} {d['avg_ns']:.0f} "
                         f"{sources_sha256(family_of(workload))}")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out_md


def trace_summary(trace_dir, out_md, command, workload, note=""):
    """Per-phase launches and durations from a kernel trace alone (no byte
    counters)."""
    stats = kernel_stats(trace_dir)
    lines = [f"# rocprofv3 summary: {workload}", "", "Commands (run from the repository root on one MI355X):", "",
             "```", command, "```", ""]
    if note:
        lines += [note, ""]
    lines += ["| phase | launches | avg (us) | total (ms) |", "|---|---|---|---|"]
    for name, d in sorted(stats.items(), key=lambda kv: -kv[1]["total_ns"]):
        lines.append(f"| {name} | {d['calls']} | {d['avg_ns'] / 1e3:.2f} | {d['total_ns'] / 1e6:.3f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out_md


def read_traffic(profiles_dir: str, workload: str, phase: str) -> Optional[dict]:
    """HBM bytes per launch of `phase` measured on the current kernel sources,
    or None if no summary matches them."""
    sha = sources_sha256(family_of(workload))
    for f in sorted(glob.glob(os.path.join(profiles_dir, "*.md"))):
        for line in open(f):
            p = line.split()
            if len(p) == 7 and p[0] == "traffic" and p[1] == workload and p[2] == phase and p[6] == sha:
                return {"read_bytes": float(p[3]), "write_bytes": float(p[4]), "avg_ns": float(p[5]),
                        "source": os.path.basename(f)}
    return None


# Counter groups of the executed-work summary; each is one rocprofv3 --pmc pass
# (per-block limits: 8 SQ, 4 TCC, 4 TCP counters).
COUNTER_PASSES = [
    ["SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES",
     "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "GRBM_GUI_ACTIVE"],
    ["TCC_HIT_sum", "TCC_MISS_sum", "TCC_EA0_RDREQ_sum"],
    ["TCP_TCC_READ_REQ_sum", "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_PENDING_STALL_CYCLES_sum"],
]
XCDS, SIMDS, CUS = 8, 1024, 256     # MI355X: SQ and GRBM counters below are summed over these


def counters_summary(pass_dirs, trace_dir, out_md, command, workload, flops_per_launch=None):
    """Executed-work summary per GEMM phase from the counter passes:
    MFMA instructions, MFMA-busy share of SIMD cycles, the shader clock implied
    by the cycle counters and the kernel duration, L2 hit rate, mean L1->L2
    read latency."""
    stats = kernel_stats(trace_dir)
    vals = {}
    for d in pass_dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                name = short_name(r["Kernel_Name"])
                if name is not None:
                    vals.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    mean = {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in vals.items()}
    lines = [f"# rocprofv3 counters: {workload}", "", "Commands (run from the repository root on one MI355X):", "",
             "```", command, "```", "", f"Kernel sources SHA-256 ({family_of(workload)}): `{sources_sha256(family_of(workload))}`", "",
             "Per launch, averaged over the profiled launches. GRBM_GUI_ACTIVE counts GPU-busy cycles per XCD "
             f"(summed over {XCDS}); dividing by the traced duration gives the shader clock under load. "
             f"SQ_VALU_MFMA_BUSY_CYCLES is summed over the {SIMDS} SIMDs.", "",
             "| phase | avg (us) | MFMA instr | MFMA busy / SIMD-cycle | clock (GHz) | L2 hit | mean L1->L2 read latency (cycles) |",
             "|---|---|---|---|---|---|---|"]
    machine = []
    for name in sorted(mean, key=lambda k: -stats.get(k, {}).get("total_ns", 0.0)):
        c = mean[name]
        if "SQ_INSTS_MFMA" not in c or c["SQ_INSTS_MFMA"] == 0:
            continue
        avg_ns = stats.get(name, {}).get("avg_ns")
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
        clock = cyc / avg_ns if avg_ns else float("nan")
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / SIMDS / cyc if cyc else float("nan")
        hit = c.get("TCC_HIT_sum", 0.0) / max(c.get("TCC_HIT_sum", 0.0) + c.get("TCC_MISS_sum", 0.0), 1.0)
        lat = c.get("TCP_TCC_READ_REQ_LATENCY_sum", 0.0) / max(c.get("TCP_TCC_READ_REQ_sum", 0.0), 1.0)
        lines.append(f"| {name} | {avg_ns / 1e3 if avg_ns else float('nan'):.1f} | {c['SQ_INSTS_MFMA']:.4g} | "
                     f"{busy:.3f} | {clock:.2f} | {hit:.3f} | {lat:.0f} |")
        machine.append(f"executed {workload} {name} {busy:.4f} {clock:.3f} {sources_sha256(family_of(workload))}")
    lines += ["", "Machine-readable (bench.py reads these lines: phase, MFMA busy share, clock in GHz):", ""]
    lines += machine
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out_md


def read_executed(profiles_dir: str, workload: str, phase: str) -> Optional[dict]:
    """MFMA-busy share and shader clock of one phase from a committed counter
    summary, if it was taken on the current kernel sources."""
    path = os.path.join(profiles_dir, f"counters_{workload}.md")
    if not os.path.exists(path):
        return None
    cur = sources_sha256(family_of(workload))
    for line in open(path):
        f = line.split()
        if len(f) == 6 and f[0] == "executed" and f[1] == workload and f[2] == phase and f[5] == cur:
            return {"mfma_busy": float(f[3]), "clock_ghz": float(f[4]), "source": os.path.basename(path)}
    return None


def _main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("trace_dir")
    s.add_argument("counter_dir")
    s.add_argument("copy_dir", help="directory with copy_FETCH_SIZE/ and copy_WRITE_SIZE/")
    s.add_argument("out_md")
    s.add_argument("--command", required=True)
    s.add_argument("--workload", required=True)
    s.add_argument("--copy-mib", type=int, default=1024)
    s.add_argument("--note", default="")
    c = sub.add_parser("counters")
    c.add_argument("trace_dir")
    c.add_argument("out_md")
    c.add_argument("pass_dirs", nargs="+")
    c.add_argument("--command", required=True)
    c.add_argument("--workload", required=True)
    t = sub.add_parser("trace")
    t.add_argument("trace_dir")
    t.add_argument("out_md")
    t.add_argument("--command", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--note", default="")
    a = ap.parse_args()
    if a.cmd == "trace":
        trace_summary(a.trace_dir, a.out_md, a.command, a.workload, a.note)
        print("wrote", a.out_md)
        return
    if a.cmd == "counters":
        counters_summary(a.pass_dirs, a.trace_dir, a.out_md, a.command, a.workload)
        print("wrote", a.out_md)
        return
    summarize(a.trace_dir, a.counter_dir,
              {"FETCH_SIZE": os.path.join(a.copy_dir, "copy_FETCH_SIZE"),
               "WRITE_SIZE": os.path.join(a.copy_dir, "copy_WRITE_SIZE")},
              a.out_md, a.command, a.workload, a.copy_mib, a.note)
    print("wrote", a.out_md)


if __name__ == "__main__":
    _main()
