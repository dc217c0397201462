"""Summaries of rocprofv3 CSV output for the encoder's kernels.

Usage:
  python -m audio_encoder_tower_amd.rocprof_summary trace <dir> [--cycle KERNEL=a,b ...]
  python -m audio_encoder_tower_amd.rocprof_summary counters <dir> [--cycle KERNEL=a,b ...]

  trace: a kernel-trace run (--kernel-trace --stats); counters: a --pmc run.
  --cycle labels the dispatches of one kernel (its short name, e.g.
  "gemm_bf16_256_kernel<2, false>") in dispatch order with the given labels in
  turn, so that two steps that run the same kernel at the same grid (the
  O-projection and FC2 of every block) are reported apart.

<dir> is the -d directory of a rocprofv3 run with --output-format csv; the
files found under it (*kernel_trace.csv, *counter_collection.csv) are read.
Rows are grouped by kernel name and grid size; counter values (rocprofv3
sums each over its instances: XCDs, SEs, SIMDs) are averaged over the
dispatches of a group. GRBM_GUI_ACTIVE is the sum over the XCDs of each
one's busy cycles, so cycles = GRBM_GUI_ACTIVE / XCDs (8 on MI355X), and the
clock is cycles over the profiled dispatch time. MFMA busy is
SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs), the fraction of SIMD
cycles with a matrix instruction in flight (256 CUs x 4 SIMDs), and CU busy
SQ_BUSY_CU_CYCLES / (cycles x 256).
Measurement tooling only: nothing on the forward path imports it.
"""
from __future__ import annotations

import collections
import csv
import glob
import os
import sys

N_CU = 256
N_SIMD = 4 * N_CU


def _files(d: str, suffix: str):
    return sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))


def _short(name: str) -> str:
    name = name.replace("aenc::", "").replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    i = name.find("(")
    return name[:i] if i > 0 else name


def _labeler(cycles):
    """(short kernel name) -> labels assigned in turn to its dispatches."""
    seen = collections.Counter()

    def label(name: str, grid: int):
        labels = cycles.get(name)
        if not labels:
            return name, grid
        i = seen[(name, grid)]
        seen[(name, grid)] += 1
        return f"{name} [{labels[i % len(labels)]}]", grid
    return label


def _rows(f: str):
    with open(f) as fh:
        rows = list(csv.DictReader(fh))
    return sorted(rows, key=lambda r: int(r.get("Dispatch_Id", r.get("Correlation_Id", 0)) or 0))


def trace(d: str, cycles=None) -> str:
    groups = collections.OrderedDict()
    label = _labeler(cycles or {})
    for f in _files(d, "kernel_trace.csv"):
        for r in _rows(f):
            key = label(_short(r["Kernel_Name"]), int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0))
            dt = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6
            groups.setdefault(key, []).append(dt)
    total = sum(sum(v) for v in groups.values()) or 1.0
    out = ["| kernel | grid | calls | avg ms | min ms | max ms | share |", "|---|---|---|---|---|---|---|"]
    for (k, g), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| {k} | {g} | {len(v)} | {sum(v) / len(v):.4f} | {min(v):.4f} | {max(v):.4f} | "
                   f"{100 * sum(v) / total:.1f}% |")
    return "\n".join(out)


def _n_xcc(d: str) -> int:
    for f in _files(d, "agent_info.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Agent_Type") == "GPU" and r.get("Num_Xcc"):
                    return int(r["Num_Xcc"])
    return 8


def counters(d: str, cycles=None) -> str:
    # (kernel, grid) -> dispatch -> counter -> value (rocprofv3 writes one row
    # per dispatch and counter, already summed over the counter's instances)
    per = collections.OrderedDict()
    dur = collections.defaultdict(dict)
    label = _labeler(cycles or {})
    for f in _files(d, "counter_collection.csv"):
        keys = {}
        for r in _rows(f):
            disp = (f, r.get("Dispatch_Id", r.get("Correlation_Id")))
            if disp not in keys:
                keys[disp] = label(_short(r["Kernel_Name"]), int(r.get("Grid_Size", 0) or 0))
            key = keys[disp]
            if True:  # noqa: SIM108 (one row per dispatch and counter)
                per.setdefault(key, collections.OrderedDict()).setdefault(disp, {})[r["Counter_Name"]] = \
                    float(r["Counter_Value"])
                if r.get("End_Timestamp") and r.get("Start_Timestamp"):
                    dur[key][disp] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6
    xcc = _n_xcc(d)
    names = sorted({n for v in per.values() for c in v.values() for n in c})
    head = ["kernel", "grid", "dispatches", "avg ms (profiled)"] + [f"{n} (avg)" for n in names]
    derived = []
    if "GRBM_GUI_ACTIVE" in names:
        derived.append("clock GHz")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in names and "GRBM_GUI_ACTIVE" in names:
        derived.append("MFMA busy")
    if "SQ_BUSY_CU_CYCLES" in names and "GRBM_GUI_ACTIVE" in names:
        derived.append("CU busy")
    out = ["| " + " | ".join(head + derived) + " |", "|" + "---|" * (len(head) + len(derived))]
    for (k, g), disps in per.items():
        avg = {n: sum(c.get(n, 0.0) for c in disps.values()) / len(disps) for n in names}
        ms = sum(dur[(k, g)].values()) / max(1, len(dur[(k, g)]))
        row = [k, str(g), str(len(disps)), f"{ms:.4f}"] + [f"{avg[n]:.4g}" for n in names]
        # GRBM_GUI_ACTIVE is the sum over the XCDs of each one's busy clock cycles
        cyc = avg.get("GRBM_GUI_ACTIVE", 0.0) / xcc
        if "clock GHz" in derived:
            row.append(f"{cyc / (ms * 1e6):.2f}" if ms > 0 else "")
        if "MFMA busy" in derived:
            row.append(f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * N_SIMD):.3f}" if cyc else "")
        if "CU busy" in derived:
            row.append(f"{avg['SQ_BUSY_CU_CYCLES'] / (cyc * N_CU):.3f}" if cyc else "")
        out.append("| " + " | ".join(row) + " |")
    return "\n".join(out)


def main(argv):
    if len(argv) < 3 or argv[1] not in ("trace", "counters"):
        sys.exit(__doc__)
    cycles = {}
    rest = argv[3:]
    while rest:
        if rest[0] != "--cycle" or len(rest) < 2 or "=" not in rest[1]:
            sys.exit(__doc__)
        name, labels = rest[1].rsplit("=", 1)
        cycles[name] = labels.split(",")
        rest = rest[2:]
    print(trace(argv[2], cycles) if argv[1] == "trace" else counters(argv[2], cycles))


if __name__ == "__main__":
    main(sys.argv)
