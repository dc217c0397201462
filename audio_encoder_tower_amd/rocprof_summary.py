"""Summaries of rocprofv3 CSV output for the encoder's kernels.

Usage:
  python -m audio_encoder_tower_amd.rocprof_summary trace <dir>     kernel trace (--kernel-trace --stats)
  python -m audio_encoder_tower_amd.rocprof_summary counters <dir>  counter runs (--pmc ...)

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
    i = name.find("(")
    return name[:i] if i > 0 else name


def trace(d: str) -> str:
    groups = collections.OrderedDict()
    for f in _files(d, "kernel_trace.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = (_short(r["Kernel_Name"]), int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0))
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


def counters(d: str) -> str:
    # (kernel, grid) -> dispatch -> counter -> value (rocprofv3 writes one row
    # per dispatch and counter, already summed over the counter's instances)
    per = collections.OrderedDict()
    dur = collections.defaultdict(dict)
    for f in _files(d, "counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = (_short(r["Kernel_Name"]), int(r.get("Grid_Size", 0) or 0))
                disp = (f, r.get("Dispatch_Id", r.get("Correlation_Id")))
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
    if len(argv) != 3 or argv[1] not in ("trace", "counters"):
        sys.exit(__doc__)
    print(trace(argv[2]) if argv[1] == "trace" else counters(argv[2]))


if __name__ == "__main__":
    main(sys.argv)
