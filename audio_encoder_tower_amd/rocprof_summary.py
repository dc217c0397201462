"""Summaries of rocprofv3 CSV output for the encoder's kernels.

Usage:
  python -m audio_encoder_tower_amd.rocprof_summary trace <dir> [--cycle KERNEL=a,b ...]
  python -m audio_encoder_tower_amd.rocprof_summary counters <dir> [--cycle KERNEL=a,b ...]
  python -m audio_encoder_tower_amd.rocprof_summary traffic <fetch dir> <write dir> --copy-mib MIB \
      --step STEP=KERNEL@GRID ... [--cycle KERNEL=a,b ...]

  trace: a kernel-trace run (--kernel-trace --stats); counters: a --pmc run.
  --cycle labels the dispatches of one kernel (its short name, e.g.
  "gemm_bf16_256_kernel<2, false>") in dispatch order with the given labels in
  turn, so that two steps that run the same kernel at the same grid (the
  O-projection and FC2 of every block) are reported apart.
  traffic: HBM bytes per launch of the named steps from a FETCH_SIZE run and a
  WRITE_SIZE run of the same program, each run having first passed MIB MiB
  through the plain copy kernel (bench.py --copy-probe-mib): each counter is
  scaled by what it reads for that copy (MIB MiB each way). Prints JSON with
  a digest of each step's kernel sources, so readings taken on other sources
  can be told apart.

<dir> is the -d directory of a rocprofv3 run with --output-format csv; the
files found under it (*kernel_trace.csv, *counter_collection.csv) are read.
Rows are grouped by kernel name and grid size; counter values (rocprofv3
sums each over its instances: XCDs, SEs, SIMDs) are averaged over the
dispatches of a group. GRBM_GUI_ACTIVE is the sum over the XCDs of each
one's busy cycles, so cycles = GRBM_GUI_ACTIVE / XCDs (8 on MI355X), and the
clock is cycles over the profiled dispatch time. MFMA busy is
SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs), the fraction of SIMD
cycles with a matrix instruction in flight (256 CUs x 4 SIMDs), and CU busy
SQ_BUSY_CU_CYCLES / (cycles x 256). On MI355X GRBM_GUI_ACTIVE counts over a
somewhat longer window than the dispatch timestamps: for a 2.45 ms kernel the
derived clock matches the shader clock that s_memtime counts inside it, for
the encoder's 0.1-0.3 ms GEMMs it reads 9-20% high, and for 30 us kernels it
exceeds the part's 2.4 GHz; the busy fractions are low by the same factor.
Measurement tooling only: nothing on the forward path imports it.
"""
from __future__ import annotations

import collections
import csv
import glob
import hashlib
import json
import os
import sys

N_CU = 256
N_SIMD = 4 * N_CU
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")

# Kernel sources whose change invalidates stored hardware-counter readings.
KERNEL_SOURCES = {
    kind: ["gemm_bf16.hip", "epilogue.h", "common.h", "launch.h"]
    for kind in ("qkv", "o_proj", "fc1", "fc2", "proj1", "proj2", "conv1", "conv2")
}
KERNEL_SOURCES["attention"] = ["attention.hip", "common.h", "launch.h"]
KERNEL_SOURCES["layernorm"] = ["norm.hip", "common.h", "launch.h"]
KERNEL_SOURCES["final_ln"] = ["norm.hip", "common.h", "launch.h"]


def source_digest(kind: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kind, []):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


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


def _counter_avgs(d: str, counter: str, cycles=None):
    """(labelled kernel, grid) -> (dispatches, average value of `counter`)."""
    per = collections.defaultdict(list)
    label = _labeler(cycles or {})
    for f in _files(d, "counter_collection.csv"):
        for r in _rows(f):
            if r["Counter_Name"] == counter:
                per[label(_short(r["Kernel_Name"]), int(r.get("Grid_Size", 0) or 0))].append(
                    float(r["Counter_Value"]))
    return {k: (len(v), sum(v) / len(v)) for k, v in per.items()}


def traffic(fetch_dir: str, write_dir: str, copy_mib: float, steps, cycles=None) -> str:
    fetch = _counter_avgs(fetch_dir, "FETCH_SIZE", cycles)
    write = _counter_avgs(write_dir, "WRITE_SIZE", cycles)
    moved_kib = copy_mib * 1024.0
    # the copy kernel's one dispatch of copy_mib MiB (its largest grid)
    copies = [k for k in fetch if k[0] == "copy_kernel"]
    if not copies:
        sys.exit("no copy_kernel dispatch in the FETCH_SIZE run (run with --copy-probe-mib)")
    ck = max(copies, key=lambda k: k[1])
    f_scale = moved_kib / fetch[ck][1]
    w_scale = moved_kib / write[ck][1]
    out = {"about": ("HBM-side bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch), "
                     f"each scaled by what the counter reads for the plain copy kernel over {copy_mib:g} MiB "
                     "in the same run"),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "kernels": {}}
    for step, (kernel, grid) in steps.items():
        keys = [k for k in fetch if k[0] == kernel and k[1] == grid]
        if not keys or keys[0] not in write:
            sys.exit(f"no dispatch of {kernel} at grid {grid} in both runs")
        k = keys[0]
        fk, wk = fetch[k][1], write[k][1]
        out["kernels"][step] = {
            "kernel": kernel, "grid": grid, "fetch_kib_raw": round(fk, 1), "write_kib_raw": round(wk, 1),
            "fetch_bytes": round(fk * f_scale * 1024), "write_bytes": round(wk * w_scale * 1024),
            "bytes_per_launch": round((fk * f_scale + wk * w_scale) * 1024),
            "dispatches": [fetch[k][0], write[k][0]], "source_digest": source_digest(step)}
    return json.dumps(out, indent=1)


def main(argv):
    if len(argv) < 3 or argv[1] not in ("trace", "counters", "traffic"):
        sys.exit(__doc__)
    cycles, steps, copy_mib = {}, {}, None
    rest = argv[3:] if argv[1] != "traffic" else argv[4:]
    while rest:
        if len(rest) < 2:
            sys.exit(__doc__)
        if rest[0] == "--cycle" and "=" in rest[1]:
            name, labels = rest[1].rsplit("=", 1)
            cycles[name] = labels.split(",")
        elif rest[0] == "--step" and "=" in rest[1] and "@" in rest[1]:
            step, spec = rest[1].split("=", 1)
            kernel, grid = spec.rsplit("@", 1)
            steps[step] = (kernel, int(grid))
        elif rest[0] == "--copy-mib":
            copy_mib = float(rest[1])
        else:
            sys.exit(__doc__)
        rest = rest[2:]
    if argv[1] == "trace":
        print(trace(argv[2], cycles))
    elif argv[1] == "counters":
        print(counters(argv[2], cycles))
    else:
        if len(argv) < 4 or copy_mib is None or not steps:
            sys.exit(__doc__)
        print(traffic(argv[2], argv[3], copy_mib, steps, cycles))


if __name__ == "__main__":
    main(sys.argv)
