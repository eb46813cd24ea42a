"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m zero_shot_rope_jl_amd.profiling stats KERNEL_STATS_CSV --title T --cmd C
    python -m zero_shot_rope_jl_amd.profiling grid KERNEL_TRACE_CSV --title T --cmd C
    python -m zero_shot_rope_jl_amd.profiling traffic --fetch FETCH_CSV --write WRITE_CSV \
        --cmd-fetch C1 --cmd-write C2

``stats`` turns a ``--kernel-trace --stats`` kernel_stats.csv into a short
markdown table.  ``traffic`` turns two ``--pmc FETCH_SIZE`` / ``--pmc
WRITE_SIZE`` counter_collection.csv files (KiB per dispatch) into HBM bytes
per dispatch of each library kernel.  The counters are scaled by what they
read for a plain device-to-device copy of a known size in the same run (the
largest ``__amd_rocclr_copyBuffer`` dispatch, 512 MiB read and 512 MiB
written), and the summary records a hash of the library sources so that a
figure taken before a kernel change is not reported after it.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CALIBRATION_BYTES = 512 << 20


def library_hash() -> str:
    """sha256 of the built library (its GPU code objects and host code): the
    counters describe this binary, and a rebuild from unchanged sources is
    byte-identical, so edits that leave the code as it was keep the hash."""
    h = hashlib.sha256()
    with open(os.path.join(PKG, "libjetlong.so"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    n = re.sub(r"\((jl::)?\w+Params\)", "", name).replace("void ", "")
    return n.replace("jl::(anonymous namespace)::", "jl::")


def stats_markdown(path: str, title: str, cmd: str, other: int = 3) -> str:
    """Every library kernel (names starting with jl::) of the trace, and the
    `other` longest-running kernels that are not the library's."""
    rows = list(csv.DictReader(open(path)))
    ours = [r for r in rows if "jl::" in r["Name"]]
    rest = [r for r in rows if "jl::" not in r["Name"]][:other]
    keep = sorted(ours + rest, key=lambda r: -float(r["Percentage"]))
    out = [f"# {title}", "", "Command (repository root on one MI355X):", "", "```", cmd, "```", "",
           "| kernel | calls | average (us) | min (us) | max (us) | % GPU time |", "|---|---|---|---|---|---|"]
    for r in keep:
        n = short_name(r["Name"])
        n = n if len(n) < 80 else n[:77] + "..."
        out.append(f"| `{n}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                   f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def grid_markdown(path: str, title: str, cmd: str) -> str:
    """Library kernels of a --kernel-trace kernel_trace.csv grouped by kernel
    and grid size (which tells apart launches of one kernel for different
    problem sizes), in order of first launch: count and average duration."""
    groups = collections.OrderedDict()
    for r in csv.DictReader(open(path)):
        if "jl::" not in r["Kernel_Name"]:
            continue
        key = (short_name(r["Kernel_Name"]), int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]),
               int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = [f"# {title}", "", "Command (repository root on one MI355X):", "", "```", cmd, "```", "",
           "| kernel | workgroups | calls | average (us) | min (us) |", "|---|---|---|---|---|"]
    for (name, grid, wg), d in groups.items():
        n = name if len(name) < 80 else name[:77] + "..."
        out.append(f"| `{n}` | {grid // wg} | {len(d)} | {sum(d) / len(d):.2f} | {min(d):.2f} |")
    return "\n".join(out) + "\n"


def _per_kernel(path: str, counter: str):
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
    if not copies:
        raise SystemExit(f"{path}: no copy dispatch to calibrate {counter} against")
    per = collections.defaultdict(list)
    for r in rows:
        if "jl::" in r["Kernel_Name"]:
            per[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return max(copies), per


def traffic_summary(fetch_csv: str, write_csv: str, cmd_fetch: str, cmd_write: str) -> dict:
    f_copy, f_per = _per_kernel(fetch_csv, "FETCH_SIZE")
    w_copy, w_per = _per_kernel(write_csv, "WRITE_SIZE")
    f_fac = CALIBRATION_BYTES / (f_copy * 1024.0)
    w_fac = CALIBRATION_BYTES / (w_copy * 1024.0)
    kernels = {}
    for k in sorted(set(f_per) | set(w_per)):
        fv, wv = f_per.get(k, []), w_per.get(k, [])
        kernels[k] = {
            "dispatches": max(len(fv), len(wv)),
            "fetch_bytes": (sum(fv) / len(fv)) * 1024.0 * f_fac if fv else None,
            "write_bytes": (sum(wv) / len(wv)) * 1024.0 * w_fac if wv else None,
        }
    return {
        "about": "HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by "
                 "what the counter reads for a plain copy of 512 MiB in the same run",
        "library_sha256": library_hash(),
        "copy_calibration": {"bytes_each_way": CALIBRATION_BYTES, "fetch_kib": f_copy, "write_kib": w_copy,
                             "fetch_factor": f_fac, "write_factor": w_fac},
        "kernels": kernels,
        "commands": {"fetch": cmd_fetch, "write": cmd_write},
    }


def pmc_markdown(paths, kernel_prefix: str, title: str, cmds, simds: int = 1024, xcds: int = 8) -> str:
    """Per-dispatch averages of every counter collected for the kernels whose
    short name starts with kernel_prefix, over one or more --pmc runs, plus
    derived shares when their counters were collected.  GRBM_GUI_ACTIVE
    comes summed over the chip's XCDs, so one XCD's active cycles are
    GRBM_GUI_ACTIVE / xcds; MFMA busy is SQ_VALU_MFMA_BUSY_CYCLES over that
    times the SIMD count.  The SQ_WAVE_CYCLES-style counters are per wave in
    units of 4 cycles, summed over waves."""
    vals = collections.defaultdict(list)
    for path in paths:
        for r in csv.DictReader(open(path)):
            if short_name(r["Kernel_Name"]).startswith(kernel_prefix):
                vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no dispatch of {kernel_prefix} in {paths}")
    out = [f"# {title}", "", f"Kernel `{kernel_prefix}`; counters averaged per dispatch.", "",
           "Commands (repository root on one MI355X, one run per counter set):", ""]
    out += ["```", *cmds, "```", "", "| counter | dispatches | value per dispatch |", "|---|---|---|"]
    avg = {}
    for k in sorted(vals):
        avg[k] = sum(vals[k]) / len(vals[k])
        out.append(f"| `{k}` | {len(vals[k])} | {avg[k]:.6g} |")
    gui = avg.get("GRBM_GUI_ACTIVE")
    gui = gui / xcds if gui else None
    derived = []
    if gui:
        derived.append(f"* active cycles of one XCD: GRBM_GUI_ACTIVE / {xcds} = {gui:.4g}")
    if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        derived.append(f"* MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (active cycles x {simds} SIMDs) = "
                       f"{100.0 * avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui * simds):.1f}%")
    if gui and "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
        derived.append(f"* MFMA and VALU in the same cycle: SQ_VALU_MFMA_COEXEC_CYCLES / (active cycles x {simds}) = "
                       f"{100.0 * avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / (gui * simds):.1f}%")
    if gui and "SQ_BUSY_CU_CYCLES" in avg:
        derived.append(f"* CUs busy on average: SQ_BUSY_CU_CYCLES / active cycles = {avg['SQ_BUSY_CU_CYCLES'] / gui:.1f}")
    if "SQ_WAVE_CYCLES" in avg and avg["SQ_WAVE_CYCLES"]:
        for k in ("SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY",
                  "SQ_WAIT_INST_LDS"):
            if k in avg:
                derived.append(f"* {k} / SQ_WAVE_CYCLES = {100.0 * avg[k] / avg['SQ_WAVE_CYCLES']:.1f}% of wave time")
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in avg:
        derived.append(f"* bf16 MFMA FLOP per dispatch (MOPS x 512) = {avg['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512:.4g}")
    if "SQ_LDS_BANK_CONFLICT" in avg and "SQ_LDS_IDX_ACTIVE" in avg and avg["SQ_LDS_IDX_ACTIVE"]:
        derived.append(f"* LDS bank-conflict cycles / LDS active cycles = "
                       f"{avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_LDS_IDX_ACTIVE']:.4g}")
    if derived:
        out += ["", "Derived:", "", *derived]
    return "\n".join(out) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(prog="python -m zero_shot_rope_jl_amd.profiling")
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--title", required=True)
    s.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    g = sub.add_parser("grid")
    g.add_argument("csv")
    g.add_argument("--title", required=True)
    g.add_argument("--cmd", required=True)
    m = sub.add_parser("pmc")
    m.add_argument("csv", nargs="+")
    m.add_argument("--kernel", required=True)
    m.add_argument("--title", required=True)
    m.add_argument("--cmd", action="append", default=[])
    a = ap.parse_args(argv)
    if a.what == "grid":
        sys.stdout.write(grid_markdown(a.csv, a.title, a.cmd))
        return 0
    if a.what == "pmc":
        sys.stdout.write(pmc_markdown(a.csv, a.kernel, a.title, a.cmd))
        return 0
    if a.what == "stats":
        sys.stdout.write(stats_markdown(a.csv, a.title, a.cmd))
    else:
        json.dump(traffic_summary(a.fetch, a.write, a.cmd_fetch, a.cmd_write), sys.stdout, indent=1)
        sys.stdout.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
