"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m zero_shot_rope_jl_amd.profiling stats KERNEL_STATS_CSV --title T --cmd C
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


def source_hash() -> str:
    """sha256 over the library's kernel and ABI sources (csrc/ and include/)."""
    h = hashlib.sha256()
    root = os.path.dirname(PKG)
    files = sorted(os.path.join(PKG, "csrc", f) for f in os.listdir(os.path.join(PKG, "csrc"))
                   if f.endswith((".hip", ".h")))
    files += sorted(os.path.join(root, "include", f) for f in os.listdir(os.path.join(root, "include"))
                    if f.endswith(".h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    n = re.sub(r"\((jl::)?\w+Params\)", "", name).replace("void ", "")
    return n.replace("jl::(anonymous namespace)::", "jl::")


def stats_markdown(path: str, title: str, cmd: str, top: int = 8) -> str:
    rows = list(csv.DictReader(open(path)))
    out = [f"# {title}", "", "Command (repository root on one MI355X):", "", "```", cmd, "```", "",
           "| kernel | calls | average (us) | min (us) | max (us) | % GPU time |", "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        n = short_name(r["Name"])
        n = n if len(n) < 80 else n[:77] + "..."
        out.append(f"| `{n}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                   f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
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
        "source_sha256": source_hash(),
        "copy_calibration": {"bytes_each_way": CALIBRATION_BYTES, "fetch_kib": f_copy, "write_kib": w_copy,
                             "fetch_factor": f_fac, "write_factor": w_fac},
        "kernels": kernels,
        "commands": {"fetch": cmd_fetch, "write": cmd_write},
    }


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
    a = ap.parse_args(argv)
    if a.what == "stats":
        sys.stdout.write(stats_markdown(a.csv, a.title, a.cmd))
    else:
        json.dump(traffic_summary(a.fetch, a.write, a.cmd_fetch, a.cmd_write), sys.stdout, indent=1)
        sys.stdout.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
