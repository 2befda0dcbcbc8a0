"""Summarise a rocprofv3 kernel trace or counter collection of a bench run.

    python -m tiled_gemm_graph_amd.profile_summary DIR [--kernel mk_persistent]
                                                       [--skip S] [--count K]

DIR is the ``-d`` directory of ``rocprofv3 --kernel-trace --output-format
csv`` (or of a ``--pmc`` run).  Every dispatch of a kernel whose name
contains ``--kernel`` is listed in launch order; ``--skip`` / ``--count``
select the timed ones (a ``bench.py --workload W --steps K --warmup W``
run launches the persistent kernel 1 + W + K times before its per-op
launches: one parity forward, the warmups, the timed forwards).  Prints a
markdown table with the median, min and max duration of the selected
dispatches (kernel trace) or the mean of each counter over them (counter
collection).
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import statistics
import sys


def _rows(d: str, suffix: str):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    out = []
    for f in files:
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def kernel_durations(d: str, name: str):
    """(dispatch id, duration ns) of every dispatch whose kernel name contains
    ``name``, in dispatch order."""
    rows = _rows(d, "kernel_trace.csv")
    sel = []
    for r in rows:
        if name in r.get("Kernel_Name", ""):
            sel.append((int(r.get("Dispatch_Id", 0) or 0),
                        int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    sel.sort()
    return sel


def counters(d: str, name: str):
    """{dispatch id: {counter: value}} for dispatches of ``name``."""
    rows = _rows(d, "counter_collection.csv")
    out = {}
    for r in rows:
        if name not in r.get("Kernel_Name", ""):
            continue
        did = int(r.get("Dispatch_Id", 0) or 0)
        out.setdefault(did, {})[r["Counter_Name"]] = out.get(did, {}).get(r["Counter_Name"], 0.0) + \
            float(r["Counter_Value"])
    return dict(sorted(out.items()))


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("dir")
    ap.add_argument("--kernel", default="mk_persistent")
    ap.add_argument("--skip", type=int, default=0)
    ap.add_argument("--count", type=int, default=0, help="0 = all after --skip")
    a = ap.parse_args(argv)
    dur = kernel_durations(a.dir, a.kernel)
    if dur:
        sel = dur[a.skip:a.skip + a.count] if a.count else dur[a.skip:]
        us = [x[1] / 1000.0 for x in sel]
        print(f"| kernel | dispatches (all) | selected | median us | min us | max us |")
        print("|---|---|---|---|---|---|")
        print(f"| {a.kernel} | {len(dur)} | {len(sel)} (from #{a.skip}) | "
              f"{statistics.median(us):.1f} | {min(us):.1f} | {max(us):.1f} |")
        print()
        print("all dispatches, us: " + ", ".join(f"{x[1] / 1000.0:.1f}" for x in dur))
        return 0
    cnt = counters(a.dir, a.kernel)
    if cnt:
        items = list(cnt.items())
        sel = items[a.skip:a.skip + a.count] if a.count else items[a.skip:]
        names = sorted({k for _, v in sel for k in v})
        print("| counter | dispatches | mean | min | max |")
        print("|---|---|---|---|---|")
        for n in names:
            v = [c[n] for _, c in sel if n in c]
            print(f"| {n} | {len(v)} | {statistics.mean(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
        return 0
    print(f"no dispatch of a kernel matching {a.kernel!r} under {a.dir}", file=sys.stderr)
    return 1


if __name__ == "__main__":
    sys.exit(main())
