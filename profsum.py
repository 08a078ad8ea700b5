"""Summaries of rocprofv3 CSV output for the logits kernels.

Reads what ``rocprofv3 --kernel-trace --stats --output-format csv`` and
``rocprofv3 --pmc <counter> --output-format csv`` write and turns it into the
short text summaries kept with the library: per-kernel average durations, and
HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE, each scaled by what the
same counter reads for a device-to-device copy of known size
(``bench.py --copy-calibration`` issues one).

  python profsum.py stats  <kernel_stats.csv>
  python profsum.py trace  <kernel_trace.csv>
  python profsum.py pmc    <counter_collection.csv> <counter> <copy_bytes>
  python profsum.py counters <counter_collection.csv>
  python profsum.py digest

``trace`` groups the dispatches of a kernel trace by kernel and launch
shape (grid and workgroup size), so one run over several workloads that share
kernels still gives each workload's durations.

``counters`` prints, per kernel and launch shape, the mean per dispatch of every
counter in a counter_collection.csv (raw values, summed over the hardware
instances the CSV lists).

``digest`` prints a hash of the decode-logits kernel sources (their code:
comments and blank lines are left out, so editing a comment keeps it); a
traffic figure is only valid for the code it was measured on.
"""
from __future__ import annotations

import csv
import hashlib
import sys
from collections import defaultdict
from pathlib import Path

CSRC = Path(__file__).resolve().parent / "paged_mqa_logits_amd" / "csrc"
LOGITS_SOURCES = ("pml_device.h", "rows.h", "logits_core.h", "paged_logits.hip")
COPY_KERNEL = "copyBuffer"  # the runtime's device-to-device copy kernel


def _code_only(text: str) -> str:
    """C++ source without its comments, trailing blanks and empty lines
    (string and character literals are kept whole)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "\n".join(l.rstrip() for l in "".join(out).splitlines() if l.strip())


def source_digest() -> str:
    """sha256 (first 16 hex digits) over the code of the decode-logits kernel sources."""
    h = hashlib.sha256()
    for name in LOGITS_SOURCES:
        h.update(name.encode())
        h.update(_code_only((CSRC / name).read_text()).encode())
    return h.hexdigest()[:16]


def kernel_stats(path: str) -> list[dict]:
    """Rows of a *_kernel_stats.csv: name, calls, average / min / max in us, share of time."""
    out = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            out.append({"name": r["Name"], "calls": int(r["Calls"]),
                        "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                        "max_us": float(r["MaxNs"]) / 1e3, "pct": float(r["Percentage"])})
    return out


def trace_by_shape(path: str) -> list[dict]:
    """Dispatches of a *_kernel_trace.csv grouped by (kernel, grid, workgroup):
    count and average / min / max duration in us."""
    groups = defaultdict(list)
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            grid = tuple(int(r[f"Grid_Size_{a}"]) for a in "XYZ")
            wg = tuple(int(r[f"Workgroup_Size_{a}"]) for a in "XYZ")
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            groups[(r["Kernel_Name"], grid, wg)].append(dur)
    out = []
    for (name, grid, wg), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        out.append({"name": name, "grid": grid, "wg": wg, "calls": len(d), "avg_us": sum(d) / len(d),
                    "min_us": min(d), "max_us": max(d)})
    return out


def counter_means(path: str, counter: str) -> dict[str, tuple[int, float]]:
    """Kernel name -> (dispatches, mean counter value per dispatch) from a counter_collection.csv."""
    per = defaultdict(dict)  # name -> dispatch -> summed value
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = per[r["Kernel_Name"]]
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return {k: (len(v), sum(v.values()) / len(v)) for k, v in per.items()}


def counters_by_shape(path: str) -> tuple[list[str], list[dict]]:
    """(counter names, rows): per (kernel, grid, workgroup) the dispatch count and
    each counter's mean per dispatch (instances of one dispatch summed)."""
    per = defaultdict(lambda: defaultdict(dict))  # shape -> counter -> dispatch -> value
    names = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            key = (r["Kernel_Name"], int(r["Grid_Size"]), int(r["Workgroup_Size"]))
            c = r["Counter_Name"]
            if c not in names:
                names.append(c)
            d = per[key][c]
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    rows = []
    for (name, grid, wg), cs in per.items():
        n = max(len(v) for v in cs.values())
        rows.append({"name": name, "grid": grid, "wg": wg, "n": n,
                     **{c: sum(v.values()) / len(v) for c, v in cs.items()}})
    return names, rows


def calibrated(path: str, counter: str, copy_bytes: int) -> tuple[float, dict[str, tuple[int, float, float]]]:
    """(scale, kernel -> (dispatches, KiB per dispatch, calibrated bytes per dispatch)).

    scale = copy_bytes / (KiB the copy kernel's dispatches read for `counter` x 1024),
    taken from the largest copy dispatch (the calibration copy)."""
    m = counter_means(path, counter)
    copies = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and COPY_KERNEL in r["Kernel_Name"]:
                copies.append(float(r["Counter_Value"]))
    if not copies:
        raise SystemExit(f"no {COPY_KERNEL} dispatch with {counter} in {path}")
    scale = copy_bytes / (max(copies) * 1024.0)
    return scale, {k: (n, v, v * 1024.0 * scale) for k, (n, v) in m.items()}


def _main(argv: list[str]) -> None:
    if not argv or argv[0] not in ("stats", "trace", "pmc", "counters", "digest"):
        print(__doc__)
        raise SystemExit(2)
    if argv[0] == "digest":
        print(source_digest())
    elif argv[0] == "trace":
        print(f"{'kernel':70s} {'grid (threads)':>22s} {'wg':>5s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} "
              f"{'max_us':>10s}")
        for r in trace_by_shape(argv[1]):
            g = "x".join(str(v) for v in r["grid"])
            print(f"{r['name'][:70]:70s} {g:>22s} {r['wg'][0]:5d} {r['calls']:6d} {r['avg_us']:10.2f} "
                  f"{r['min_us']:10.2f} {r['max_us']:10.2f}")
    elif argv[0] == "counters":
        names, rows = counters_by_shape(argv[1])
        for r in sorted(rows, key=lambda r: (r["name"], r["grid"])):
            print(f"{r['name'][:100]}  grid {r['grid']} wg {r['wg']}  dispatches {r['n']}")
            for c in names:
                if c in r:
                    print(f"    {c:34s} {r[c]:16.6g}")
    elif argv[0] == "stats":
        print(f"{'kernel':90s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'time%':>7s}")
        for r in kernel_stats(argv[1]):
            print(f"{r['name'][:90]:90s} {r['calls']:6d} {r['avg_us']:10.2f} {r['min_us']:10.2f} "
                  f"{r['max_us']:10.2f} {r['pct']:7.2f}")
    else:
        path, counter, nbytes = argv[1], argv[2], int(argv[3])
        scale, rows = calibrated(path, counter, nbytes)
        print(f"{counter}: copy calibration {nbytes} bytes -> scale {scale:.4f}")
        print(f"{'kernel':90s} {'n':>4s} {'KiB/dispatch':>14s} {'bytes/dispatch':>16s}")
        for k, (n, kib, b) in sorted(rows.items(), key=lambda kv: -kv[1][2]):
            print(f"{k[:90]:90s} {n:4d} {kib:14.1f} {b:16.0f}")
    print(f"logits sources digest {source_digest()}")


if __name__ == "__main__":
    _main(sys.argv[1:])
