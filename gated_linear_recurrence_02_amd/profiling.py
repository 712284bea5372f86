"""Summaries of rocprofv3 output (CSV format) for the kernels of librglru.so.

rocprofv3 writes one `<pid>_counter_collection.csv` per profiled process for a
`--pmc` run and `<pid>_kernel_trace.csv` / `<pid>_kernel_stats.csv` for a
`--kernel-trace --stats` run, under the directory given with `-d`.  The
functions here read those files and reduce them per kernel:

* counters(dir, match): mean per dispatch of every counter over the dispatches
  whose kernel name the regular expression `match` finds (re.search; names
  come demangled or, for some template arguments, mangled); a counter's rows
  for one dispatch (one per XCD or instance) are summed first;
* traffic(...): HBM bytes per launch of a kernel from a FETCH_SIZE run and a
  WRITE_SIZE run, each scaled by what the same counter reads for a plain copy
  of known size (FETCH_SIZE and WRITE_SIZE count the traffic between L2 and
  the fabric in KiB, and the scale turns that into bytes moved);
* durations(dir, match): calls and mean/min/max duration from a kernel trace.

bench.py --summarize-traffic / --summarize-counters / --summarize-trace drive
them and prints the summaries kept in profiles/.
"""
from __future__ import annotations

import collections
import csv
import glob
import os
import re


def _files(d: str, suffix: str) -> list:
    out = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not out:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return out


def counters(d: str, match: str):
    """{counter: mean over dispatches of the per-dispatch sum}, number of dispatches."""
    per = collections.defaultdict(float)
    seen = set()
    for f in _files(d, "counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if not re.search(match, r["Kernel_Name"]):
                    continue
                key = (f, r["Dispatch_Id"])
                seen.add(key)
                per[(key, r["Counter_Name"])] += float(r["Counter_Value"])
    if not seen:
        raise ValueError(f"no dispatch of a kernel matching {match!r} under {d}")
    tot = collections.defaultdict(float)
    for (_, c), v in per.items():
        tot[c] += v
    return {c: v / len(seen) for c, v in tot.items()}, len(seen)


def durations(d: str, match: str):
    """(calls, mean us, min us, max us) of the kernels matching `match` in a kernel trace."""
    us = []
    for f in _files(d, "kernel_trace.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if re.search(match, r["Kernel_Name"]):
                    us.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if not us:
        raise ValueError(f"no dispatch of a kernel matching {match!r} under {d}")
    return len(us), sum(us) / len(us), min(us), max(us)


def traffic(fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str, match: str,
            copy_bytes: int, copy_match: str = "copyBuffer") -> dict:
    """HBM bytes per launch of the kernels matching `match`, calibrated on a
    plain device copy that reads and writes `copy_bytes` bytes each."""
    f, nf = counters(fetch_dir, match)
    w, nw = counters(write_dir, match)
    cf, _ = counters(copy_fetch_dir, copy_match)
    cw, _ = counters(copy_write_dir, copy_match)
    fetch_scale = copy_bytes / (cf["FETCH_SIZE"] * 1024.0)
    write_scale = copy_bytes / (cw["WRITE_SIZE"] * 1024.0)
    read = f["FETCH_SIZE"] * 1024.0 * fetch_scale
    written = w["WRITE_SIZE"] * 1024.0 * write_scale
    return {"fetch_kib_per_dispatch": round(f["FETCH_SIZE"], 1),
            "write_kib_per_dispatch": round(w["WRITE_SIZE"], 1),
            "dispatches_averaged": min(nf, nw),
            "copy_calibration": {"bytes_read": copy_bytes, "bytes_written": copy_bytes,
                                 "fetch_kib": round(cf["FETCH_SIZE"], 1), "write_kib": round(cw["WRITE_SIZE"], 1),
                                 "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4)},
            "hbm_read_bytes_per_launch": int(read), "hbm_write_bytes_per_launch": int(written),
            "hbm_bytes_per_launch": int(read + written)}


def counter_table(dirs: list, kernels: list) -> str:
    """Text table: for each (label, match) kernel the mean per dispatch of every
    counter found for it in any of `dirs` (one directory per counter pass)."""
    lines = []
    for label, match in kernels:
        vals, n = {}, 0
        for d in dirs:
            try:
                m, k = counters(d, match)
            except ValueError:
                continue
            vals.update(m)
            n = max(n, k)
        lines.append(f"{label}  (kernel name matches {match!r}; mean over {n} dispatches)")
        for c in sorted(vals):
            lines.append(f"  {c:32s} {vals[c]:18.1f}")
        lines.append("")
    return "\n".join(lines)


def _demangle(name: str) -> str:
    """Itanium-mangled names that the profiler left mangled (its demangler does
    not know the bf16 type code DF16b) through c++filt, with that code spelled
    as the vendor type __bf16; other names unchanged."""
    if not name.startswith("_Z"):
        return name
    import shutil
    import subprocess
    if shutil.which("c++filt") is None:
        return name
    r = subprocess.run(["c++filt"], input=name.replace("DF16b", "u6__bf16"), capture_output=True, text=True)
    return r.stdout.strip() or name


def _short(name: str) -> str:
    """Kernel name without return type, namespaces and parameter list."""
    n = _demangle(name)
    n = re.sub(r"^void ", "", n)
    n = n.replace("(anonymous namespace)::", "")
    n = re.sub(r"\(.*$", "", n)
    return re.sub(r"\b[A-Za-z_][A-Za-z_0-9]*::", "", n)


def trace_table(d: str) -> str:
    """Calls and mean/min/max duration per kernel from `--kernel-trace --stats`
    output, slowest total first; library GEMM kernels (names with Cijk_) on
    one line."""
    rows = []
    for f in _files(d, "kernel_stats.csv"):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    gemm = [r for r in rows if "Cijk_" in r["Name"]]
    out = [f"{'kernel':62s} {'calls':>7s} {'avg us':>9s} {'min us':>9s} {'max us':>9s} {'total ms':>9s}"]
    body = []
    for r in rows:
        if "Cijk_" in r["Name"]:
            continue
        body.append((float(r["TotalDurationNs"]), _short(r["Name"])[:62], int(r["Calls"]), float(r["AverageNs"]),
                     float(r["MinNs"]), float(r["MaxNs"])))
    if gemm:
        tot = sum(float(r["TotalDurationNs"]) for r in gemm)
        calls = sum(int(r["Calls"]) for r in gemm)
        body.append((tot, f"library GEMMs ({len(gemm)} kernels)", calls, tot / calls,
                     min(float(r["MinNs"]) for r in gemm), max(float(r["MaxNs"]) for r in gemm)))
    for tot, n, c, a, lo, hi in sorted(body, reverse=True):
        out.append(f"{n:62s} {c:7d} {a / 1e3:9.1f} {lo / 1e3:9.1f} {hi / 1e3:9.1f} {tot / 1e6:9.2f}")
    return "\n".join(out)
