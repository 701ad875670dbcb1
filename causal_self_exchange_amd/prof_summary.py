"""Summaries of rocprofv3 CSV output for the committed profile notes.

kernel_stats(csv): per-kernel call count and average / min / max duration from
a `rocprofv3 --kernel-trace --stats --output-format csv` kernel_stats file.
trace_avg(csv, kernel_substr, last_n, within_first): mean duration (us) of the
last `last_n` dispatches of one kernel from a `--kernel-trace` kernel_trace
file (the timed launches of a run that first warms up), optionally within its
first `within_first` dispatches.
trace_series(csv, kernel_substr, first_n): durations (us) of the first
`first_n` dispatches of one kernel, in dispatch order (a launch curve).
counter_avg(csv, kernel_substr, counter): a counter's mean over dispatches of
one kernel from a `--pmc` counter_collection file.
traffic(...): HBM bytes per launch of a kernel from FETCH_SIZE / WRITE_SIZE
(KiB per dispatch), each scaled by the same counter's reading for a plain
copy of known size (bytes read = bytes written = copy_bytes).
"""
from __future__ import annotations

import csv
import json
import sys


def kernel_stats(path: str) -> list[dict]:
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            out.append({"kernel": r["Name"], "calls": int(r["Calls"]),
                        "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                        "max_us": float(r["MaxNs"]) / 1e3, "pct": float(r["Percentage"])})
    return out


def trace_avg(path: str, kernel_substr: str, last_n: int, within_first: int | None = None) -> dict:
    """Mean duration of the last `last_n` dispatches (in dispatch order) of the
    kernels whose name contains `kernel_substr`, counting only the first
    `within_first` such dispatches when given (a run that launches the kernel
    again after its timed region)."""
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel_substr in r["Kernel_Name"]:
                rows.append((int(r["Dispatch_Id"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    rows.sort()
    if within_first is not None:
        rows = rows[:within_first]
    durs = [d for _, d in rows[-last_n:]]
    if not durs:
        raise ValueError(f"no dispatches of {kernel_substr} in {path}")
    return {"dispatches": len(rows), "last_n": len(durs), "avg_us": sum(durs) / len(durs),
            "min_us": min(durs), "max_us": max(durs)}


def trace_series(path: str, kernel_substr: str, first_n: int) -> list[float]:
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel_substr in r["Kernel_Name"]:
                rows.append((int(r["Dispatch_Id"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    rows.sort()
    return [round(d, 1) for _, d in rows[:first_n]]


def counter_avg(path: str, kernel_substr: str, counter: str) -> float:
    vals = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise ValueError(f"no {counter} for {kernel_substr} in {path}")
    return sum(vals) / len(vals)


def traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, kernel_substr, copy_kernel_substr,
            copy_bytes) -> dict:
    f_k = counter_avg(fetch_csv, kernel_substr, "FETCH_SIZE")
    w_k = counter_avg(write_csv, kernel_substr, "WRITE_SIZE")
    f_c = counter_avg(copy_fetch_csv, copy_kernel_substr, "FETCH_SIZE")
    w_c = counter_avg(copy_write_csv, copy_kernel_substr, "WRITE_SIZE")
    sf = copy_bytes / (f_c * 1024.0)
    sw = copy_bytes / (w_c * 1024.0)
    return {"fetch_kib": f_k, "write_kib": w_k, "copy_fetch_kib": f_c, "copy_write_kib": w_c,
            "fetch_scale": sf, "write_scale": sw,
            "read_bytes": f_k * 1024.0 * sf, "write_bytes": w_k * 1024.0 * sw,
            "bytes_per_launch": f_k * 1024.0 * sf + w_k * 1024.0 * sw}


if __name__ == "__main__":
    for row in kernel_stats(sys.argv[1]):
        print(json.dumps(row))
