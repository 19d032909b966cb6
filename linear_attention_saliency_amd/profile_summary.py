"""Summaries of rocprofv3 CSV output for the kernels of this library.

  python -m linear_attention_saliency_amd.profile_summary stats <run_kernel_stats.csv>
  python -m linear_attention_saliency_amd.profile_summary trace <run_kernel_trace.csv> <last_n>
  python -m linear_attention_saliency_amd.profile_summary traffic <fetch_dir> <write_dir> <copy_bytes> [kernel]

`trace` averages each library kernel over its last N dispatches (the timed steps of a
bench run, after the warm-up steps have brought the clocks up).

`traffic` reads the counter_collection CSVs of a FETCH_SIZE pass and a WRITE_SIZE pass
(rocprofv3 --pmc ... -- python3 bench.py --calibrate-copy ...): the device-to-device copy
of known size (the first dispatch of the runtime's copyBuffer kernel) gives the scale from
counter units to bytes, which is applied to the mean per launch of the library kernel
whose name contains `kernel` (default attn_kernel).
"""

from __future__ import annotations

import collections
import csv
import glob
import os
import sys


def stats(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    lines = ["| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        short = name.split("(")[0]
        lines.append(f"| {short[:70]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    return "\n".join(lines)


def trace(path: str, last_n: int) -> str:
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if "still" in r["Kernel_Name"]:
            per[r["Kernel_Name"]].append((int(r["Dispatch_Id"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    lines = [f"| kernel | dispatches | mean us over the last {last_n} | min us | max us |", "|---|---|---|---|---|"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(x for _, x in kv[1])):
        if len(v) < last_n:  # launched only outside the timed window (set-up)
            continue
        xs = [x for _, x in sorted(v)][-last_n:]
        lines.append(f"| {k.split('(')[0][:70]} | {len(v)} | {sum(xs) / len(xs):.1f} | {min(xs):.1f} | {max(xs):.1f} |")
    return "\n".join(lines)


def _per_kernel(dirpath: str, counter: str):
    """counter values per kernel name, each list in dispatch order"""
    out = collections.defaultdict(list)
    for f in glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True):
        rows = [r for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]
        for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
            out[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return out


def traffic(fetch_dir: str, write_dir: str, copy_bytes: int, kernel: str = "attn_kernel") -> str:
    lines = []
    total = 0.0
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _per_kernel(d, counter)
        copies = [k for k in per if "copyBuffer" in k]
        if len(copies) != 1:
            raise SystemExit(f"expected one copy kernel, found {copies}")
        ck = copies[0]
        scale = copy_bytes / per[ck][0]  # bytes per counter unit (the first copy is the calibration)
        hits = [k for k in per if kernel in k and "still" in k]
        if len(hits) != 1:
            raise SystemExit(f"expected one library kernel matching {kernel!r}, found {hits}")
        val = sum(per[hits[0]]) / len(per[hits[0]]) * scale
        total += val
        lines.append(f"{counter}: copy kernel {ck[:60]} read {per[ck][0]:.0f} for {copy_bytes} bytes "
                     f"(scale {scale:.2f} B/unit); {kernel} mean {val / 1e6:.2f} MB per launch")
    lines.append(f"hbm_bytes_per_launch: {total:.0f}")
    return "\n".join(lines)


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        print(stats(sys.argv[2]))
    elif sys.argv[1] == "trace":
        print(trace(sys.argv[2], int(sys.argv[3])))
    elif sys.argv[1] == "traffic":
        print(traffic(sys.argv[2], sys.argv[3], int(sys.argv[4]), *sys.argv[5:6]))
