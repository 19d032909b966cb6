"""Summaries of rocprofv3 CSV output for the kernels of this library.

  python -m linear_attention_saliency_amd.profile_summary stats <run_kernel_stats.csv>
  python -m linear_attention_saliency_amd.profile_summary trace <run_kernel_trace.csv> <last_n>
  python -m linear_attention_saliency_amd.profile_summary traffic <fetch_dir> <write_dir> <copy_bytes> [kernel]
  python -m linear_attention_saliency_amd.profile_summary counters [--match=<substring>] <pass_dir> [<pass_dir> ...]

`trace` averages each library kernel over its last N dispatches (the timed steps of a
bench run, after the warm-up steps have brought the clocks up).

`traffic` reads the counter_collection CSVs of a FETCH_SIZE pass and a WRITE_SIZE pass
(rocprofv3 --pmc ... -- python3 bench.py --calibrate-copy ...): the device-to-device copy
of known size (the first dispatch of the runtime's copyBuffer kernel) gives the scale from
counter units to bytes, which is applied to the mean per launch of the library kernel
whose name contains `kernel` (default attn_, the attention kernel the workload launches).

`counters` merges the counter_collection CSVs of several --pmc passes (one directory per
pass) into one row per library kernel (those whose name contains the --match substring):
per-wave instruction counts, and per-SIMD busy
shares, which divide the summed busy cycles by the 1024 SIMDs and by GRBM_GUI_ACTIVE / 8
(one XCD's active cycles; SQ_ACTIVE_INST_VALU counts quad cycles and is scaled by 4).
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


def traffic(fetch_dir: str, write_dir: str, copy_bytes: int, kernel: str = "attn_", others=()) -> str:
    """HBM bytes per launch of `kernel` (the machine-read line), then of each kernel in
    `others` (name substrings) as comment lines."""
    lines = []
    total = 0.0
    extra = collections.defaultdict(float)
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
        for o in others:
            for k in per:
                if o in k and "still" in k:
                    extra[(_short_name(k), counter)] = sum(per[k]) / len(per[k]) * scale
    lines.append(f"hbm_bytes_per_launch: {total:.0f}")
    for name in sorted({n for n, _ in extra}):
        f, w = extra.get((name, "FETCH_SIZE"), 0.0), extra.get((name, "WRITE_SIZE"), 0.0)
        lines.append(f"# {name}: {f / 1e6:.2f} MB read + {w / 1e6:.2f} MB written = {(f + w) / 1e6:.2f} MB per launch")
    return "\n".join(lines)


def _short_name(k: str) -> str:
    """name<args> from a mangled kernel name of this library (bf16, f32 and integer template
    arguments), else the demangled name without its namespace"""
    import re

    m = re.match(r"_ZN5still(\d+)", k)
    if not m:
        return k.split("(")[0].replace("still::", "")
    n = int(m.group(1))
    name = k[m.end():m.end() + n]
    rest = k[m.end() + n:]
    if not rest.startswith("I"):
        return name
    args = []
    for tok in re.findall(r"DF16b|Li\d+E|f|i", rest[1:rest.find("EEv")] if "EEv" in rest else ""):
        args.append({"DF16b": "bf16", "f": "f32", "i": "int"}.get(tok, tok[2:-1]))
    return f"{name}<{','.join(args)}>"


def counters(dirs, match: str = "") -> str:
    val = collections.defaultdict(dict)
    for d in dirs:
        agg = collections.defaultdict(lambda: collections.defaultdict(list))
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if "still" in r["Kernel_Name"] and match in r["Kernel_Name"]:
                    agg[r["Kernel_Name"].split("(")[0]][r["Counter_Name"]].append(float(r["Counter_Value"]))
        for k, v in agg.items():
            for c, xs in v.items():
                val[k][c] = sum(xs) / len(xs)
    coexec = any("SQ_VALU_MFMA_COEXEC_CYCLES" in v for v in val.values())
    dep = any("SQ_WAIT_INST_ANY" in v for v in val.values())
    head = ["kernel", "waves", "VALU / MFMA / LDS / transcendental insts per wave", "VALU per MFMA", "MFMA busy",
            "VALU busy"] + (["both at once"] if coexec else []) + ["waiting (any)"] + \
        (["waiting on dependencies"] if dep else []) + ["LDS bank conflicts"]
    lines = ["| " + " | ".join(head) + " |", "|" + "---|" * len(head)]
    for k, v in val.items():
        w = v.get("SQ_WAVES")
        g = v.get("GRBM_GUI_ACTIVE", 0.0) / 8 * 1024
        if not w or not g:
            continue
        wc = v.get("SQ_WAVE_CYCLES", 0.0)
        per = " / ".join("%.0f" % (v.get(c, 0.0) / w) for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
                                                                 "SQ_INSTS_VALU_TRANS_F32"))
        mf = v.get("SQ_INSTS_MFMA", 0.0)
        cells = [_short_name(k), f"{w:.0f}", per, f"{v.get('SQ_INSTS_VALU', 0.0) / mf:.1f}" if mf else "—",
                 f"{100 * v.get('SQ_VALU_MFMA_BUSY_CYCLES', 0.0) / g:.1f}%",
                 f"{100 * 4 * v.get('SQ_ACTIVE_INST_VALU', 0.0) / g:.1f}%"]
        if coexec:
            cells.append(f"{100 * v.get('SQ_VALU_MFMA_COEXEC_CYCLES', 0.0) / g:.1f}%")
        cells.append(f"{100 * v['SQ_WAIT_ANY'] / wc:.0f}% of wave time" if "SQ_WAIT_ANY" in v and wc else "—")
        if dep:
            cells.append(f"{100 * v['SQ_WAIT_INST_ANY'] / wc:.0f}% of wave time" if "SQ_WAIT_INST_ANY" in v and wc else "—")
        if v.get("SQ_LDS_IDX_ACTIVE"):
            cells.append(f"{100 * v.get('SQ_LDS_BANK_CONFLICT', 0.0) / v['SQ_LDS_IDX_ACTIVE']:.0f}% of LDS cycles")
        else:
            cells.append(f"{v.get('SQ_LDS_BANK_CONFLICT', 0.0) / 1e6:.2f}M cycles")
        lines.append("| " + " | ".join(cells) + " |")
    return "\n".join(lines)


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        print(stats(sys.argv[2]))
    elif sys.argv[1] == "trace":
        print(trace(sys.argv[2], int(sys.argv[3])))
    elif sys.argv[1] == "traffic":
        print(traffic(sys.argv[2], sys.argv[3], int(sys.argv[4]), *sys.argv[5:6], others=sys.argv[6:]))
    elif sys.argv[1] == "counters":
        opts = [a for a in sys.argv[2:] if a.startswith("--match=")]
        print(counters([a for a in sys.argv[2:] if not a.startswith("--match=")],
                       opts[-1].split("=", 1)[1] if opts else ""))
