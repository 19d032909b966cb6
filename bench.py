"""Benchmark of one STILL hybrid attention layer (prefill) on one MI355X.

Workload: the Llama-3.2-1B-shaped layer at 16384 tokens (batch 1, 32 query / 8 KV heads,
head_dim 64, window 64, chunk 64, top_k 8, NP-Map dim 64, bf16 in, fp32 accumulate), on
seeded synthetic inputs that are resident in HBM before timing starts.

A step is one still_prefill call: saliency, per-chunk top-k, gather, NP-Map, chunk
states, prefix scan and the fused softmax + linear attention. Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--calibrate-copy]

--calibrate-copy runs one device-to-device copy of COPY_BYTES before the steps, so that
a rocprofv3 --pmc run of this script also records what FETCH_SIZE / WRITE_SIZE read for a
transfer of known size (the scale applied to the attention kernel's counters).
The roofline "traffic" field is read from profiles/attn_kernel_traffic.txt when that
file was measured on the current attention-kernel source (matching SHA-1), else null.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s per layer at 16K (bf16); % of HBM/MFMA roofline"
COPY_BYTES = 256 << 20
_CSRC = os.path.join(ROOT, "linear_attention_saliency_amd", "csrc")
# the attention kernel's source and every header it includes
ATTN_SRCS = [os.path.join(_CSRC, f) for f in ("still_attn.hip", "still_common.hpp", "still_layout.hpp",
                                              "still_launch.hpp", "still_route.hpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kernel_traffic.txt")


def source_sha1(paths) -> str:
    import hashlib

    h = hashlib.sha1()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per attention-kernel launch from the committed counter summary, if it
    was taken on the current kernel source; None otherwise."""
    try:
        kv = dict(line.split(":", 1) for line in open(TRAFFIC_FILE) if ":" in line)
    except OSError:
        return None
    if kv.get("attn_source_sha1", "").strip() != source_sha1(ATTN_SRCS):
        return None
    return float(kv["hbm_bytes_per_launch"])
PEAK_BF16_MFMA = 2.5e15   # dense, FLOP/s
PEAK_HBM = 8.0e12         # bytes/s


def algorithmic_work(wl, sel_idx: np.ndarray) -> dict:
    """Algorithmic flops and bytes of the layer, from the routing the device chose.

    Softmax: 4*D flops per (query head, softmax key) pair, the keys being the window
    plus every selected key outside it. Linear attention: the recurrent minimum, 2*F*D+2*F
    per query-head token (read-out) plus the same per KV-head token (state update).
    NP-Map: 2*D*F per query-head and per KV-head row. Saliency: 2*D per (query head,
    window key). Bytes: Q, K, V and O once each (bf16), plus the NP-Map weights.
    """
    B, T, Hq, Hkv, D, F = wl.batch, wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.feat_dim
    w, C = wl.window, wl.chunk
    G = Hq // Hkv
    i = np.arange(T)
    win = np.minimum(i + 1, w).astype(np.float64)
    pairs = 0.0
    for b in range(B):
        for h in range(Hkv):
            pos = np.sort(sel_idx[b, h].reshape(-1))
            # selected keys of earlier chunks that are out of query i's window (j <= i - w)
            lim = np.minimum(i - w, (i // C) * C - 1)
            n_out = np.searchsorted(pos, lim, side="right").astype(np.float64)
            pairs += float(np.sum(win + n_out)) * G
    sa = 4.0 * D * pairs
    la_q = (2.0 * F * D + 2.0 * F) * Hq * B * T
    la_k = (2.0 * F * D + 2.0 * F) * Hkv * B * T
    np_q = 2.0 * D * F * Hq * B * T
    np_k = 2.0 * D * F * Hkv * B * T
    sal = 2.0 * D * float(np.sum(win)) * Hq * B
    esz = 2 if wl.dtype == "bf16" else 4
    bytes_ = esz * (B * T * (2 * Hq + 2 * Hkv) * D + Hkv * F * D)
    return {"flops": sa + la_q + la_k + np_q + np_k + sal, "bytes": float(bytes_),
            "attn_flops": sa + la_q + np_q, "sa_pairs": pairs}


def cpu_baseline(wl, q, k, v, w, sel_idx) -> dict:
    """The fp64 oracle on the whole layer (all KV heads, all tokens), timed on the host."""
    import threadpoolctl
    from oracle import still_oracle as O

    t0 = time.perf_counter()
    s_kv, _ = O.saliency(q, k, wl.window)
    _, sel = O.route(s_kv, wl.chunk, wl.top_k)
    O.attend(q, k, v, w, wl.window, wl.chunk, wl.top_k, sel=sel)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] + [1])
    return {"value": wl.batch * wl.seq_len / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the whole layer ({wl.n_kv_heads} KV heads, {wl.n_q_heads} query heads, {wl.seq_len} "
                      f"tokens) in {dt:.1f} s on a host with {os.cpu_count()} CPUs"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (every step is "
              "independent per (batch, KV head), so more GPUs would shard heads with no exchange)",
              file=sys.stderr)
        return 2

    import torch

    from linear_attention_saliency_amd import still, synth

    wl = synth.L1B_16K
    q, k, v, w = synth.make_inputs(wl)
    dev = torch.device("cuda:0")
    tq, tk, tv, tw = (torch.from_numpy(a).to(dev, torch.bfloat16).contiguous() for a in (q, k, v, w))
    out = torch.empty_like(tq)
    call = still.Prefill(tq, tk, tv, tw, window=wl.window, top_k=wl.top_k, chunk=wl.chunk)
    sel = torch.empty((wl.batch, wl.n_kv_heads, wl.seq_len // wl.chunk, wl.top_k), dtype=torch.int32, device=dev)
    call(tq, tk, tv, tw, out, sel_idx=sel)
    torch.cuda.synchronize()
    sel_idx = sel.cpu().numpy()
    work = algorithmic_work(wl, sel_idx)

    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        call(tq, tk, tv, tw, out)
    stream = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for step in evs:  # torch creates the underlying HIP event on first record
        for e in step:
            e.record(stream)
    import ctypes
    handles = [(ctypes.c_void_p * 4)(*[e.cuda_event for e in step]) for step in evs]
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.steps):
        call(tq, tk, tv, tw, out, events=handles[s])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    k_ms = np.array([[step[j].elapsed_time(step[j + 1]) for j in range(3)] for step in evs])
    prep_ms, scan_ms, attn_ms = (float(x) for x in k_ms.mean(axis=0))

    tokens = wl.batch * wl.seq_len
    value = tokens / (ms_step * 1e-3)
    attn_ach = work["attn_flops"] / (attn_ms * 1e-3)
    layer_tflops = work["flops"] / (ms_step * 1e-3)
    layer_gbs = work["bytes"] / (ms_step * 1e-3)
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1)/sqrt(D) Q/K/V, 1% planted keys x4, W_phi N(0,1/D); bf16",
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.seq_len, "n_q_heads": wl.n_q_heads,
                   "n_kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "feat_dim": wl.feat_dim,
                   "window": wl.window, "chunk": wl.chunk, "top_k": wl.top_k},
        "roofline": {"bound": "mfma", "kernel": "attn_kernel", "achieved": attn_ach / 1e12,
                     "peak": PEAK_BF16_MFMA / 1e12, "unit": "TFLOP/s", "frac": attn_ach / PEAK_BF16_MFMA,
                     "traffic": measured_traffic()},
        "layer_roofline": {"flops": work["flops"], "bytes": work["bytes"],
                           "mfma_frac": layer_tflops / PEAK_BF16_MFMA, "hbm_frac": layer_gbs / PEAK_HBM,
                           "frac": max(layer_tflops / PEAK_BF16_MFMA, layer_gbs / PEAK_HBM)},
        "kernel_ms": {"prep": prep_ms, "scan": scan_ms, "attn": attn_ms},
        "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, q, k, v, w, sel_idx)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
