"""Benchmark of one STILL hybrid attention layer on one MI355X. Prints one JSON line.

Default workload: prefill of the Llama-3.2-1B-shaped layer at 16384 tokens (batch 1,
32 query / 8 KV heads, head_dim 64, window 64, chunk 64, top_k 8, NP-Map dim 64, bf16 in,
fp32 accumulate), on seeded synthetic inputs that are resident in HBM before timing
starts. A step is one still_prefill call: saliency, per-chunk top-k, gather, NP-Map,
chunk states, prefix scan and the fused softmax + linear attention.

--workload selects another layer shape: l8b-4k (Llama-3.1-8B-shaped, 8 x 4096 tokens),
l8b-64k (1 x 65536 tokens), or l8b-decode: 32 sequences whose 65536-token prefix is put
into a decode cache by one still_prefill call, then one still_decode_step per generated
token (a step = one token for all 32 sequences; 64 timed steps cross one chunk boundary,
so one selection / append / fold is inside the timed window).

  python bench.py [--workload W] [--steps K] [--warmup W] [--no-cpu-baseline] [--calibrate-copy]

--calibrate-copy runs one device-to-device copy of COPY_BYTES before anything else (the
run's first copy dispatch), so that a rocprofv3 --pmc run of this script also records what
FETCH_SIZE / WRITE_SIZE read for a transfer of known size (the scale applied to the
dominant kernel's counters).
The roofline "traffic" field is read from profiles/attn_kernel_traffic_<workload>.txt when
that file was measured on this workload and the current attention-kernel source (matching
SHA-1), else null.
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
def traffic_file(workload_key: str) -> str:
    """The committed HBM-traffic summary of the attention kernel on one prefill workload."""
    return os.path.join(ROOT, "profiles", f"attn_kernel_traffic_{workload_key}.txt")
# the decode compact-cache kernel's source and the headers it includes
DECODE_SRCS = [os.path.join(_CSRC, f) for f in ("still_decode.hip", "still_common.hpp", "still_layout.hpp",
                                                "still_launch.hpp", "still_route.hpp")]
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_split_kernel_traffic.txt")


def source_sha1(paths) -> str:
    import hashlib

    h = hashlib.sha1()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, path: str, srcs=ATTN_SRCS):
    """HBM bytes per launch of the bench's dominant kernel from a committed counter
    summary, if it was taken on this workload and the current kernel source; else None."""
    try:
        kv = dict(line.split(":", 1) for line in open(path) if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    if kv.get("workload", "").strip() != workload:
        return None
    if kv.get("source_sha1", "").strip() != source_sha1(srcs):
        return None
    return float(kv["hbm_bytes_per_launch"])
PEAK_BF16_MFMA = 2.5e15   # dense, FLOP/s
SETTLE_STEPS = 100        # untimed prefill steps before the timed ones, --warmup included
PEAK_HBM = 8.0e12         # bytes/s


def algorithmic_work(wl, sel_idx: np.ndarray, score: str = "saliency") -> dict:
    """Algorithmic flops and bytes of the layer, from the routing the device chose.

    Softmax: 4*D flops per (query head, softmax key) pair, the keys being the window
    plus every selected key outside it. Linear attention: the recurrent minimum, 2*F*D+2*F
    per query-head token (read-out) plus the same per KV-head token (state update).
    NP-Map: 2*D*F per query-head and per KV-head row. Saliency: 2*D per (query head,
    window key); routed by the diagonal logit, 2*D per query head. Bytes: Q, K, V and O once
    each (bf16), plus the NP-Map weights.
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
    sal = 2.0 * D * (float(np.sum(win)) if score == "saliency" else float(T)) * Hq * B
    esz = 2 if wl.dtype == "bf16" else 4
    bytes_ = esz * (B * T * (2 * Hq + 2 * Hkv) * D + Hkv * F * D)
    return {"flops": sa + la_q + la_k + np_q + np_k + sal, "bytes": float(bytes_),
            "attn_flops": sa + la_q + np_q, "sa_pairs": pairs}


def attention_kernel_name(wl, scope: str) -> str:
    """The attention kernel the library launches for this layer: the fixed-frame kernel for
    bf16 with head_dim = feat_dim (64 or 128), window = chunk and groups of four query heads
    per routing head, else the general one."""
    group = wl.n_q_heads // wl.n_kv_heads if scope == "kv_head" else 1
    if (wl.dtype == "bf16" and wl.head_dim == wl.feat_dim and wl.head_dim in (64, 128) and wl.window == wl.chunk
            and group % 4 == 0):
        return "attn_ff_kernel"
    return "attn_kernel"


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


def _events(torch, still, n_steps, per_step):
    """Timing events (device-scope release, so a record between kernels costs no system-scope
    cache write-back) and their raw handles for the *_timed entry points."""
    evs = [[still.TimingEvent() for _ in range(per_step)] for _ in range(n_steps)]
    import ctypes
    handles = [(ctypes.c_void_p * per_step)(*[e.handle for e in step]) for step in evs]
    torch.cuda.synchronize()
    return evs, handles


def run_prefill(wl, args, torch, still, synth) -> dict:
    dev = torch.device("cuda:0")
    q, k, v, w = synth.make_inputs(wl)
    tq, tk, tv, tw = (torch.from_numpy(a).to(dev, torch.bfloat16).contiguous() for a in (q, k, v, w))
    if not (wl is synth.L1B_16K and not args.no_cpu_baseline):
        del q, k, v, w
    out = torch.empty_like(tq)
    call = still.Prefill(tq, tk, tv, tw, window=wl.window, top_k=wl.top_k, chunk=wl.chunk, score=args.score,
                         scope=args.scope)
    n_sel_heads = wl.n_q_heads if args.scope == "query_head" else wl.n_kv_heads
    sel = torch.empty((wl.batch, n_sel_heads, wl.seq_len // wl.chunk, wl.top_k), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    # inside the timed region only the attention kernel is bracketed (two events per step);
    # the other kernels' durations come from a short untimed pass with all four afterwards
    evs, handles = _events(torch, still, args.steps, 2)
    import ctypes
    attn_only = [(ctypes.c_void_p * 4)(None, None, h[0], h[1]) for h in handles]
    n_side = min(args.steps, 10)
    side, side_h = _events(torch, still, n_side, 4)
    t_start = still.TimingEvent()
    t_end = still.TimingEvent()
    torch.cuda.reset_peak_memory_stats()
    # the routing call, the warm-up and the timed steps run back to back; the host-side work
    # count (a few ms of NumPy) comes after the timed region
    call(tq, tk, tv, tw, out, sel_idx=sel)  # the routing the device chooses (for the work count)
    # clock settling: the GPU's clocks take tens of ms of load to reach their steady state, so
    # at least SETTLE_STEPS untimed steps run before the timed ones, whatever --warmup asks
    settle = max(0, SETTLE_STEPS - args.warmup)
    for _ in range(settle + args.warmup):
        call(tq, tk, tv, tw, out)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.steps):
        call(tq, tk, tv, tw, out, events=attn_only[s])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    attn_ms = float(np.mean([step[0].elapsed_time(step[1]) for step in evs]))
    for s in range(n_side):
        call(tq, tk, tv, tw, out, events=side_h[s])
    torch.cuda.synchronize()
    k_ms = np.array([[step[j].elapsed_time(step[j + 1]) for j in range(2)] for step in side])
    prep_ms, scan_ms = (float(x) for x in k_ms.mean(axis=0))
    sel_idx = sel.cpu().numpy()
    work = algorithmic_work(wl if args.scope == "kv_head" else wl.replace(n_kv_heads=wl.n_q_heads), sel_idx, args.score)

    tokens = wl.batch * wl.seq_len
    value = tokens / (ms_step * 1e-3)
    attn_ach = work["attn_flops"] / (attn_ms * 1e-3)
    layer_tflops = work["flops"] / (ms_step * 1e-3)
    layer_gbs = work["bytes"] / (ms_step * 1e-3)
    esz = 2
    io_bytes = esz * wl.batch * wl.seq_len * (2 * wl.n_q_heads + 2 * wl.n_kv_heads) * wl.head_dim
    res = {
        "metric": METRIC if wl is synth.L1B_16K else
        f"prefill tokens/s per layer ({wl.name}, bf16); % of HBM/MFMA roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1)/sqrt(D) Q/K/V, 1% planted keys x4, W_phi N(0,1/D); bf16",
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.seq_len, "n_q_heads": wl.n_q_heads,
                   "n_kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "feat_dim": wl.feat_dim,
                   "window": wl.window, "chunk": wl.chunk, "top_k": wl.top_k, "score": args.score,
                   "routing_scope": args.scope},
        "roofline": {"bound": "mfma", "kernel": attention_kernel_name(wl, args.scope), "achieved": attn_ach / 1e12,
                     "peak": PEAK_BF16_MFMA / 1e12, "unit": "TFLOP/s", "frac": attn_ach / PEAK_BF16_MFMA,
                     "traffic": measured_traffic(wl.name, traffic_file(args.workload))},
        "layer_roofline": {"flops": work["flops"], "bytes": work["bytes"],
                           "mfma_frac": layer_tflops / PEAK_BF16_MFMA, "hbm_frac": layer_gbs / PEAK_HBM,
                           "frac": max(layer_tflops / PEAK_BF16_MFMA, layer_gbs / PEAK_HBM)},
        "kernel_ms": {"prep": prep_ms, "scan": scan_ms, "attn": attn_ms},
        "memory": {"peak_allocated_bytes": int(torch.cuda.max_memory_allocated()),
                   "io_bytes": int(io_bytes), "workspace_bytes": int(call.workspace.numel()),
                   "dense_scores_bf16_bytes": int(2 * wl.batch * wl.n_q_heads * wl.seq_len * wl.seq_len)},
        "wall_s": wall,
    }
    if wl is synth.L1B_16K and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, q, k, v, w, sel_idx)
    return res


BWD_STAGES = ("kprep", "scan_fwd", "dq", "scan_rev", "dkv_far", "dkv_local", "dw")


def backward_work(wl, sel_idx) -> dict:
    """Algorithmic flops of the backward pass, from the routing.

    Softmax pairs (query head, softmax key) as in the forward count: 10*D flops each (the
    scores recomputed, dout.v, and the dq, dk and dv products). Linear attention: 4*F*D per
    query-head token (S_c dout and its share of R) and 4*F*D per KV-head token (R v and
    R^T phi(k)). NP-Map: 6*F*D per query-head and per KV-head row (W x recomputed, W^T dz and
    dz x^T).
    """
    fw = algorithmic_work(wl, sel_idx)
    B, T, Hq, Hkv, D, F = wl.batch, wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.feat_dim
    sa = 10.0 * D * fw["sa_pairs"]
    la = 4.0 * F * D * (Hq + Hkv) * B * T
    npm = 6.0 * F * D * (Hq + Hkv) * B * T
    return {"flops": sa + la + npm, "sa_flops": sa}


def run_backward(wl, args, torch, still, synth) -> dict:
    dev = torch.device("cuda:0")
    q, k, v, w = synth.make_inputs(wl)
    dout = synth.make_grad_out(wl)
    tq, tk, tv, tw, tdo = (torch.from_numpy(a).to(dev, torch.bfloat16).contiguous() for a in (q, k, v, w, dout))
    del q, k, v, w, dout
    out, sel = still.prefill(tq, tk, tv, tw, window=wl.window, top_k=wl.top_k, return_routing=True)
    call = still.Backward(tq, tk, tv, tw, window=wl.window, top_k=wl.top_k)
    dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
    dw = torch.empty(tw.shape, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    work = backward_work(wl, sel.cpu().numpy())
    for _ in range(args.warmup):
        call(tq, tk, tv, tw, out, tdo, sel, dq, dk, dv, dw)
    stream = torch.cuda.current_stream()
    evs, handles = _events(torch, still, args.steps, 8)
    t_start = still.TimingEvent()
    t_end = still.TimingEvent()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s_ in range(args.steps):
        call(tq, tk, tv, tw, out, tdo, sel, dq, dk, dv, dw, events=handles[s_])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    k_ms = np.array([[step[j].elapsed_time(step[j + 1]) for j in range(7)] for step in evs]).mean(axis=0)
    stage_ms = {n: float(x) for n, x in zip(BWD_STAGES, k_ms)}
    tflops = work["flops"] / (ms_step * 1e-3)
    dom = max(("dq", "dkv_far", "dkv_local"), key=lambda n: stage_ms[n])
    return {
        "metric": f"backward tokens/s per layer ({wl.name}, bf16, routing fixed); % of MFMA roofline",
        "value": wl.batch * wl.seq_len / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1)/sqrt(D) Q/K/V and dout, 1% planted keys x4, W_phi N(0,1/D); bf16",
        "config": {"workload": wl.name + "-backward", "batch": wl.batch, "seq_len": wl.seq_len,
                   "n_q_heads": wl.n_q_heads, "n_kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim,
                   "feat_dim": wl.feat_dim, "window": wl.window, "chunk": wl.chunk, "top_k": wl.top_k},
        "roofline": {"bound": "mfma", "kernel": "whole backward pass", "achieved": tflops / 1e12,
                     "peak": PEAK_BF16_MFMA / 1e12, "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_MFMA,
                     "traffic": None},
        "dominant_stage": dom,
        "kernel_ms": stage_ms,
        "flops": work["flops"],
        "memory": {"workspace_bytes": int(call.workspace.numel())},
        "wall_s": wall,
    }


def run_fidelity(wl, args, torch, still, synth) -> dict:
    """The local-global consistency diagnostic on the workload: attention from far-future
    queries under full causal softmax (timed), its per-chunk top-k, and the overlap with the
    layer's own routing."""
    dev = torch.device("cuda:0")
    q, k, v, w = synth.make_inputs(wl)
    tq, tk, tw = (torch.from_numpy(a).to(dev, torch.bfloat16).contiguous() for a in (q, k, w))
    del q, k, v, w
    B, T, Hq, D = tq.shape
    Hkv = tk.shape[2]
    call = still.FutureAttentionMass(tq, tk, window=wl.window)
    mass = torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        call(tq, tk, mass)
    e0, e1 = still.TimingEvent(), still.TimingEvent()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        call(tq, tk, mass)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = e0.elapsed_time(e1) / args.steps
    fid = still.saliency_fidelity(tq, tk, tw, window=wl.window, top_k=wl.top_k)
    wd = wl.window
    pairs = T * (T + 1) / 2.0 + (T - wd) * (T - wd + 1) / 2.0  # both passes, per query head
    flops = 2.0 * D * pairs * Hq * B
    ach = flops / (ms * 1e-3)
    return {
        "metric": f"far-future attention mass, tokens/s per layer ({wl.name}, bf16); % of MFMA roofline",
        "value": B * T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1)/sqrt(D) Q/K, 1% planted keys x4; bf16",
        "config": {"workload": wl.name + "-fidelity", "batch": B, "seq_len": T, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "head_dim": D, "window": wl.window, "chunk": wl.chunk, "top_k": wl.top_k},
        "roofline": {"bound": "mfma", "kernel": "mass_lse_kernel + mass_col_kernel", "achieved": ach / 1e12,
                     "peak": PEAK_BF16_MFMA / 1e12, "unit": "TFLOP/s", "frac": ach / PEAK_BF16_MFMA, "traffic": None},
        "overlap": fid["overlap"],
        "wall_s": wall,
    }


def run_decode(wl, args, torch, still, synth) -> dict:
    dev = torch.device("cuda:0")
    B, Hq, Hkv, D, F = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.feat_dim
    T0, C = wl.seq_len, wl.chunk
    n_tok = args.warmup + args.steps
    cache = still.DecodeCache(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, feat_dim=F, window=wl.window,
                              top_k=wl.top_k, max_tokens=T0 + n_tok, dtype=torch.bfloat16, device=dev,
                              score=args.score)
    # the 64K-token prefix of all sequences goes into the cache through one prefill
    q, k, v, w = synth.make_inputs_device(wl, dev)
    out = torch.empty_like(q)
    call = still.Prefill(q, k, v, w, window=wl.window, top_k=wl.top_k, chunk=C, score=args.score)
    e0, e1 = still.TimingEvent(), still.TimingEvent()
    e0.record()
    call(q, k, v, w, out, cache=cache)
    e1.record()
    torch.cuda.synchronize()
    prefill_ms = e0.elapsed_time(e1)
    del q, k, v, out, call
    torch.cuda.empty_cache()
    # the generated tokens: step t uses [:, t]
    qs, ks, vs, _ = synth.make_inputs_device(wl, dev, seq_len=n_tok, seed_offset=1)
    toks = [(qs[:, t].contiguous(), ks[:, t].contiguous(), vs[:, t].contiguous()) for t in range(n_tok)]
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    for t in range(args.warmup):
        cache.step(*toks[t], w, out)
    stream = torch.cuda.current_stream()
    evs, handles = _events(torch, still, args.steps, 3)
    pos0 = cache.n_tokens
    t_start = still.TimingEvent()
    t_end = still.TimingEvent()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.steps):
        cache.step(*toks[args.warmup + s], w, out, events=handles[s])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    k_ms = np.array([[step[j].elapsed_time(step[j + 1]) for j in range(2)] for step in evs])
    split_ms, token_ms = (float(x) for x in k_ms.mean(axis=0))

    # algorithmic bytes: the compact rows each step must read (K and V, bf16), per launch
    nsel = [max(0, (p // C) - 1) * wl.top_k for p in range(pos0, pos0 + args.steps)]
    split_bytes = float(np.mean(nsel)) * B * Hkv * 2 * D * 2
    ring_bytes = B * Hkv * 2 * C * D * 2 * 2      # chunks c-1 and c, K and V
    state_bytes = B * Hkv * (F * D + F) * 4
    io_bytes = 2 * (2 * B * Hq * D + 2 * B * Hkv * D) + Hkv * F * D * 2
    step_bytes = split_bytes + ring_bytes + state_bytes + io_bytes
    ach = split_bytes / (split_ms * 1e-3)
    return {
        "metric": f"decode tokens/s per layer ({wl.name}, bf16); % of HBM roofline",
        "value": B / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded (torch generator on the device) N(0,1)/sqrt(D) Q/K/V, W_phi N(0,1/D); bf16",
        "config": {"workload": wl.name, "batch": B, "context": T0, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "head_dim": D, "feat_dim": F, "window": wl.window, "chunk": C, "top_k": wl.top_k,
                   "score": args.score},
        "roofline": {"bound": "hbm", "kernel": "decode_split_kernel", "achieved": ach / 1e9,
                     "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": ach / PEAK_HBM,
                     "traffic": measured_traffic(wl.name, DECODE_TRAFFIC_FILE, DECODE_SRCS)},
        "layer_roofline": {"bytes": step_bytes, "hbm_frac": step_bytes / (ms_step * 1e-3) / PEAK_HBM},
        "kernel_ms": {"split": split_ms, "token": token_ms},
        "memory": {"cache_bytes": int(cache.buffer.numel()), "compact_rows_per_head": int(max(nsel)),
                   "dense_kv_bytes": int(2 * B * Hkv * (T0 + n_tok) * D * 2)},
        "prefill_into_cache_ms": prefill_ms,
        "wall_s": wall,
    }


WORKLOAD_NAMES = {"l1b-16k": "L1B_16K", "l8b-4k": "L8B_4K", "l8b-64k": "L8B_64K", "l8b-decode": "L8B_DECODE"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", choices=sorted(WORKLOAD_NAMES), default="l1b-16k")
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 50; 64 for decode)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps (default 100 for prefill, enough for the clocks to settle; 8 for decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--top-k", type=int, default=None,
                    help="override the workload's top_k on the same kernels: 0 gives the sliding-window plus "
                         "linear-attention baseline, 64 (= chunk) full causal softmax")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (routing fixed) instead of the forward")
    ap.add_argument("--fidelity", action="store_true",
                    help="time the local-global consistency diagnostic (far-future attention mass)")
    ap.add_argument("--scope", choices=["kv_head", "query_head"], default="kv_head",
                    help="who selects: each KV head for its group, or each query head for itself (prefill)")
    ap.add_argument("--score", choices=["saliency", "diag"], default="saliency",
                    help="routing score: the Self-Saliency Score, or the diagonal logit alone")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (every step is "
              "independent per (batch, KV head), so more GPUs would shard heads with no exchange)",
              file=sys.stderr)
        return 2

    import torch

    from linear_attention_saliency_amd import still, synth

    if args.calibrate_copy:  # the run's first device-to-device copy: COPY_BYTES read and written
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    wl = getattr(synth, WORKLOAD_NAMES[args.workload])
    if args.top_k is not None and args.top_k != wl.top_k:
        wl = wl.replace(top_k=args.top_k, name=f"{wl.name}-k{args.top_k}")
    if args.score != "saliency":
        wl = wl.replace(name=f"{wl.name}-{args.score}")
    if args.scope != "kv_head":
        wl = wl.replace(name=f"{wl.name}-per-query-head")
    decode = wl.decode_steps > 0
    if args.steps is None:
        args.steps = 64 if decode else 50
    if args.warmup is None:
        args.warmup = 8 if decode else 100
    if args.scope != "kv_head" and (decode or args.backward or args.fidelity):
        print("--scope query_head is timed for prefill only", file=sys.stderr)
        return 2
    if args.fidelity:
        if decode or wl.head_dim != 64:
            print("--fidelity covers prefill workloads with head_dim 64", file=sys.stderr)
            return 2
        res = run_fidelity(wl, args, torch, still, synth)
    elif args.backward:
        if decode or wl.head_dim != wl.feat_dim or wl.head_dim not in (64, 128):
            print("--backward covers prefill workloads with head_dim = feat_dim = 64 or 128", file=sys.stderr)
            return 2
        res = run_backward(wl, args, torch, still, synth)
    else:
        res = (run_decode if decode else run_prefill)(wl, args, torch, still, synth)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
