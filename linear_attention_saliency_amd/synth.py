"""Seeded synthetic inputs for one STILL attention layer.

This module draws inputs only: it holds none of the layer's arithmetic, so both the
fp64 oracle and the HIP path can be fed the identical bits from here.

The workloads mirror the layer shapes the STILL pages run on (a Llama-3.2-1B-shaped
layer at 16K context, Llama-3.1-8B-shaped layers at 4K and 64K, and batched 64K
decoding; page "STILL: Content-Aware Intra-Layer Hybrid Attention Cuts Memory 80%,
Speeds Prefill 83%", summary, and page "STILL: Selecting Tokens for Intra-Layer Hybrid
Attention to Linearize LLMs", sections Key results and Experimental setup). The pages
measure on trained models and public benchmarks; these seeded draws stand in for those
activations and keep only their shapes.

Recipe (fixed, so any consumer can regenerate the same bits):
  rng = numpy.random.default_rng(seed)   (PCG64)
  Q = rng.standard_normal([B,T,Hq,D],  float32) * qk_scale
  K = rng.standard_normal([B,T,Hkv,D], float32) * qk_scale
  V = rng.standard_normal([B,T,Hkv,D], float32) / sqrt(D)
  for b in range(B), for h in range(Hkv):   (in that order)
      pos = rng.choice(T, n_planted, replace=False);  K[b, pos, h, :] *= 4
  W = rng.standard_normal([Hkv,d_f,D], float32) / sqrt(D)     (variance 1/D)
  then every array is rounded to bfloat16 (round-to-nearest-even) unless dtype is f32.
qk_scale is 1/sqrt(D) for the standard workloads and 1 for the routing-stress variant.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    feat_dim: int
    window: int
    chunk: int
    top_k: int
    dtype: str  # "f32" | "bf16"
    seed: int
    n_planted: int | None = None  # None -> round(1% of T)
    qk_scale: float | None = None  # None -> 1/sqrt(D)
    decode_steps: int = 0

    def planted(self) -> int:
        if self.n_planted is not None:
            return self.n_planted
        return int(round(0.01 * self.seq_len))

    def scale(self) -> float:
        return self.qk_scale if self.qk_scale is not None else 1.0 / math.sqrt(self.head_dim)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads (sizes fixed by the layer shapes above).
TINY_F32 = Workload("tiny-f32-T512", 1, 512, 1, 1, 64, 64, 64, 64, 8, "f32", seed=0, n_planted=16)
L1B_16K = Workload("llama3.2-1b-layer-prefill-T16384", 1, 16384, 32, 8, 64, 64, 64, 64, 8, "bf16", seed=1)
L8B_4K = Workload("llama3.1-8b-layer-prefill-B8-T4096", 8, 4096, 32, 8, 128, 128, 64, 64, 16, "bf16", seed=2)
L8B_64K = Workload("llama3.1-8b-layer-prefill-T65536", 1, 65536, 32, 8, 128, 128, 64, 64, 16, "bf16", seed=3)
L8B_DECODE = Workload("llama3.1-8b-layer-decode-B32-ctx65536", 32, 65536, 32, 8, 128, 128, 64, 64, 16,
                      "bf16", seed=4, n_planted=0, decode_steps=64)

WORKLOADS = {w.name: w for w in (TINY_F32, L1B_16K, L8B_4K, L8B_64K, L8B_DECODE)}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The bfloat16 bit patterns (uint16) of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def make_inputs(wl: Workload, seq_len: int | None = None, batch: int | None = None):
    """Draw (q, k, v, w_phi) as float32 numpy arrays whose values are exact in wl.dtype.

    q [B,T,Hq,D], k/v [B,T,Hkv,D], w_phi [Hkv,d_f,D].
    seq_len / batch override the workload's sizes (same recipe, same seed).
    """
    B = wl.batch if batch is None else batch
    T = wl.seq_len if seq_len is None else seq_len
    D, Hq, Hkv, F = wl.head_dim, wl.n_q_heads, wl.n_kv_heads, wl.feat_dim
    rng = np.random.default_rng(wl.seed)
    s = np.float32(wl.scale())
    q = rng.standard_normal((B, T, Hq, D), dtype=np.float32) * s
    k = rng.standard_normal((B, T, Hkv, D), dtype=np.float32) * s
    v = rng.standard_normal((B, T, Hkv, D), dtype=np.float32) * np.float32(1.0 / math.sqrt(D))
    n_pl = min(wl.planted(), T)
    if n_pl > 0:
        for b in range(B):
            for h in range(Hkv):
                pos = rng.choice(T, n_pl, replace=False)
                k[b, pos, h, :] *= np.float32(4.0)
    w = rng.standard_normal((Hkv, F, D), dtype=np.float32) * np.float32(1.0 / math.sqrt(D))
    if wl.dtype == "bf16":
        q, k, v, w = (round_bf16(a) for a in (q, k, v, w))
    return q, k, v, w


def make_grad_out(wl: Workload, seq_len: int | None = None, batch: int | None = None) -> np.ndarray:
    """The gradient of a scalar loss with respect to the layer output, for backward-pass
    cases: N(0, 1/D) entries [B,T,Hq,D] (seed wl.seed + 7919), exact in wl.dtype."""
    B = wl.batch if batch is None else batch
    T = wl.seq_len if seq_len is None else seq_len
    rng = np.random.default_rng(wl.seed + 7919)
    g = rng.standard_normal((B, T, wl.n_q_heads, wl.head_dim), dtype=np.float32) * np.float32(1.0 / math.sqrt(wl.head_dim))
    return round_bf16(g) if wl.dtype == "bf16" else g


def small_case(seed: int, B: int, T: int, Hq: int, Hkv: int, D: int, F: int, window: int,
               chunk: int, top_k: int, dtype: str = "f32", qk_scale: float | None = None,
               n_planted: int = 0) -> tuple[Workload, tuple]:
    """A small workload for parity tests, drawn with the same recipe."""
    wl = Workload(f"case-s{seed}", B, T, Hq, Hkv, D, F, window, chunk, top_k, dtype, seed,
                  n_planted=n_planted, qk_scale=qk_scale)
    return wl, make_inputs(wl)


def make_inputs_device(wl: Workload, device, seq_len: int | None = None, batch: int | None = None,
                       seed_offset: int = 0):
    """The same distributions drawn on the device with torch's generator (seed wl.seed +
    seed_offset), for sizes where drawing on the host would dominate a benchmark. Returns
    device tensors q, k, v, w_phi in wl.dtype. These bits differ from make_inputs'."""
    import torch

    B = wl.batch if batch is None else batch
    T = wl.seq_len if seq_len is None else seq_len
    D, Hq, Hkv, F = wl.head_dim, wl.n_q_heads, wl.n_kv_heads, wl.feat_dim
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed + seed_offset)
    s = wl.scale()

    def draw(shape, scale):
        out = torch.empty(shape, dtype=dt, device=device)
        for b in range(shape[0]):  # one sequence at a time keeps the fp32 temporary small
            out[b] = (torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32) * scale).to(dt)
        return out

    q = draw((B, T, Hq, D), s)
    k = draw((B, T, Hkv, D), s)
    v = draw((B, T, Hkv, D), 1.0 / math.sqrt(D))
    n_pl = min(wl.planted(), T)
    if n_pl > 0:
        for b in range(B):
            for h in range(Hkv):
                pos = torch.randperm(T, generator=g, device=device)[:n_pl]
                k[b, pos, h, :] = (k[b, pos, h, :].float() * 4.0).to(dt)
    w = (torch.randn((Hkv, F, D), generator=g, device=device, dtype=torch.float32) / math.sqrt(D)).to(dt)
    return q.contiguous(), k.contiguous(), v.contiguous(), w.contiguous()
