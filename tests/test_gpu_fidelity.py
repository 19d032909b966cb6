"""Parity of the local-global consistency diagnostic (through the C ABI) with the oracle.

The attention each key receives from far-future queries (full causal softmax) is compared
with the oracle's as max-abs error relative to the largest oracle value: 1e-4 in fp32 and
2e-4 in bf16 (the inputs are exact in both; every product and sum runs in fp32). The
per-chunk top-k of that mass is bit-exact wherever the oracle's k-th/(k+1)-th gap exceeds
both 1e-5 of the largest value and 50 times the measured error, and the overlap counts are
exact integers.
"""

import sys
import zlib

import numpy as np
import pytest
import torch

from linear_attention_saliency_amd import still, synth
from oracle import still_oracle as O

pytestmark = pytest.mark.gpu

REL_TOL = {"f32": 1e-4, "bf16": 2e-4}


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32).contiguous()


CASES = [
    # name, B, T, Hq, Hkv, w, k, dtype, qk_scale
    ("f32-ragged", 1, 300, 2, 1, 64, 8, "f32", 1.0),
    ("bf16-gqa4", 2, 333, 8, 2, 64, 8, "bf16", 1.0),
    ("bf16-window16", 1, 260, 4, 1, 16, 8, "bf16", None),
    ("bf16-window0", 1, 200, 2, 1, 0, 0, "bf16", 1.0),
    ("bf16-short", 1, 37, 4, 1, 64, 8, "bf16", 1.0),
    ("f32-k16", 1, 512, 2, 1, 64, 16, "f32", 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fidelity_matches_oracle(case):
    name, B, T, Hq, Hkv, w, k, dt, sc = case
    _say(name)
    wl, (q, kk, v, wp) = synth.small_case(seed=zlib.crc32(name.encode()) % 1000, B=B, T=T, Hq=Hq, Hkv=Hkv, D=64,
                                           F=64, window=w, chunk=64, top_k=k, dtype=dt, qk_scale=sc,
                                           n_planted=max(1, T // 50))
    tq, tk, tw = _dev(q, dt), _dev(kk, dt), _dev(wp, dt)
    mass = still.future_attention_mass(tq, tk, window=w)
    torch.cuda.synchronize()
    got = mass.cpu().numpy().astype(np.float64)
    ref = O.future_attention_mass(q, kk, w)
    abs_err = float(np.abs(got - ref).max())
    e = abs_err / max(np.abs(ref).max(), 1e-30)
    _say(name, "mass rel max err", e)
    assert e <= REL_TOL[dt]
    if k == 0 or T < 64:
        return
    fid = still.saliency_fidelity(tq, tk, tw, window=w, top_k=k)
    sel_g = fid["sel_global"].cpu().numpy()
    ref_idx, _ = O.route(ref, 64, k)
    margins = O.route_margins(ref, 64, k)
    decided = margins > max(1e-5 * np.abs(ref).max(), 50 * abs_err)
    same = np.all(sel_g == ref_idx, axis=-1)
    assert np.all(same[decided]), f"global top-k differs in {int((~same[decided]).sum())} decided chunks"
    common = fid["common"].cpu().numpy()
    assert np.array_equal(common, O.selection_overlap(fid["sel_local"].cpu().numpy(), sel_g))
    _say(name, "decided", int(decided.sum()), "of", decided.size, "overlap", fid["overlap"])


def test_mass_at_headline_shape():
    """16K Llama-3.2-1B-shaped layer: the keys of the last four chunks and the window before
    them against the oracle's exact tail, and, with window 0, the identity that every row's
    probabilities sum to 1 (the mass of a KV head sums to G * T)."""
    wl = synth.L1B_16K
    _say("mass headline", wl.name)
    q, k, _, _ = synth.make_inputs(wl)
    tq, tk = _dev(q, "bf16"), _dev(k, "bf16")
    T, w, G = wl.seq_len, wl.window, wl.n_q_heads // wl.n_kv_heads
    mass = still.future_attention_mass(tq, tk, window=w)
    torch.cuda.synchronize()
    got = mass.cpu().numpy().astype(np.float64)
    t0 = T - 4 * wl.chunk
    ref = O.future_attention_mass(q, k, w, q_from=t0)
    lo = t0 - w
    e = float(np.abs(got[..., lo:] - ref[..., lo:]).max() / np.abs(ref[..., lo:]).max())
    _say("headline mass rel max err over the last", T - lo, "keys", e)
    assert e <= REL_TOL["bf16"]
    m0 = still.future_attention_mass(tq, tk, window=0)
    torch.cuda.synchronize()
    tot = m0.double().sum(dim=-1).cpu().numpy()
    e0 = float(np.abs(tot - G * T).max() / (G * T))
    _say("headline window-0 mass sum rel err", e0)
    assert e0 <= 1e-4
