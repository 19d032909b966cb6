"""Parity of the backward pass (through the C ABI) with the fp64 oracle's gradients.

The routing is the one the device's forward pass chose; the oracle differentiates the
dense form of the layer under that routing. Bars, as max-abs error over a tensor relative
to that tensor's largest oracle entry (at least 1e-3): 1e-4 in fp32 (fp32 MFMA sums, the fp32 output in
Delta) and 3e-2 in bf16 (every MFMA operand, including the probabilities and the scores'
gradients, is rounded to bf16, and Delta uses the bf16-rounded output).
"""

import sys
import zlib

import numpy as np
import pytest
import torch

import parity_check as PC
from linear_attention_saliency_amd import still, synth
from oracle import still_oracle as O

pytestmark = pytest.mark.gpu

REL_TOL = {"f32": 1e-4, "bf16": 3e-2}


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32).contiguous()


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _sel_from_idx(idx, T):
    B, H, nc, k = idx.shape
    sel = np.zeros((B, H, T), dtype=bool)
    for b in range(B):
        for h in range(H):
            sel[b, h, idx[b, h].reshape(-1)] = True
    return sel


def _forward_backward(wl, q, k, v, w, dout):
    dt = wl.dtype
    tq, tk, tv, tw, tdo = (_dev(a, dt) for a in (q, k, v, w, dout))
    out, idx = still.prefill(tq, tk, tv, tw, window=wl.window, top_k=wl.top_k, return_routing=True)
    dq, dk, dv, dw = still.backward(tq, tk, tv, tw, out, tdo, idx, window=wl.window, top_k=wl.top_k)
    torch.cuda.synchronize()
    return out, idx, (dq, dk, dv, dw)


def _rel_err(got, ref):
    # a floor of 1e-3 (gradients here are of order 0.1 to 1): where the exact gradient is 0,
    # as dq of a token whose only softmax key is itself, rounding noise is not divided by 0
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-3))


CASES = [
    # name, B, T, Hq, Hkv, w, k, dtype, qk_scale
    ("f32-ragged", 1, 200, 2, 1, 64, 8, "f32", 1.0),
    ("f32-gqa2-b2", 2, 150, 4, 2, 64, 4, "f32", None),
    ("bf16-gqa4-ragged", 1, 333, 8, 2, 64, 8, "bf16", 1.0),
    ("bf16-window16", 1, 260, 4, 1, 16, 8, "bf16", 1.0),
    ("bf16-window1", 1, 200, 2, 1, 1, 8, "bf16", None),
    ("f32-window0-k0", 1, 170, 2, 1, 0, 0, "f32", 1.0),
    ("bf16-k64-full-softmax", 1, 200, 4, 1, 64, 64, "bf16", 1.0),
    ("bf16-g6", 1, 150, 6, 1, 64, 8, "bf16", 1.0),
    ("bf16-g3-odd-group", 1, 210, 6, 2, 64, 8, "bf16", 1.0),
    ("bf16-g8-b2", 2, 300, 16, 2, 64, 16, "bf16", 1.0),
    ("bf16-w33-k3", 1, 290, 4, 1, 33, 3, "bf16", 1.0),
    ("bf16-k63", 1, 330, 4, 2, 64, 63, "bf16", 1.0),
    ("f32-k1", 1, 300, 2, 1, 64, 1, "f32", 1.0),
    ("bf16-short", 1, 37, 4, 1, 64, 8, "bf16", 1.0),
    ("f32-one-token", 2, 1, 2, 1, 64, 8, "f32", None),
    ("f32-two-chunks", 1, 128, 2, 1, 64, 16, "f32", 1.0),
    # an even number of compact tiles (padded to an odd tile stride): 8 x 16 rows = 2 tiles,
    # 4 x 64 rows = 4 tiles
    ("f32-even-tiles-k16", 1, 512, 2, 1, 64, 16, "f32", 1.0),
    ("bf16-even-tiles-k64", 1, 256, 4, 1, 64, 64, "bf16", 1.0),
    # large logits: the query kernel's fixed softmax frame is too loose for every wave (4.0)
    # or for the waves past the first planted key (2.0), which take the running reference
    ("f32-large-logits", 1, 300, 2, 1, 64, 8, "f32", 4.0),
    ("bf16-large-logits-gqa4", 1, 333, 8, 2, 64, 8, "bf16", 2.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case):
    name, B, T, Hq, Hkv, w, k, dt, sc = case
    _say(name)
    wl, (q, kk, v, wp) = synth.small_case(seed=zlib.crc32(name.encode()) % 1000, B=B, T=T, Hq=Hq, Hkv=Hkv, D=64,
                                           F=64, window=w, chunk=64, top_k=k, dtype=dt, qk_scale=sc,
                                           n_planted=max(1, T // 50))
    dout = synth.make_grad_out(wl)
    out, idx, grads = _forward_backward(wl, q, kk, v, wp, dout)
    sel = _sel_from_idx(idx.cpu().numpy().astype(np.int64), T)
    ref = O.attend_backward(q, kk, v, wp, w, 64, sel, dout)
    for nm, g, r in zip(("dq", "dk", "dv", "dw"), grads, ref):
        assert np.all(np.isfinite(_np(g))), nm
        e = _rel_err(_np(g), r)
        _say(name, nm, "rel max err", e)
        assert e <= REL_TOL[dt], (nm, e)


CASES_128 = [
    # name, B, T, Hq, Hkv, w, k (bf16, head_dim = feat_dim = 128); even groups take the
    # query kernel's eight-wave form (two heads per workgroup), odd groups its four-wave form
    ("d128-gqa4-ragged", 1, 333, 8, 2, 64, 16),
    ("d128-gqa3-ragged", 1, 270, 6, 2, 64, 8),
    # 2 x 16 KV heads: enough (batch, KV head, element) threads for the one-pass reverse scan
    ("d128-b2-kv16", 2, 150, 32, 16, 64, 8),
    ("d128-b2-window16", 2, 200, 4, 1, 16, 8),
    ("d128-k64", 1, 190, 4, 1, 64, 64),
]


@pytest.mark.parametrize("case", CASES_128, ids=[c[0] for c in CASES_128])
def test_backward_head_dim_128(case):
    name, B, T, Hq, Hkv, w, k = case
    _say(name)
    wl, (q, kk, v, wp) = synth.small_case(seed=zlib.crc32(name.encode()) % 1000, B=B, T=T, Hq=Hq, Hkv=Hkv, D=128,
                                           F=128, window=w, chunk=64, top_k=k, dtype="bf16", qk_scale=1.0,
                                           n_planted=max(1, T // 50))
    dout = synth.make_grad_out(wl)
    out, idx, grads = _forward_backward(wl, q, kk, v, wp, dout)
    sel = _sel_from_idx(idx.cpu().numpy().astype(np.int64), T)
    ref = O.attend_backward(q, kk, v, wp, w, 64, sel, dout)
    for nm, g, r in zip(("dq", "dk", "dv", "dw"), grads, ref):
        assert np.all(np.isfinite(_np(g))), nm
        e = _rel_err(_np(g), r)
        _say(name, nm, "rel max err", e)
        assert e <= REL_TOL["bf16"], (nm, e)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_backward_per_query_head_routing(dt):
    """Per-query-head routing: the gradients of K, V and W_h are the sums over each group of
    the oracle's gradients for the copies repeated per query head."""
    B, T, Hq, Hkv, w, k = 1, 260, 4, 1, 64, 8
    _say("per-query-head backward", dt)
    wl, (q, kk, v, wp) = synth.small_case(seed=23, B=B, T=T, Hq=Hq, Hkv=Hkv, D=64, F=64, window=w, chunk=64,
                                           top_k=k, dtype=dt, qk_scale=1.0, n_planted=5)
    dout = synth.make_grad_out(wl)
    tq, tk, tv, tw, tdo = (_dev(a, dt) for a in (q, kk, v, wp, dout))
    out, idx = still.prefill(tq, tk, tv, tw, window=w, top_k=k, return_routing=True, scope="query_head")
    grads = still.backward(tq, tk, tv, tw, out, tdo, idx, window=w, top_k=k, scope="query_head")
    torch.cuda.synchronize()
    G = Hq // Hkv
    k_e, v_e, w_e = np.repeat(kk, G, axis=2), np.repeat(v, G, axis=2), np.repeat(wp, G, axis=0)
    sel = _sel_from_idx(idx.cpu().numpy().astype(np.int64), T)
    dq_r, dk_e, dv_e, dw_e = O.attend_backward(q, k_e, v_e, w_e, w, 64, sel, dout)
    ref = (dq_r, dk_e.reshape(B, T, Hkv, G, 64).sum(axis=3), dv_e.reshape(B, T, Hkv, G, 64).sum(axis=3),
           dw_e.reshape(Hkv, G, 64, 64).sum(axis=1))
    for nm, g, r in zip(("dq", "dk", "dv", "dw"), grads, ref):
        e = _rel_err(_np(g), r)
        _say("per-query-head", dt, nm, "rel max err", e)
        assert e <= REL_TOL[dt], (nm, e)


def test_backward_is_deterministic():
    wl, (q, kk, v, wp) = synth.small_case(seed=5, B=1, T=300, Hq=8, Hkv=2, D=64, F=64, window=64, chunk=64,
                                           top_k=8, dtype="bf16", qk_scale=1.0, n_planted=6)
    dout = synth.make_grad_out(wl)
    _say("deterministic")
    _, _, g1 = _forward_backward(wl, q, kk, v, wp, dout)
    _, _, g2 = _forward_backward(wl, q, kk, v, wp, dout)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def _sparse_grad_out(wl, positions):
    """The workload's dout, zero except at the given positions (all batches and heads)."""
    dout = synth.make_grad_out(wl)
    keep = np.zeros(wl.seq_len, dtype=bool)
    keep[positions] = True
    dout[:, ~keep] = 0.0
    return dout


SPARSE = [
    # id, workload, seq_len override, batches compared against the oracle
    ("l1b-16k", "L1B_16K", None, (0,)),
    ("l1b-64k", "L1B_16K", 65536, (0,)),
    ("l8b-b8-4k", "L8B_4K", None, (0, 7)),
]


@pytest.mark.parametrize("stress", [False, True], ids=["bench-draw", "stress"])
@pytest.mark.parametrize("case", SPARSE, ids=[c[0] for c in SPARSE])
def test_backward_full_size_sparse_rows(case, stress):
    """Full-size layers (the 16K Llama-3.2-1B shape, the same shape at 65536 tokens, and the
    8 x 4096 Llama-3.1-8B shape at head_dim 128) with dout zero except on about 70 query
    positions spread over the sequence: the loss is then those rows alone, so the oracle's
    gradients for them (attend_backward with rows=) are the whole gradients, and dq, dk and
    dv are compared at every position (dW too), within the relative bar. The value-gradient
    identity (sum over positions of dv = sum of the group's dout) is checked on every batch."""
    cid, wname, T_over, batches = case
    wl = getattr(synth, wname)
    if T_over is not None:
        wl = wl.replace(seq_len=T_over)
    if stress:
        wl = wl.replace(qk_scale=1.0)
    name = f"backward-{cid}-{'stress' if stress else 'bench'}"
    _say(name, wl.name)
    q, k, v, wp = synth.make_inputs(wl)
    B, T, G = wl.batch, wl.seq_len, wl.n_q_heads // wl.n_kv_heads
    positions = np.array(sorted({i for (_, _, i) in PC.sample_rows(np.random.default_rng(T + 3), 1, T, 1, 64)}))
    dout = _sparse_grad_out(wl, positions)
    out, idx, (dq, dk, dv, dw) = _forward_backward(wl, q, k, v, wp, dout)
    sel = _sel_from_idx(idx.cpu().numpy().astype(np.int64), T)
    dwn = _np(dw)
    dw_ref = np.zeros_like(dwn)
    for b in batches:
        s_ = slice(b, b + 1)
        ref = O.attend_backward(q[s_], k[s_], v[s_], wp, wl.window, wl.chunk, sel[s_], dout[s_], rows=positions)
        for nm, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
            gn = _np(g[s_])
            assert np.all(np.isfinite(gn)), nm
            e = _rel_err(gn, r)
            rowmax = np.abs(r).reshape(r.shape[0] * r.shape[1], -1).max(axis=1)
            rowerr = np.abs(gn - r).reshape(rowmax.shape[0], -1).max(axis=1)
            floor = 1e-2 * np.abs(r).max()
            big = rowmax > floor
            rr = float((rowerr[big] / rowmax[big]).max(initial=0.0))
            _say(name, "batch", b, nm, "rel max err over every position", e, "worst row err / row size", rr,
                 "rows above 1% of the max", int(big.sum()))
            assert e <= REL_TOL["bf16"], (nm, e)
            # dv_j sums P_ij dout_i with P >= 0, so each sizeable row holds to its own size too
            # (dq and dk rows add terms of both signs: their rounding follows the terms)
            if nm == "dv":
                assert rr <= 2e-2, ("dv row", rr)
        dw_ref += ref[3]
    if len(batches) == B:
        e = _rel_err(dwn, dw_ref)
        _say(name, "dw rel max err", e)
        assert e <= REL_TOL["bf16"], ("dw", e)
    assert np.all(np.isfinite(_np(dq))) and np.all(np.isfinite(_np(dk))) and np.all(np.isfinite(dwn))
    want = dout.astype(np.float64).reshape(B, T, wl.n_kv_heads, G, wl.head_dim).sum(axis=(1, 3))
    e = float(np.abs(_np(dv).sum(axis=1) - want).max() / np.abs(want).max())
    _say(name, "sum of dv rel err", e)
    assert e <= 1e-2
