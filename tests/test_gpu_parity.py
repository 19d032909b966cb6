"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bars: routing indices bit-exact in every chunk whose oracle saliency margin exceeds 1e-3
(other chunks are counted as flips, and only then may outputs be compared under the
oracle's routing); outputs within max-abs 1e-4 (fp32) and 2e-2 (bf16).
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

TOL = {"f32": 1e-4, "bf16": 2e-2}
MARGIN = 1e-3


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32).contiguous()


def _run(q, k, v, w, wl, routing=None, score="saliency"):
    dt = wl.dtype
    tq, tk, tv, tw = (_dev(a, dt) for a in (q, k, v, w))
    r = None if routing is None else torch.from_numpy(routing.astype(np.int32)).cuda()
    if wl.window >= 1:
        out, sal, sel = still.prefill(tq, tk, tv, tw, window=wl.window, top_k=wl.top_k, routing=r,
                                      return_saliency=True, return_routing=True, score=score)
    else:
        out, sel = still.prefill(tq, tk, tv, tw, window=wl.window, top_k=wl.top_k, routing=r, return_routing=True)
        sal = None
    torch.cuda.synchronize()
    return (out.float().cpu().numpy().astype(np.float64),
            None if sal is None else sal.cpu().numpy().astype(np.float64),
            sel.cpu().numpy().astype(np.int64))


def _sel_from_idx(idx, T):
    B, H, nc, k = idx.shape
    sel = np.zeros((B, H, T), dtype=bool)
    for b in range(B):
        for h in range(H):
            sel[b, h, idx[b, h].reshape(-1)] = True
    return sel


def _check_routing(s_gpu, sel_gpu, s_ref, wl):
    """Saliency close; routing bit-exact wherever the oracle's margin is above 1e-3."""
    fin = np.isfinite(s_ref)
    assert np.array_equal(np.isfinite(s_gpu), fin)
    err = np.abs(s_gpu[fin] - s_ref[fin])
    assert np.all(err <= 1e-4 * (1.0 + np.abs(s_ref[fin]))), float(err.max())
    if wl.top_k == 0:
        return 0, 0
    ref_idx, _ = O.route(s_ref, wl.chunk, wl.top_k)
    margins = O.route_margins(s_ref, wl.chunk, wl.top_k)
    same = np.all(sel_gpu == ref_idx, axis=-1)
    decided = margins > MARGIN
    assert np.all(same[decided]), f"routing differs in {int((~same[decided]).sum())} decided chunks"
    return int(decided.sum()), int((~same).sum())


CASES = [
    # name, B, T, Hq, Hkv, D, F, w, k, dtype, qk_scale
    ("tiny-f32-ragged", 1, 300, 1, 1, 64, 64, 64, 8, "f32", None),
    ("f32-stress", 2, 200, 2, 1, 64, 64, 64, 8, "f32", 1.0),
    ("bf16-gqa4", 1, 333, 8, 2, 64, 64, 64, 8, "bf16", None),
    ("bf16-stress-gqa4", 1, 256, 4, 1, 64, 64, 64, 8, "bf16", 1.0),
    ("bf16-d128", 2, 200, 8, 2, 128, 128, 64, 16, "bf16", 1.0),
    ("bf16-d64-f128", 1, 190, 4, 1, 64, 128, 64, 4, "bf16", 1.0),
    ("bf16-d128-f64", 1, 130, 4, 2, 128, 64, 64, 16, "bf16", None),
    ("bf16-window16", 1, 260, 4, 1, 64, 64, 16, 8, "bf16", 1.0),
    ("bf16-window1", 1, 200, 2, 1, 64, 64, 1, 8, "bf16", None),
    ("bf16-g6-split", 1, 150, 6, 1, 64, 64, 64, 8, "bf16", 1.0),
    ("bf16-short", 1, 37, 4, 1, 64, 64, 64, 8, "bf16", 1.0),
    ("bf16-one-token", 2, 1, 4, 2, 64, 64, 64, 8, "bf16", None),
    ("f32-window-only-k0", 1, 200, 1, 1, 64, 64, 64, 0, "f32", 1.0),
    ("bf16-full-softmax", 1, 256, 4, 1, 64, 64, 64, 64, "bf16", 1.0),
    # top-k values whose compact rows straddle the 64-row tiles at odd offsets, an odd window
    ("bf16-k1", 1, 300, 4, 1, 64, 64, 64, 1, "bf16", 1.0),
    ("bf16-d128-k63", 1, 330, 4, 2, 128, 128, 64, 63, "bf16", 1.0),
    ("bf16-w33-k3", 2, 290, 4, 1, 64, 64, 33, 3, "bf16", 1.0),
    # fp32 at head_dim / feat_dim 128 (the sequential LDS plan of the attention kernel)
    ("f32-d128", 2, 200, 8, 2, 128, 128, 64, 16, "f32", 1.0),
    ("f32-d128-f64-w16", 1, 330, 4, 1, 128, 64, 16, 8, "f32", 1.0),
    ("f32-d64-f128", 1, 290, 4, 1, 64, 128, 64, 4, "f32", 1.0),
    ("f32-d128-k63", 1, 260, 2, 1, 128, 128, 64, 63, "f32", 1.0),
    # windows longer than a chunk (two band chunks), each dtype and head / feature width,
    # several compact tiles
    ("bf16-w65", 1, 300, 4, 1, 64, 64, 65, 8, "bf16", 1.0),
    ("f32-w66-f128", 1, 260, 4, 1, 64, 128, 66, 8, "f32", 1.0),
    ("f32-w96", 1, 420, 2, 1, 64, 64, 96, 8, "f32", 1.0),
    ("bf16-w96-gqa4", 1, 600, 8, 2, 64, 64, 96, 8, "bf16", 1.0),
    ("bf16-w96-many-tiles", 1, 1300, 4, 1, 64, 64, 96, 16, "bf16", 1.0),
    ("f32-w128-d128", 1, 390, 4, 1, 128, 128, 128, 16, "f32", 1.0),
    ("bf16-w128-d128", 2, 333, 8, 2, 128, 128, 128, 16, "bf16", 1.0),
    ("bf16-w127-f128-k3", 1, 450, 4, 1, 64, 128, 127, 3, "bf16", 1.0),
    ("f32-w100-d128-f64", 1, 300, 2, 1, 128, 64, 100, 8, "f32", None),
    # logits of hundreds of log2 units (|q|, |k| ~ 32, planted keys ~ 128): the key-norm
    # bound of the compact logits is far above every score of the window, so the attention
    # kernel takes the exact largest compact logit in a pre-pass before the compact tiles
    ("f32-huge-logits", 1, 400, 4, 1, 64, 64, 64, 8, "f32", 4.0),
    ("bf16-huge-logits-gqa4", 1, 700, 8, 2, 64, 64, 64, 8, "bf16", 4.0),
    ("bf16-huge-logits-d128", 1, 500, 4, 1, 128, 128, 64, 16, "bf16", 4.0),
    ("f32-huge-logits-d128-w96", 1, 450, 2, 1, 128, 128, 96, 16, "f32", 4.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_matches_oracle(case):
    name, B, T, Hq, Hkv, D, F, w, k, dt, sc = case
    _say(name)
    wl, (q, kk, v, wp) = synth.small_case(seed=zlib.crc32(name.encode()) % 1000, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, F=F,
                                           window=w, chunk=64, top_k=k, dtype=dt, qk_scale=sc,
                                           n_planted=max(1, T // 50))
    out, s_gpu, idx_gpu = _run(q, kk, v, wp, wl)
    if w >= 1:
        s_ref, _ = O.saliency(q, kk, w)
        decided, flips = _check_routing(s_gpu, idx_gpu, s_ref, wl)
        _say(name, "decided chunks", decided, "flips", flips)
        sel_gpu = _sel_from_idx(idx_gpu, T)
    else:
        sel_gpu = np.zeros((B, Hkv, T), dtype=bool)
    # outputs under the routing the device chose (equal to the oracle's where decided)
    ref = O.attend(q, kk, v, wp, w, 64, k, sel=sel_gpu)
    err = np.abs(out - ref).max()
    _say(name, "max abs err", err)
    assert err <= TOL[dt], err
    # with the oracle's own routing fed in, the outputs must match too
    if k > 0 and T >= 64:
        ref_idx = O.route(s_ref, 64, k)[0]
        out2, _, idx2 = _run(q, kk, v, wp, wl, routing=ref_idx)
        assert np.array_equal(idx2, ref_idx)
        ref2 = O.attend(q, kk, v, wp, w, 64, k, sel=_sel_from_idx(ref_idx, T))
        assert np.abs(out2 - ref2).max() <= TOL[dt]


def test_pure_linear_attention():
    """window 0, top_k 0: the layer is causal NP-Map linear attention."""
    _say("pure-LA")
    wl, (q, k, v, wp) = synth.small_case(seed=3, B=2, T=210, Hq=4, Hkv=2, D=64, F=64, window=0, chunk=64,
                                         top_k=0, dtype="bf16")
    out, _, _ = _run(q, k, v, wp, wl)
    ref = O.attend(q, k, v, wp, 0, 64, 0)
    assert np.abs(out - ref).max() <= TOL["bf16"]
    wl32, (q, k, v, wp) = synth.small_case(seed=4, B=1, T=150, Hq=2, Hkv=1, D=64, F=64, window=0, chunk=64,
                                           top_k=0, dtype="f32")
    out, _, _ = _run(q, k, v, wp, wl32)
    ref = O.attend(q, k, v, wp, 0, 64, 0)
    assert np.abs(out - ref).max() <= TOL["f32"]


def test_full_softmax_special_case():
    """window = top_k = chunk: every earlier token is selected, so the layer is causal softmax."""
    _say("full-softmax-sdpa")
    wl, (q, k, v, wp) = synth.small_case(seed=5, B=1, T=192, Hq=4, Hkv=1, D=64, F=64, window=64, chunk=64,
                                         top_k=64, dtype="f32", qk_scale=1.0)
    out, _, _ = _run(q, k, v, wp, wl)
    G = 4
    tq = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)
    tk = torch.from_numpy(np.repeat(k, G, axis=2).astype(np.float64)).permute(0, 2, 1, 3)
    tv = torch.from_numpy(np.repeat(v, G, axis=2).astype(np.float64)).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True).permute(0, 2, 1, 3).numpy()
    assert np.abs(out - ref).max() <= TOL["f32"]


def test_topk_alone_is_bit_exact():
    """The device top-k on the oracle's saliency (as fp32) equals the oracle's top-k on the
    same fp32 values, ties and infinities included."""
    _say("topk-alone")
    rng = np.random.default_rng(9)
    B, H, T = 2, 3, 64 * 7 + 5
    s = rng.integers(0, 5, size=(B, H, T)).astype(np.float32) * np.float32(0.25)
    s[0, 0, :64] = np.inf
    s[1, 2, 70:75] = np.inf
    s += (rng.random((B, H, T)) < 0.5).astype(np.float32) * rng.random((B, H, T)).astype(np.float32)
    for k in (1, 5, 8, 16, 63, 64):
        got = still.select_topk(torch.from_numpy(s).cuda(), chunk=64, top_k=k).cpu().numpy()
        want = O.route(s.astype(np.float64), 64, k)[0]
        assert np.array_equal(got, want), k


@pytest.mark.parametrize("dt,D,F", [("f32", 64, 64), ("bf16", 64, 64), ("bf16", 128, 128), ("bf16", 64, 128),
                                    ("bf16", 128, 64), ("f32", 128, 128)])
def test_feature_map_matches_oracle(dt, D, F):
    _say("np-map", dt, D, F)
    wl, (q, k, v, wp) = synth.small_case(seed=D + F, B=2, T=100, Hq=2, Hkv=2, D=D, F=F, window=64, chunk=64,
                                         top_k=0, dtype=dt, qk_scale=1.0, n_planted=3)
    k[0, 5, 1] = 0.0  # phi(0) = 0
    phi = still.feature_map(_dev(k, dt), _dev(wp, dt)).cpu().numpy().astype(np.float64)
    ref = np.stack([O.np_map(k[:, :, h], wp[h]) for h in range(2)], axis=2)
    assert np.all(phi[0, 5, 1] == 0.0)
    rel = np.abs(phi - ref).max() / np.abs(ref).max()
    assert rel < 1e-5, rel
    np.testing.assert_allclose(np.linalg.norm(phi, axis=-1), np.linalg.norm(k, axis=-1), rtol=1e-5, atol=1e-6)


def test_run_twice_bitwise():
    """Two identical calls give identical bits (no unsynchronised LDS reuse)."""
    _say("determinism")
    wl, arrs = synth.small_case(seed=21, B=1, T=640, Hq=8, Hkv=2, D=64, F=64, window=64, chunk=64, top_k=8,
                                dtype="bf16", qk_scale=1.0)
    a = _run(*arrs, wl)
    b = _run(*arrs, wl)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("dt,D,F,G", [("f32", 64, 64, 1), ("bf16", 64, 64, 4), ("bf16", 128, 128, 4)])
def test_diagonal_score_routing(dt, D, F, G):
    """Routing by the diagonal logit alone: the device's scores against the oracle's, the
    selection of every decided chunk, and the output under the device's routing."""
    _say("diag-score", dt, D, F, G)
    wl, (q, kk, v, wp) = synth.small_case(seed=91 + D + G, B=1, T=330, Hq=G, Hkv=1, D=D, F=F, window=64,
                                           chunk=64, top_k=8, dtype=dt, qk_scale=1.0, n_planted=6)
    out, s_gpu, idx_gpu = _run(q, kk, v, wp, wl, score="diag")
    s_ref, _ = O.diagonal_score(q, kk)
    decided, flips = _check_routing(s_gpu, idx_gpu, s_ref, wl)
    _say("diag-score decided", decided, "flips", flips)
    ref = O.attend(q, kk, v, wp, wl.window, wl.chunk, wl.top_k, sel=_sel_from_idx(idx_gpu, wl.seq_len))
    err = np.abs(out - ref).max()
    _say("diag-score max abs err", err)
    assert decided > 0 and err <= TOL[dt]


@pytest.mark.parametrize("dt,D,F,Hq,Hkv,T,w", [("f32", 64, 64, 2, 1, 300, 64), ("bf16", 64, 64, 8, 2, 300, 64),
                                               ("bf16", 128, 128, 4, 1, 300, 64), ("bf16", 64, 64, 4, 1, 1100, 64),
                                               ("f32", 64, 128, 4, 2, 420, 96), ("bf16", 128, 64, 6, 2, 333, 33)])
def test_per_query_head_routing(dt, D, F, Hq, Hkv, T, w):
    """Each query head selects on its own saliency: the score and routing per query head
    against the oracle on K, V and W_h repeated per query head (the same layer with
    n_kv_heads = n_q_heads), and the output under the device's routing."""
    _say("per-query-head", dt, D, F, Hq, Hkv, T, w)
    wl, (q, kk, v, wp) = synth.small_case(seed=17 + D + Hq + T, B=1, T=T, Hq=Hq, Hkv=Hkv, D=D, F=F, window=w,
                                           chunk=64, top_k=8, dtype=dt, qk_scale=1.0, n_planted=6)
    G = Hq // Hkv
    tq, tk, tv, tw = (_dev(a, dt) for a in (q, kk, v, wp))
    out, sal, idx = still.prefill(tq, tk, tv, tw, window=w, top_k=8, return_saliency=True, return_routing=True,
                                  scope="query_head")
    torch.cuda.synchronize()
    assert tuple(sal.shape) == (1, Hq, T) and tuple(idx.shape) == (1, Hq, T // 64, 8)
    k_e, v_e, w_e = np.repeat(kk, G, axis=2), np.repeat(v, G, axis=2), np.repeat(wp, G, axis=0)
    wl_e = wl.replace(n_kv_heads=Hq)
    s_ref, _ = O.saliency(q, k_e, w)
    idx_np = idx.cpu().numpy().astype(np.int64)
    decided, flips = _check_routing(sal.cpu().numpy().astype(np.float64), idx_np, s_ref, wl_e)
    ref = O.attend(q, k_e, v_e, w_e, w, 64, 8, sel=_sel_from_idx(idx_np, T))
    err = np.abs(out.float().cpu().numpy().astype(np.float64) - ref).max()
    _say("per-query-head decided", decided, "flips", flips, "max abs err", err)
    assert decided > 0 and err <= TOL[dt]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_softmax_scores_far_below_linear_weights(dt):
    """Every query points away from every key, so all softmax scores sit tens of log2 units
    below 0 while the NP-Map weights phi(q).phi(k) stay near |q||k|: the linear part dominates
    the shared normaliser and the running frame must follow it (the oracle has no frame)."""
    _say("far-scores", dt)
    wl, (q, k, v, wp) = synth.small_case(seed=77, B=1, T=200, Hq=2, Hkv=1, D=64, F=64, window=64, chunk=64,
                                         top_k=8, dtype=dt, qk_scale=1.0)
    rng = np.random.default_rng(78)
    k0 = rng.standard_normal(64).astype(np.float32)
    k0 *= np.float32(8.0 / np.linalg.norm(k0))
    k = np.broadcast_to(k0, k.shape).astype(np.float32) + np.float32(0.01) * rng.standard_normal(k.shape).astype(np.float32)
    q = (-4.0 * np.broadcast_to(k0, q.shape)).astype(np.float32)
    if dt == "bf16":
        q, k = synth.round_bf16(q), synth.round_bf16(k)
    out, s_gpu, idx_gpu = _run(q, k, v, wp, wl)
    ref = O.attend(q, k, v, wp, 64, 64, 8, sel=_sel_from_idx(idx_gpu, wl.seq_len))
    err = np.abs(out - ref).max()
    _say("far-scores", dt, "max abs err", err)
    assert np.all(np.isfinite(out))
    assert err <= TOL[dt], err


@pytest.mark.parametrize("stress", [False, True], ids=["as-specified", "stress"])
def test_tiny_f32_workload(stress):
    """The tiny fp32 workload as specified (batch 1, 512 tokens, one head, head_dim 64, w = C
    = 64, top_k 8, d_f 64, 16 planted keys x4, seed 0) and its routing-stress twin: saliency
    and routing over every chunk, and every output element against the chunked oracle at
    1e-4 and at 1e-3 of its row's largest entry."""
    wl = synth.TINY_F32.replace(qk_scale=1.0) if stress else synth.TINY_F32
    _say("tiny-f32", wl.name, "stress" if stress else "")
    q, k, v, wp = synth.make_inputs(wl)
    out, s_gpu, idx_gpu = _run(q, k, v, wp, wl)
    s_ref, _ = O.saliency(q, k, wl.window)
    decided, flips = _check_routing(s_gpu, idx_gpu, s_ref, wl)
    _say("tiny-f32 decided chunks", decided, "of", wl.seq_len // 64, "flips", flips)
    ref = O.attend(q, k, v, wp, wl.window, wl.chunk, wl.top_k, sel=_sel_from_idx(idx_gpu, wl.seq_len))
    ok, ea, er, nbad = PC.check_rows(out.reshape(-1, wl.head_dim), ref.reshape(-1, wl.head_dim), "f32")
    _say("tiny-f32 worst abs err", ea, "worst err / row size", er)
    assert ok, (ea, er, nbad)


@pytest.mark.parametrize("T,D,k", [(4352, 64, 8), (16448, 64, 8), (4352, 128, 16)])
def test_f32_many_compact_tiles(T, D, k):
    """fp32 at the reference precision with many compact tiles (GQA 4, stress draw):
    T = 4352 (68 chunks: the 16-chunk scan segment; 9 compact tiles for the last chunk at
    top_k 8, 17 at head_dim 128 and top_k 16), every output against the chunked oracle;
    T = 16448 (257 chunks: a second scan round, 32 compact tiles), about 70 sampled rows
    against the per-query oracle. Routing bit-exact on every decided chunk; outputs within
    1e-4 and 1e-3 of each row's size."""
    topk = k
    wl, (q, k, v, wp) = synth.small_case(seed=T % 997 + D, B=1, T=T, Hq=8, Hkv=2, D=D, F=D, window=64, chunk=64,
                                         top_k=topk, dtype="f32", qk_scale=1.0, n_planted=T // 100)
    _say("f32-many-tiles", T, D, topk)
    out, s_gpu, idx_gpu = _run(q, k, v, wp, wl)
    s_ref, _ = O.saliency(q, k, wl.window)
    decided, flips = _check_routing(s_gpu, idx_gpu, s_ref, wl)
    _say("f32-many-tiles", T, "decided chunks", decided, "flips", flips)
    assert decided >= s_ref.shape[1] * (T // 64) // 2
    sel = _sel_from_idx(idx_gpu, T)
    if T <= 4352:
        ref = O.attend(q, k, v, wp, 64, 64, topk, sel=sel)
        got, ref = out.reshape(-1, D), ref.reshape(-1, D)
    else:
        rows = PC.sample_rows(np.random.default_rng(T), 1, T, 8, 64)
        ref = O.brute_rows(q, k, v, wp, 64, 64, sel, rows)
        got = np.stack([out[b, i, hq] for (b, hq, i) in rows])
    ok, ea, er, nbad = PC.check_rows(got, ref, "f32")
    _say("f32-many-tiles", T, "worst abs err", ea, "worst err / row size", er)
    assert ok, (ea, er, nbad)
