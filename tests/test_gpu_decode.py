"""Parity of the decode step (through the C ABI) with the prefill and with the fp64 oracle.

* prefill(T0) into a cache, then one decode step per token up to T: the saliency of every
  decoded token and every chunk selection are bit-identical to those of a prefill of T
  tokens (the same device routine computes them); the decoded outputs match the oracle
  under that routing (max-abs 1e-4 fp32, 2e-2 bf16); the cache afterwards holds what a
  prefill of T tokens leaves in it.
* decoding from an empty cache: saliency against the oracle, routing bit-exact where the
  oracle's margin exceeds 1e-3, outputs against the oracle under the device's routing.
"""

import sys
import zlib

import numpy as np
import pytest
import torch

from linear_attention_saliency_amd import still, synth
from oracle import still_oracle as O

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
STATE_TOL = {"f32": 1e-4, "bf16": 2e-2}  # relative to the largest state entry
MARGIN = 1e-3


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32).contiguous()


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _mask_bits(m):
    """int64 tensor of 64-bit masks -> bool [..., 64]."""
    u = m.cpu().numpy().astype(np.int64).view(np.uint64)
    return ((u[..., None] >> np.arange(64, dtype=np.uint64)) & np.uint64(1)).astype(bool)


def _new_cache(wl, max_tokens, score="saliency", scope="kv_head"):
    return still.DecodeCache(batch=wl.batch, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                             head_dim=wl.head_dim, feat_dim=wl.feat_dim, window=wl.window, top_k=wl.top_k,
                             max_tokens=max_tokens,
                             dtype=torch.bfloat16 if wl.dtype == "bf16" else torch.float32, score=score,
                             scope=scope)


def _decode_steps(cache, tq, tk, tv, tw, t0, t1):
    """Decode tokens t0..t1-1. Returns outputs [B, t1-t0, Hq, D] (float64), the saliency of
    each decoded token [B, Hkv, t1-t0] and the selection of every chunk completed on the way
    {chunk: bool [B, Hkv, 64]}."""
    outs, sals, masks = [], [], {}
    for t in range(t0, t1):
        o = cache.step(tq[:, t].contiguous(), tk[:, t].contiguous(), tv[:, t].contiguous(), tw)
        outs.append(o)
        st = cache.tensors()
        sals.append(st["cur_saliency"][:, :, t % 64].clone())
        if t % 64 == 63:
            masks[t // 64] = _mask_bits(st["sel_mask"][:, :, (t // 64) % st["sel_mask"].shape[2]])
    torch.cuda.synchronize()
    out = np.stack([_np(o) for o in outs], axis=1)
    sal = np.stack([s.cpu().numpy() for s in sals], axis=-1)
    return out, sal, masks


PREFILL_THEN_DECODE = [
    # name, B, T0, T, Hq, Hkv, D, F, w, k, dtype, qk_scale
    ("f32-gqa2-mid-chunk", 2, 100, 260, 4, 2, 64, 64, 64, 8, "f32", 1.0),
    ("bf16-d128-at-boundary", 2, 128, 268, 8, 2, 128, 128, 64, 16, "bf16", 1.0),
    ("bf16-window16", 1, 70, 200, 4, 1, 64, 64, 16, 8, "bf16", 1.0),
    ("bf16-window0-k0", 1, 50, 150, 4, 1, 64, 64, 0, 0, "bf16", None),
    ("bf16-g6", 1, 64, 200, 6, 1, 64, 64, 64, 8, "bf16", 1.0),
    ("bf16-d64-f128-from-1", 2, 1, 141, 4, 2, 64, 128, 64, 4, "bf16", None),
    ("bf16-d128-f64-k64", 1, 190, 330, 4, 1, 128, 64, 64, 64, "bf16", 1.0),
    ("bf16-w33-k3", 1, 100, 300, 4, 1, 64, 64, 33, 3, "bf16", 1.0),
    ("bf16-d128-k63", 1, 120, 280, 4, 2, 128, 128, 64, 63, "bf16", 1.0),
    ("f32-d128-at-boundary", 2, 128, 268, 8, 2, 128, 128, 64, 16, "f32", 1.0),
    ("f32-d128-f64-w16", 1, 70, 200, 4, 1, 128, 64, 16, 8, "f32", 1.0),
    # routed by the diagonal logit instead of the Self-Saliency Score
    ("bf16-diag-score", 2, 100, 270, 4, 1, 64, 64, 64, 8, "bf16", 1.0, "diag"),
    ("bf16-d128-diag-score", 1, 64, 200, 4, 2, 128, 128, 64, 16, "bf16", None, "diag"),
    # windows longer than a chunk: a ring of three chunks, chunk c-2 folded at completion
    ("f32-w96-mid-chunk", 1, 150, 400, 4, 1, 64, 64, 96, 8, "f32", 1.0),
    ("bf16-w128-d128-at-boundary", 2, 192, 330, 8, 2, 128, 128, 128, 16, "bf16", 1.0),
    ("f32-w127-d128-f128", 1, 70, 300, 2, 1, 128, 128, 127, 8, "f32", 1.0),
    ("bf16-w65", 1, 100, 260, 4, 1, 64, 64, 65, 8, "bf16", 1.0),
    # each query head selects for itself: per-query-head rings, compact rows and states over
    # shared K and V (the oracle runs on K, V and W_h repeated per query head)
    ("bf16-query-head-gqa4", 1, 100, 300, 8, 2, 64, 64, 64, 8, "bf16", 1.0, "saliency", "query_head"),
    ("f32-query-head-w96-d128", 1, 130, 330, 4, 1, 128, 128, 96, 16, "f32", 1.0, "saliency", "query_head"),
    ("bf16-query-head-diag", 2, 64, 200, 4, 2, 128, 64, 64, 8, "bf16", None, "diag", "query_head"),
]


@pytest.mark.parametrize("case", PREFILL_THEN_DECODE, ids=[c[0] for c in PREFILL_THEN_DECODE])
def test_prefill_then_decode_equals_prefill(case):
    name, B, T0, T, Hq, Hkv, D, F, w, k, dt, sc, *rest = case
    score = rest[0] if rest else "saliency"
    scope = rest[1] if len(rest) > 1 else "kv_head"
    Hr = Hq if scope == "query_head" else Hkv  # heads that select
    _say(name)
    wl, (q, kk, v, wp) = synth.small_case(seed=zlib.crc32(name.encode()) % 1000, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D,
                                           F=F, window=w, chunk=64, top_k=k, dtype=dt, qk_scale=sc,
                                           n_planted=max(1, T // 50))
    tq, tk, tv, tw = (_dev(a, dt) for a in (q, kk, v, wp))

    # reference: one prefill of all T tokens, into a cache as well
    full_cache = _new_cache(wl, T + 16, score, scope)
    if w >= 1:
        out_full, sal_full, idx_full = still.prefill(tq, tk, tv, tw, window=w, top_k=k, return_saliency=True,
                                                     return_routing=True, cache=full_cache, score=score, scope=scope)
    else:
        out_full, idx_full = still.prefill(tq, tk, tv, tw, window=w, top_k=k, return_routing=True,
                                           cache=full_cache, scope=scope)
        sal_full = None

    cache = _new_cache(wl, T + 16, score, scope)
    still.prefill(tq[:, :T0].contiguous(), tk[:, :T0].contiguous(), tv[:, :T0].contiguous(), tw, window=w,
                  top_k=k, cache=cache, score=score, scope=scope)
    out_dec, sal_dec, masks = _decode_steps(cache, tq, tk, tv, tw, T0, T)
    assert cache.n_tokens == T

    # routing: bit-identical saliency and selections
    if w >= 1:
        s_full = sal_full.cpu().numpy()
        assert np.array_equal(sal_dec.view(np.uint32), s_full[:, :, T0:T].view(np.uint32)), "saliency bits differ"
    idx = idx_full.cpu().numpy()
    for c, m in masks.items():
        ref = np.zeros((B, Hr, 64), dtype=bool)
        for b in range(B):
            for h in range(Hr):
                ref[b, h, idx[b, h, c] - 64 * c] = k > 0
        assert np.array_equal(m, ref), f"selection of chunk {c} differs"
    _say(name, "chunks completed while decoding", sorted(masks))

    # outputs against the oracle under that routing
    sel = np.zeros((B, Hr, T), dtype=bool)
    for b in range(B):
        for h in range(Hr):
            sel[b, h, idx[b, h].reshape(-1)] = k > 0
    if scope == "query_head":  # the same layer with every query head its own KV head
        G = Hq // Hkv
        kk, v, wp = np.repeat(kk, G, axis=2), np.repeat(v, G, axis=2), np.repeat(wp, G, axis=0)
    ref = O.attend(q, kk, v, wp, w, 64, k, sel=sel)
    err = np.abs(out_dec - ref[:, T0:T]).max()
    err_full = np.abs(_np(out_full) - ref).max()
    _say(name, "decode max abs err", err, "prefill", err_full)
    assert err <= TOL[dt], err
    assert err_full <= TOL[dt], err_full

    # the cache after decoding holds what the prefill of T tokens leaves
    a, bb = cache.tensors(), full_cache.tensors()
    c_next, r_next = T // 64, T % 64
    bl = still.band_chunks(w)
    nr = bl + 1
    nsel = max(0, c_next - bl) * k
    assert torch.equal(a["sel_k"][:, :, :nsel], bb["sel_k"][:, :, :nsel])
    sv_a = a["sel_v"].reshape(B, Hr, -1, D, 64)
    sv_b = bb["sel_v"].reshape(B, Hr, -1, D, 64)
    full_tiles = nsel // 64
    assert torch.equal(sv_a[:, :, :full_tiles], sv_b[:, :, :full_tiles])
    for l in range(1, bl + 1):  # the band chunks c_next - l
        if c_next >= l:
            sp = (c_next - l) % nr
            assert torch.equal(a["ring_k"][:, :, sp], bb["ring_k"][:, :, sp])
            assert torch.equal(a["ring_v"][:, :, sp], bb["ring_v"][:, :, sp])
            assert torch.equal(a["sel_mask"][:, :, sp], bb["sel_mask"][:, :, sp])
    sc_ = c_next % nr
    assert torch.equal(a["ring_k"][:, :, sc_, :r_next], bb["ring_k"][:, :, sc_, :r_next])
    if w >= 1:
        assert torch.equal(a["cur_saliency"][:, :, :r_next], bb["cur_saliency"][:, :, :r_next])
    for key in ("state_s", "state_z"):
        x, y = a[key].double().cpu(), bb[key].double().cpu()
        scale = max(float(y.abs().max()), 1e-30)
        assert float((x - y).abs().max()) <= STATE_TOL[dt] * scale, key


FROM_EMPTY = [
    # name, B, T, Hq, Hkv, D, F, w, k, dtype, qk_scale
    ("f32-from-empty", 2, 200, 2, 1, 64, 64, 64, 8, "f32", 1.0),
    ("bf16-from-empty-gqa4", 1, 210, 8, 2, 128, 128, 64, 16, "bf16", 1.0),
    ("f32-d128-from-empty", 1, 200, 4, 1, 128, 128, 64, 16, "f32", 1.0),
    ("bf16-w100-from-empty", 1, 330, 4, 1, 64, 64, 100, 8, "bf16", 1.0),
    ("f32-w65-from-empty", 1, 270, 2, 1, 64, 64, 65, 8, "f32", 1.0),
]


@pytest.mark.parametrize("case", FROM_EMPTY, ids=[c[0] for c in FROM_EMPTY])
def test_decode_from_empty_matches_oracle(case):
    name, B, T, Hq, Hkv, D, F, w, k, dt, sc = case
    _say(name)
    wl, (q, kk, v, wp) = synth.small_case(seed=zlib.crc32(name.encode()) % 1000, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D,
                                           F=F, window=w, chunk=64, top_k=k, dtype=dt, qk_scale=sc,
                                           n_planted=max(1, T // 50))
    tq, tk, tv, tw = (_dev(a, dt) for a in (q, kk, v, wp))
    cache = _new_cache(wl, T)
    out, sal, masks = _decode_steps(cache, tq, tk, tv, tw, 0, T)
    with pytest.raises(still.StillError) as e:  # the cache is full now
        cache.step(tq[:, 0].contiguous(), tk[:, 0].contiguous(), tv[:, 0].contiguous(), tw)
    assert e.value.code == -4

    s_ref, _ = O.saliency(q, kk, w)
    fin = np.isfinite(s_ref)
    assert np.array_equal(np.isfinite(sal), fin)
    assert np.all(np.abs(sal[fin] - s_ref[fin]) <= 1e-4 * (1 + np.abs(s_ref[fin])))
    nc = T // 64
    idx_ref, _ = O.route(s_ref, 64, k)
    margins = O.route_margins(s_ref, 64, k)
    sel = np.zeros((B, Hkv, T), dtype=bool)
    decided = 0
    for c in range(nc):
        m = masks[c]
        for b in range(B):
            for h in range(Hkv):
                sel[b, h, 64 * c + np.nonzero(m[b, h])[0]] = True
                assert m[b, h].sum() == k
                if margins[b, h, c] > MARGIN:
                    decided += 1
                    assert np.array_equal(np.nonzero(m[b, h])[0] + 64 * c, idx_ref[b, h, c])
    _say(name, "decided chunks", decided, "of", B * Hkv * nc)
    ref = O.attend(q, kk, v, wp, w, 64, k, sel=sel)
    err = np.abs(out - ref).max()
    _say(name, "max abs err", err)
    assert err <= TOL[dt], err


def test_prefill_into_cache_beyond_4gib():
    """A decode cache sized for 2^24 tokens at head_dim 128 and top_k 64 holds 2^18 + 1
    compact tiles per (batch, KV head): 4 GiB + 16 KiB of compact K rows, past a 32-bit byte
    range. A prefill into it reads its compact rows back from the cache, and must give the
    same output bits as the same prefill without a cache; two decode steps then match the
    prefill of the extended sequence within the bf16 bar."""
    name = "cache-beyond-4gib"
    _say(name)
    wl, (q, kk, v, wp) = synth.small_case(seed=404, B=1, T=302, Hq=4, Hkv=1, D=128, F=128, window=64, chunk=64,
                                           top_k=64, dtype="bf16", qk_scale=1.0, n_planted=3)
    tq, tk, tv, tw = (_dev(a, "bf16") for a in (q, kk, v, wp))
    T0 = 300
    cache = _new_cache(wl, 1 << 24)
    assert cache.c.sel_capacity * 128 * 2 > (1 << 32)
    ref_out = still.prefill(tq[:, :T0].contiguous(), tk[:, :T0].contiguous(), tv[:, :T0].contiguous(), tw,
                            window=64, top_k=64)
    out = still.prefill(tq[:, :T0].contiguous(), tk[:, :T0].contiguous(), tv[:, :T0].contiguous(), tw, window=64,
                        top_k=64, cache=cache)
    dec, _, _ = _decode_steps(cache, tq, tk, tv, tw, T0, 302)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    full = _np(still.prefill(tq, tk, tv, tw, window=64, top_k=64))
    err = float(np.abs(dec - full[:, T0:]).max())
    _say(name, "decode against prefill max abs err", err)
    assert err <= TOL["bf16"], err
    del cache
    torch.cuda.empty_cache()
