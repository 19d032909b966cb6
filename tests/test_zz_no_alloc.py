"""still_decode_step_noalloc (the decode step that allocates nothing, its split partials in the
library's own device scratch) against still_decode_step, through the C ABI: two calls in a
row, the second with a smaller input, each bit-identical to the step that takes a workspace
and within the bf16 bar of it."""

import ctypes
import sys

import numpy as np
import pytest
import torch

from linear_attention_saliency_amd import still, synth

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda", torch.bfloat16).contiguous()


def _pair(B, T0, Hq, Hkv, D, k, seed):
    """Two caches holding the same prefix (prefill of T0 tokens), the next token's q, k, v."""
    wl, (q, kk, v, wp) = synth.small_case(seed=seed, B=B, T=T0 + 1, Hq=Hq, Hkv=Hkv, D=D, F=D, window=64,
                                           chunk=64, top_k=k, dtype="bf16", qk_scale=1.0, n_planted=4)
    tq, tk, tv, tw = (_dev(a) for a in (q, kk, v, wp))
    caches = []
    for _ in range(2):
        c = still.DecodeCache(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, feat_dim=D, window=64, top_k=k,
                              max_tokens=T0 + 8, dtype=torch.bfloat16)
        still.prefill(tq[:, :T0].contiguous(), tk[:, :T0].contiguous(), tv[:, :T0].contiguous(), tw, window=64,
                      top_k=k, cache=c)
        caches.append(c)
    new = (tq[:, T0].contiguous(), tk[:, T0].contiguous(), tv[:, T0].contiguous())
    return caches, new, tw


def test_noalloc_decode_matches_workspace_decode():
    lib = still.load()
    # first call: 4 sequences at 1000 cached tokens (GQA 4, head_dim 128, 15 chunks of compact
    # rows over many splits); second call: a smaller step (2 sequences, head_dim 64, 300 tokens)
    for (B, T0, Hq, Hkv, D, k, seed) in ((4, 1000, 8, 2, 128, 16, 1), (2, 300, 4, 1, 64, 8, 2)):
        _say("noalloc", B, T0, Hq, Hkv, D, k)
        (ca, cb), (q, kk, v), w = _pair(B, T0, Hq, Hkv, D, k, seed)
        out_ws = ca.step(q, kk, v, w)
        out_na = torch.empty_like(q)
        cb.step_noalloc(q, kk, v, w, out_na)
        torch.cuda.synchronize()
        assert cb.n_tokens == ca.n_tokens == T0 + 1
        err = float((out_na.float() - out_ws.float()).abs().max())
        _say("noalloc max abs diff", err)
        assert err <= 2e-2
        assert torch.equal(out_na, out_ws)
        # the caches advanced alike (the step also folds nothing here: T0 + 1 is inside a chunk)
        for key in ("ring_k", "ring_v", "cur_saliency"):
            assert torch.equal(ca.tensors()[key], cb.tensors()[key]), key
    assert lib.still_last_hip_error() == 0


def test_noalloc_rejects_steps_beyond_its_scratch():
    """A step whose partials would not fit the library's scratch is refused before launch."""
    lib = still.load()
    cfg = still.make_config(2048, 0, 64, 16, 128, 128, 64, 64, 16, "bf16")
    c = still.Cache()
    c.cfg = cfg
    c.max_tokens = 1 << 20
    c.n_tokens = 1 << 19  # many compact tiles: one split per (b, KV head), 2048 * 16 * 4 records
    c.sel_capacity = 64
    p = ctypes.c_void_p(1 << 20)
    rc = lib.still_decode_step_noalloc(ctypes.byref(cfg), ctypes.byref(c), p, p, p, p, p, None)
    assert rc == -3
    assert c.n_tokens == 1 << 19
