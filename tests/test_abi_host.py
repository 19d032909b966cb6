"""Host-side checks of the C ABI: the library loads, exports every declared entry point,
and rejects bad arguments before enqueuing any GPU work (no GPU needed)."""

import ctypes
import os
import re

import pytest

from linear_attention_saliency_amd import still

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "still.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w[\w\s\*]*?\b(still_\w+)\s*\(", text, re.M)))


def _cfg(**kw):
    base = dict(batch=1, seq_len=256, n_q_heads=4, n_kv_heads=1, head_dim=64, feat_dim=64, window=64, chunk=64,
                top_k=8, dtype="bf16")
    base.update(kw)
    return still.make_config(**base)


def test_library_exports_every_declared_symbol():
    lib = still.load()
    names = _declared()
    assert len(names) >= 9
    assert set(names) == set(still.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = still.load()
    for code, text in still.STATUS.items():
        assert lib.still_status_string(code).decode() == text
    assert lib.still_status_string(42).decode() == "unknown status"


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), -1), (dict(seq_len=0), -1), (dict(n_q_heads=6, n_kv_heads=4), -1), (dict(dtype="f16"), -1),
    (dict(window=-1), -1), (dict(top_k=65), -1), (dict(window=0, top_k=1), -1), (dict(chunk=32, window=32), -2),
    (dict(window=129), -2), (dict(head_dim=96), -2), (dict(feat_dim=32), -2), (dict(dtype="f32", head_dim=96), -2),
    (dict(seq_len=4_200_000, head_dim=128, feat_dim=128), -2),
])
def test_invalid_configs_rejected_before_launch(kw, code):
    lib = still.load()
    cfg = _cfg(**kw)
    assert lib.still_prefill_workspace_bytes(ctypes.byref(cfg)) == 0
    dummy = ctypes.c_void_p(4096)
    rc = lib.still_prefill(ctypes.byref(cfg), dummy, dummy, dummy, dummy, dummy, None, None, None, None, dummy,
                           1 << 40, None)
    assert rc == code


def test_windows_longer_than_a_chunk():
    """Windows up to 2 chunks are built for the forward and decode paths: the decode cache then
    holds one more chunk of raw rows (and its selection mask); the backward refuses them."""
    lib = still.load()
    for w in (65, 96, 128):
        cfg = _cfg(window=w)
        assert lib.still_prefill_workspace_bytes(ctypes.byref(cfg)) > 0, w
        assert lib.still_backward_workspace_bytes(ctypes.byref(cfg)) == 0, w
    assert lib.still_backward_workspace_bytes(ctypes.byref(_cfg(window=64))) > 0
    b1, b64, b65, b128 = (lib.still_cache_bytes(ctypes.byref(_cfg(window=w)), 4096) for w in (1, 64, 65, 128))
    assert b1 == b64 and b65 == b128 and b65 > b64
    cfg = _cfg()
    ring_row = cfg.batch * cfg.n_kv_heads * 64 * cfg.head_dim * 2  # one chunk of K (or V) rows, bf16
    assert b65 - b64 >= 2 * ring_row
    assert [still.band_chunks(w) for w in (0, 1, 64, 65, 128)] == [1, 1, 1, 2, 2]


def test_pointer_and_workspace_checks():
    lib = still.load()
    cfg = _cfg()
    need = lib.still_prefill_workspace_bytes(ctypes.byref(cfg))
    assert need > 0
    p = ctypes.c_void_p(1 << 20)
    bad = ctypes.c_void_p((1 << 20) + 8)
    assert lib.still_prefill(ctypes.byref(cfg), None, p, p, p, p, None, None, None, None, p, need, None) == -1
    assert lib.still_prefill(ctypes.byref(cfg), bad, p, p, p, p, None, None, None, None, p, need, None) == -1
    assert lib.still_prefill(ctypes.byref(cfg), p, p, p, p, p, None, None, None, None, p, need - 1, None) == -3
    cfg0 = _cfg(window=0, top_k=0)
    sal = ctypes.c_void_p(1 << 21)
    need0 = lib.still_prefill_workspace_bytes(ctypes.byref(cfg0))
    assert lib.still_prefill(ctypes.byref(cfg0), p, p, p, p, p, None, sal, None, None, p, need0, None) == -1


def test_f32_covers_every_head_and_feature_width():
    lib = still.load()
    for D in (64, 128):
        for F in (64, 128):
            assert lib.still_prefill_workspace_bytes(ctypes.byref(_cfg(dtype="f32", head_dim=D, feat_dim=F))) > 0
            assert lib.still_cache_bytes(ctypes.byref(_cfg(dtype="f32", head_dim=D, feat_dim=F)), 1024) > 0


def test_workspace_scales_with_sequence():
    lib = still.load()
    a = lib.still_prefill_workspace_bytes(ctypes.byref(_cfg(seq_len=1024)))
    b = lib.still_prefill_workspace_bytes(ctypes.byref(_cfg(seq_len=2048)))
    assert 1.8 < b / a < 2.2


def _fake_cache(cfg, max_tokens=4096, n_tokens=0):
    c = still.Cache()
    c.cfg = cfg
    c.max_tokens = max_tokens
    c.n_tokens = n_tokens
    c.sel_capacity = 64
    for f in ("sel_k", "sel_v", "ring_k", "ring_v", "state_s", "state_z", "sel_mask", "cur_saliency"):
        setattr(c, f, 1 << 24)
    return c


def test_cache_bytes_layout():
    lib = still.load()
    cfg = _cfg(n_q_heads=32, n_kv_heads=8, head_dim=128, feat_dim=128, top_k=16, batch=32)
    n = lib.still_cache_bytes(ctypes.byref(cfg), 65600)
    # compact rows: 1025 complete chunks x 16 rows, rounded up to tiles of 64 rows
    rows = (65600 // 64 * 16 + 63) // 64 * 64
    bh = 32 * 8
    compact = 2 * bh * rows * 128 * 2
    assert compact <= n < compact + 64 * 1024 * 1024
    assert lib.still_cache_bytes(ctypes.byref(cfg), 0) == 0
    assert lib.still_cache_bytes(ctypes.byref(_cfg(n_q_heads=17 * 2, n_kv_heads=2)), 1024) == 0  # group > 16
    assert lib.still_decode_workspace_bytes(ctypes.byref(cfg), 65600) > 0


def test_cache_init_rejects_bad_buffers():
    lib = still.load()
    cfg = _cfg()
    need = lib.still_cache_bytes(ctypes.byref(cfg), 1024)
    out = still.Cache()
    assert lib.still_cache_init(ctypes.byref(cfg), 1024, None, need, ctypes.byref(out), None) == -1
    assert lib.still_cache_init(ctypes.byref(cfg), 1024, ctypes.c_void_p((1 << 20) + 16), need,
                                ctypes.byref(out), None) == -1
    assert lib.still_cache_init(ctypes.byref(cfg), 1024, ctypes.c_void_p(1 << 20), need - 1,
                                ctypes.byref(out), None) == -3


def test_decode_step_validation():
    lib = still.load()
    cfg = _cfg()
    p = ctypes.c_void_p(1 << 20)
    ws = lib.still_decode_workspace_bytes(ctypes.byref(cfg), 4096)

    def step(cache, c=cfg, wsb=ws, q=p):
        return lib.still_decode_step(ctypes.byref(c), None if cache is None else ctypes.byref(cache), q, p, p, p,
                                     p, p, wsb, None)

    assert step(None) == -1
    assert step(_fake_cache(cfg), q=None) == -1
    assert step(_fake_cache(_cfg(top_k=4))) == -5
    assert step(_fake_cache(cfg, max_tokens=100, n_tokens=100)) == -4
    assert step(_fake_cache(cfg), wsb=ws - 1) == -3
    # prefill into a cache: wrong layer, non-empty cache, too short
    need = lib.still_prefill_workspace_bytes(ctypes.byref(cfg))
    for cache, code in ((_fake_cache(_cfg(window=32)), -5), (_fake_cache(cfg, n_tokens=5), -1),
                        (_fake_cache(cfg, max_tokens=100), -4)):
        assert lib.still_prefill(ctypes.byref(cfg), p, p, p, p, p, None, None, None, ctypes.byref(cache), p, need,
                                 None) == code


def test_routing_scope_checks():
    """Per-query-head routing: a bad scope is rejected; the prefill keeps per-query-head
    records (scores, selections, compact rows, states) but no copy of K or V; the decode
    cache holds per-query-head records; the backward workspace includes expanded copies."""
    lib = still.load()
    assert lib.still_prefill_workspace_bytes(ctypes.byref(_cfg(scope="bogus"))) == 0
    cq, ckv = _cfg(scope="query_head"), _cfg()
    q1 = lib.still_prefill_workspace_bytes(ctypes.byref(cq))
    kv = lib.still_prefill_workspace_bytes(ctypes.byref(ckv))
    assert q1 > kv > 0
    kv_copies = 2 * ckv.batch * ckv.seq_len * ckv.n_q_heads * ckv.head_dim * 2  # K and V per query head, bf16
    assert q1 - kv < kv_copies
    assert lib.still_cache_bytes(ctypes.byref(cq), 1024) > lib.still_cache_bytes(ctypes.byref(ckv), 1024) > 0
    assert lib.still_backward_workspace_bytes(ctypes.byref(_cfg(scope="query_head"))) > \
        lib.still_backward_workspace_bytes(ctypes.byref(_cfg())) > 0
    assert lib.still_future_attention_mass_workspace_bytes(ctypes.byref(_cfg(scope="query_head"))) == 0


def test_routing_override_is_validated_on_the_host():
    """routing_in is host memory, checked before anything is enqueued: each chunk's top_k
    entries strictly ascending inside the chunk, else INVALID_ARG."""
    import numpy as np

    lib = still.load()
    cfg = _cfg(seq_len=200, top_k=4)  # 3 complete chunks
    need = lib.still_prefill_workspace_bytes(ctypes.byref(cfg))
    p = ctypes.c_void_p(1 << 20)
    good = np.array([[[[1, 5, 9, 63], [64, 65, 66, 127], [130, 140, 150, 191]]]], dtype=np.int32)
    bad_cases = []
    for (c, i, val) in ((0, 3, 64), (1, 0, 63), (2, 1, 130), (2, 2, 139), (0, 0, -1)):
        r = good.copy()
        r[0, 0, c, i] = val  # out of its chunk, repeated, or descending
        bad_cases.append(r)
    for r in bad_cases:
        rc = lib.still_prefill(ctypes.byref(cfg), p, p, p, p, p, ctypes.c_void_p(r.ctypes.data), None, None, None,
                               p, need, None)
        assert rc == -1
    # per-query-head routing validates [batch, n_q_heads, ...] records
    cfgq = _cfg(seq_len=200, top_k=4, scope="query_head")
    needq = lib.still_prefill_workspace_bytes(ctypes.byref(cfgq))
    rq = np.broadcast_to(good, (1, 4, 3, 4)).copy()
    rq[0, 3, 1, 2] = 200
    assert lib.still_prefill(ctypes.byref(cfgq), p, p, p, p, p, ctypes.c_void_p(rq.ctypes.data), None, None, None,
                             p, needq, None) == -1


def test_last_hip_error_starts_clear():
    lib = still.load()
    assert lib.still_last_hip_error() == 0


def test_timing_event_helpers_reject_null_arguments():
    # argument checks come before any HIP call, so they run without a GPU
    lib = still.load()
    assert lib.still_timing_event_create(None) == -1
    assert lib.still_timing_event_destroy(None) == -1
    assert lib.still_timing_event_record(None, None) == -1
    ms = ctypes.c_float()
    assert lib.still_timing_event_elapsed_ms(None, None, ctypes.byref(ms)) == -1
    assert lib.still_timing_event_elapsed_ms(ctypes.c_void_p(16), ctypes.c_void_p(32), None) == -1
