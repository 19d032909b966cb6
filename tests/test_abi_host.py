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
    (dict(window=65), -2), (dict(head_dim=96), -2), (dict(feat_dim=32), -2), (dict(dtype="f32", head_dim=128), -2),
])
def test_invalid_configs_rejected_before_launch(kw, code):
    lib = still.load()
    cfg = _cfg(**kw)
    assert lib.still_prefill_workspace_bytes(ctypes.byref(cfg)) == 0
    dummy = ctypes.c_void_p(4096)
    rc = lib.still_prefill(ctypes.byref(cfg), dummy, dummy, dummy, dummy, dummy, None, None, None, None, dummy,
                           1 << 40, None)
    assert rc == code


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


def test_workspace_scales_with_sequence():
    lib = still.load()
    a = lib.still_prefill_workspace_bytes(ctypes.byref(_cfg(seq_len=1024)))
    b = lib.still_prefill_workspace_bytes(ctypes.byref(_cfg(seq_len=2048)))
    assert 1.8 < b / a < 2.2
