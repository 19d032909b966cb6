"""Python binding of libstill.so (argument marshalling only).

Every step of the layer runs in the library's HIP kernels; torch is used here only to
allocate device memory and to name the current HIP stream. If the library is missing
this module raises: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libstill.so")

STILL_F32, STILL_BF16 = 0, 1
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported configuration", -3: "workspace too small",
          -4: "decode cache full", -5: "decode cache built for another configuration",
          -6: "HIP launch error"}

EXPORTS = ("still_status_string", "still_prefill_workspace_bytes", "still_prefill", "still_prefill_timed",
           "still_select_topk",
           "still_feature_map", "still_cache_bytes", "still_cache_init", "still_decode_workspace_bytes",
           "still_decode_step", "still_decode_step_timed", "still_backward_workspace_bytes", "still_backward",
           "still_backward_timed", "still_future_attention_mass_workspace_bytes", "still_future_attention_mass",
           "still_selection_overlap", "still_last_hip_error", "still_decode_step_noalloc",
           "still_timing_event_create", "still_timing_event_destroy", "still_timing_event_record",
           "still_timing_event_elapsed_ms")


class StillError(RuntimeError):
    def __init__(self, code: int, what: str = "", hip_error: int = 0):
        msg = f"{what}: status {code} ({STATUS.get(code, 'unknown')})"
        if hip_error:
            msg += f", hipError_t {hip_error}"
        super().__init__(msg)
        self.code = code
        self.hip_error = hip_error


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("batch", "seq_len", "n_q_heads", "n_kv_heads", "head_dim",
                                               "feat_dim", "window", "chunk", "top_k", "dtype", "score",
                                               "routing_scope")]


class Cache(ctypes.Structure):
    _fields_ = [("cfg", Config), ("max_tokens", ctypes.c_int64), ("n_tokens", ctypes.c_int64),
                ("sel_capacity", ctypes.c_int64),
                ("sel_k", ctypes.c_void_p), ("sel_v", ctypes.c_void_p), ("ring_k", ctypes.c_void_p),
                ("ring_v", ctypes.c_void_p), ("state_s", ctypes.c_void_p), ("state_z", ctypes.c_void_p),
                ("sel_mask", ctypes.c_void_p), ("cur_saliency", ctypes.c_void_p)]


_lib = None


def load():
    """Load libstill.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, S, V = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    CP = ctypes.POINTER(Config)
    KP = ctypes.POINTER(Cache)
    lib.still_status_string.argtypes = [I]
    lib.still_status_string.restype = ctypes.c_char_p
    lib.still_prefill_workspace_bytes.argtypes = [CP]
    lib.still_prefill_workspace_bytes.restype = S
    lib.still_prefill.argtypes = [CP, P, P, P, P, P, P, P, P, KP, P, S, V]
    lib.still_prefill.restype = I
    lib.still_prefill_timed.argtypes = [CP, P, P, P, P, P, P, P, P, KP, P, S, V, P]
    lib.still_prefill_timed.restype = I
    lib.still_select_topk.argtypes = [CP, P, P, V]
    lib.still_select_topk.restype = I
    lib.still_feature_map.argtypes = [CP, P, P, P, V]
    lib.still_feature_map.restype = I
    lib.still_cache_bytes.argtypes = [CP, ctypes.c_int64]
    lib.still_cache_bytes.restype = S
    lib.still_cache_init.argtypes = [CP, ctypes.c_int64, P, S, KP, V]
    lib.still_cache_init.restype = I
    lib.still_decode_workspace_bytes.argtypes = [CP, ctypes.c_int64]
    lib.still_decode_workspace_bytes.restype = S
    lib.still_decode_step.argtypes = [CP, KP, P, P, P, P, P, P, S, V]
    lib.still_decode_step.restype = I
    lib.still_decode_step_timed.argtypes = [CP, KP, P, P, P, P, P, P, S, V, P]
    lib.still_decode_step_timed.restype = I
    lib.still_backward_workspace_bytes.argtypes = [CP]
    lib.still_backward_workspace_bytes.restype = S
    lib.still_backward.argtypes = [CP, P, P, P, P, P, P, P, P, P, P, P, P, S, V]
    lib.still_backward.restype = I
    lib.still_backward_timed.argtypes = [CP, P, P, P, P, P, P, P, P, P, P, P, P, S, V, P]
    lib.still_backward_timed.restype = I
    lib.still_future_attention_mass_workspace_bytes.argtypes = [CP]
    lib.still_future_attention_mass_workspace_bytes.restype = S
    lib.still_future_attention_mass.argtypes = [CP, P, P, P, P, S, V]
    lib.still_future_attention_mass.restype = I
    lib.still_selection_overlap.argtypes = [CP, P, P, P, V]
    lib.still_selection_overlap.restype = I
    lib.still_decode_step_noalloc.argtypes = [CP, KP, P, P, P, P, P, V]
    lib.still_decode_step_noalloc.restype = I
    lib.still_timing_event_create.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.still_timing_event_create.restype = I
    lib.still_timing_event_destroy.argtypes = [V]
    lib.still_timing_event_destroy.restype = I
    lib.still_timing_event_record.argtypes = [V, V]
    lib.still_timing_event_record.restype = I
    lib.still_timing_event_elapsed_ms.argtypes = [V, V, ctypes.POINTER(ctypes.c_float)]
    lib.still_timing_event_elapsed_ms.restype = I
    lib.still_last_hip_error.argtypes = []
    lib.still_last_hip_error.restype = I
    _lib = lib
    return lib


SCORES = {"saliency": 0, "diag": 1}  # still_score: the routing score
SCOPES = {"kv_head": 0, "query_head": 1}  # still_routing_scope: who selects


def band_chunks(window: int) -> int:
    """Earlier chunks a query's window can reach, at least 1 (the library's band length): a
    decode cache holds band_chunks(window) + 1 chunks of raw rows, chunk x in slot
    x % (band_chunks(window) + 1)."""
    return 1 if window <= 64 else (window + 63) // 64


def make_config(batch, seq_len, n_q_heads, n_kv_heads, head_dim, feat_dim, window, chunk, top_k,
                dtype, score: str = "saliency", scope: str = "kv_head") -> Config:
    dt = STILL_BF16 if dtype in (torch.bfloat16, "bf16") else STILL_F32 if dtype in (torch.float32, "f32") else -1
    return Config(batch, seq_len, n_q_heads, n_kv_heads, head_dim, feat_dim, window, chunk, top_k, dt,
                  SCORES.get(score, -1), SCOPES.get(scope, -1))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int, what: str):
    if rc != 0:
        raise StillError(rc, what, load().still_last_hip_error() if rc == -6 else 0)


def _host_i32(t):
    """A C-contiguous int32 host copy of a tensor or array (kept alive by the caller)."""
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        t = t.detach().to("cpu", torch.int32).numpy()
    import numpy as np

    return np.ascontiguousarray(t, dtype=np.int32)


def _tensor_cfg(q, k, w_phi, window, chunk, top_k, score="saliency", scope="kv_head"):
    if q.dim() != 4 or k.dim() != 4 or w_phi.dim() != 3:
        raise ValueError("q/k must be [B,T,H,D] and w_phi [Hkv,d_f,D]")
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    return make_config(B, T, Hq, Hkv, D, w_phi.shape[1], window, chunk, top_k, q.dtype, score, scope)


def workspace_bytes(cfg: Config) -> int:
    return int(load().still_prefill_workspace_bytes(ctypes.byref(cfg)))


class Prefill:
    """A prepared prefill call: the config and a reusable workspace for fixed shapes."""

    def __init__(self, q, k, v, w_phi, *, window: int, top_k: int, chunk: int = 64, score: str = "saliency",
                 scope: str = "kv_head"):
        self.cfg = _tensor_cfg(q, k, w_phi, window, chunk, top_k, score, scope)
        nbytes = workspace_bytes(self.cfg)
        if nbytes == 0:
            rc = load().still_prefill(ctypes.byref(self.cfg), None, None, None, None, None, None, None, None,
                                      None, None, 0, None)
            _check(rc, "still_prefill config")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)

    def __call__(self, q, k, v, w_phi, out, *, routing=None, saliency=None, sel_idx=None, cache=None,
                 stream=None, events=None):
        """events: optional array of 4 hipEvent_t handles (ctypes c_void_p * 4); a None entry is not recorded.
        cache: optional DecodeCache with no tokens; it is left holding the sequence.
        routing: optional selection override (host or device tensor, or array), passed to the
        library as host memory."""
        for t in (q, k, v, w_phi, out):
            if not (t.is_cuda and t.is_contiguous()):
                raise ValueError("tensors must be contiguous device tensors")
        r = _host_i32(routing)
        rptr = None if r is None else ctypes.c_void_p(r.ctypes.data)
        rc = load().still_prefill_timed(ctypes.byref(self.cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(w_phi),
                                        _ptr(out), rptr, _ptr(saliency), _ptr(sel_idx),
                                        None if cache is None else ctypes.byref(cache.c),
                                        _ptr(self.workspace), self.workspace.numel(), _stream(stream),
                                        events)
        _check(rc, "still_prefill")
        return out


def prefill(q, k, v, w_phi, *, window: int, top_k: int, chunk: int = 64, routing=None,
            return_saliency: bool = False, return_routing: bool = False, cache=None, score: str = "saliency",
            scope: str = "kv_head"):
    """One STILL layer over whole sequences.

    q [B,T,Hq,D], k/v [B,T,Hkv,D], w_phi [Hkv,d_f,D] (all float32 or all bfloat16, on the
    GPU). routing: optional int32 [B,Hkv,T//chunk,top_k] override of the selection (ascending
    positions inside each chunk; anything else raises StillError with status -1).
    cache: optional empty DecodeCache (of the same scope), left ready to decode token T.
    score: "saliency" (the Self-Saliency Score) or "diag" (the diagonal logit alone).
    scope: "kv_head" (each KV head selects for its group) or "query_head" (each query head
    selects for itself; the score and routing are then [B,Hq,...]).
    Returns out (and the routing score [B,Hkv,T] fp32, sel_idx [B,Hkv,T//chunk,top_k] int32
    on request).
    """
    call = Prefill(q, k, v, w_phi, window=window, top_k=top_k, chunk=chunk, score=score, scope=scope)
    B, T, Hq, _ = q.shape
    Hkv = Hq if scope == "query_head" else k.shape[2]  # heads that select
    out = torch.empty_like(q)
    sal = torch.empty((B, Hkv, T), dtype=torch.float32, device=q.device) if return_saliency else None
    sel = torch.empty((B, Hkv, T // chunk, top_k), dtype=torch.int32, device=q.device) if return_routing else None
    call(q, k, v, w_phi, out, routing=routing, saliency=sal, sel_idx=sel, cache=cache)
    res = [out]
    if return_saliency:
        res.append(sal)
    if return_routing:
        res.append(sel)
    return res[0] if len(res) == 1 else tuple(res)


class Backward:
    """A prepared backward call (routing held fixed): the config and a reusable workspace."""

    def __init__(self, q, k, v, w_phi, *, window: int, top_k: int, chunk: int = 64, scope: str = "kv_head"):
        self.cfg = _tensor_cfg(q, k, w_phi, window, chunk, top_k, scope=scope)
        nbytes = int(load().still_backward_workspace_bytes(ctypes.byref(self.cfg)))
        if nbytes == 0:
            raise StillError(-2, "still_backward_workspace_bytes")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)

    def __call__(self, q, k, v, w_phi, out, dout, sel_idx, dq, dk, dv, dw_phi, *, stream=None, events=None):
        """events: optional array of 8 hipEvent_t handles (ctypes c_void_p * 8)."""
        for t in (q, k, v, w_phi, out, dout, dq, dk, dv, dw_phi):
            if not (t.is_cuda and t.is_contiguous()):
                raise ValueError("tensors must be contiguous device tensors")
        if sel_idx is not None and not (sel_idx.is_cuda and sel_idx.is_contiguous() and sel_idx.dtype == torch.int32):
            raise ValueError("sel_idx must be a contiguous int32 device tensor")
        rc = load().still_backward_timed(ctypes.byref(self.cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(w_phi), _ptr(out),
                                         _ptr(dout), _ptr(sel_idx), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dw_phi),
                                         _ptr(self.workspace), self.workspace.numel(), _stream(stream), events)
        _check(rc, "still_backward")
        return dq, dk, dv, dw_phi


def backward(q, k, v, w_phi, out, dout, sel_idx, *, window: int, top_k: int, chunk: int = 64, scope: str = "kv_head"):
    """Gradients of sum(out * dout) for one STILL layer with the routing sel_idx held fixed.

    q [B,T,Hq,D], k/v [B,T,Hkv,D], w_phi [Hkv,d_f,D], out and dout like q (one dtype, on the
    GPU); sel_idx int32 [B,Hkv,T//chunk,top_k] as prefill(return_routing=True) gives it.
    Returns (dq, dk, dv) in the inputs' dtype and dw_phi in float32.
    """
    call = Backward(q, k, v, w_phi, window=window, top_k=top_k, chunk=chunk, scope=scope)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dw = torch.empty(w_phi.shape, dtype=torch.float32, device=q.device)
    if sel_idx is not None:
        sel_idx = sel_idx.to(device=q.device, dtype=torch.int32).contiguous()
    return call(q, k, v, w_phi, out, dout, sel_idx, dq, dk, dv, dw)


class FutureAttentionMass:
    """A prepared call of still_future_attention_mass (fixed shapes, reusable workspace)."""

    def __init__(self, q, k, *, window: int):
        B, T, Hq, D = q.shape
        self.cfg = make_config(B, T, Hq, k.shape[2], D, 64, window, 64, 0, q.dtype)
        nbytes = int(load().still_future_attention_mass_workspace_bytes(ctypes.byref(self.cfg)))
        if nbytes == 0:
            raise StillError(-2, "still_future_attention_mass_workspace_bytes")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)

    def __call__(self, q, k, mass, *, stream=None):
        for t in (q, k, mass):
            if not (t.is_cuda and t.is_contiguous()):
                raise ValueError("tensors must be contiguous device tensors")
        rc = load().still_future_attention_mass(ctypes.byref(self.cfg), _ptr(q), _ptr(k), _ptr(mass),
                                                _ptr(self.workspace), self.workspace.numel(), _stream(stream))
        _check(rc, "still_future_attention_mass")
        return mass


def future_attention_mass(q, k, *, window: int):
    """Attention each key receives from queries at distance >= window under full causal
    softmax, summed over the query heads of its KV head: fp32 [B,Hkv,T]."""
    B, T, _, _ = q.shape
    mass = torch.empty((B, k.shape[2], T), dtype=torch.float32, device=q.device)
    return FutureAttentionMass(q, k, window=window)(q, k, mass)


def selection_overlap(sel_a, sel_b):
    """Tokens two per-chunk selections [B,Hkv,nC,k] (int32, device) share: int32 [B,Hkv,nC]."""
    B, Hkv, nC, k = sel_a.shape
    cfg = make_config(B, nC * 64, Hkv, Hkv, 64, 64, 64, 64, k, torch.bfloat16)
    out = torch.zeros((B, Hkv, nC), dtype=torch.int32, device=sel_a.device)
    rc = load().still_selection_overlap(ctypes.byref(cfg), _ptr(sel_a.contiguous()), _ptr(sel_b.contiguous()),
                                        _ptr(out), _stream())
    _check(rc, "still_selection_overlap")
    return out


def saliency_fidelity(q, k, w_phi, *, window: int, top_k: int, score: str = "saliency"):
    """Local-global consistency of the routing on these inputs: the layer's own per-chunk
    selection (from the local routing score) against the top_k of each chunk by attention
    from far-future queries under full causal softmax.

    Returns a dict of device tensors: sel_local and sel_global [B,Hkv,T//64,top_k], common
    [B,Hkv,T//64] (tokens both selections hold), mass [B,Hkv,T]; and `overlap`, the mean of
    common / top_k over the chunks whose every token has at least one far-future query.
    """
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    _, sel_local = prefill(q, k, k, w_phi, window=window, top_k=top_k, return_routing=True, score=score)
    mass = future_attention_mass(q, k, window=window)
    sel_global = select_topk(mass, chunk=64, top_k=top_k, n_q_heads=Hq // Hkv, head_dim=D,
                             feat_dim=w_phi.shape[1], dtype=q.dtype)
    common = selection_overlap(sel_local, sel_global)
    n_ok = max(0, min(T // 64, (T - window) // 64))  # chunks c with 64 c + 63 + window <= T - 1
    overlap = float(common[:, :, :n_ok].double().mean() / top_k) if n_ok > 0 else float("nan")
    return {"sel_local": sel_local, "sel_global": sel_global, "common": common, "mass": mass, "overlap": overlap}


def select_topk(saliency, *, chunk: int, top_k: int, n_q_heads: int = 1, head_dim: int = 64, feat_dim: int = 64,
                dtype=torch.bfloat16):
    """Per-chunk top-k of a device saliency tensor [B,Hkv,T] fp32 -> int32 [B,Hkv,T//chunk,top_k]."""
    B, Hkv, T = saliency.shape
    cfg = make_config(B, T, Hkv * n_q_heads, Hkv, head_dim, feat_dim, chunk, chunk, top_k, dtype)
    sel = torch.empty((B, Hkv, T // chunk, top_k), dtype=torch.int32, device=saliency.device)
    rc = load().still_select_topk(ctypes.byref(cfg), _ptr(saliency.contiguous()), _ptr(sel), _stream())
    _check(rc, "still_select_topk")
    return sel


def feature_map(x, w_phi):
    """NP-Map of device rows x [B,T,Hkv,D] with w_phi [Hkv,d_f,D] -> fp32 [B,T,Hkv,d_f]."""
    B, T, Hkv, D = x.shape
    F = w_phi.shape[1]
    cfg = make_config(B, T, Hkv, Hkv, D, F, 64, 64, 0, x.dtype)
    phi = torch.empty((B, T, Hkv, F), dtype=torch.float32, device=x.device)
    rc = load().still_feature_map(ctypes.byref(cfg), _ptr(x), _ptr(w_phi), _ptr(phi), _stream())
    _check(rc, "still_feature_map")
    return phi


class TimingEvent:
    """A HIP event from still_timing_event_create (device-scope release): for timing the
    library's kernels without a system-scope cache write-back at every record."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(load().still_timing_event_create(ctypes.byref(h)), "still_timing_event_create")
        self.handle = h.value

    def record(self, stream=None):
        _check(load().still_timing_event_record(self.handle, _stream(stream)), "still_timing_event_record")

    def elapsed_time(self, end: "TimingEvent") -> float:
        """Milliseconds from this event to `end` (both completed: synchronise first)."""
        ms = ctypes.c_float()
        _check(load().still_timing_event_elapsed_ms(self.handle, end.handle, ctypes.byref(ms)),
               "still_timing_event_elapsed_ms")
        return float(ms.value)

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.still_timing_event_destroy(self.handle)
            self.handle = None


class DecodeCache:
    """Device decode state of one layer for `batch` sequences of up to `max_tokens` tokens.

    Owns one device buffer (allocated by torch) carved by still_cache_init, plus the
    decode workspace. `c` is the C record (n_tokens advances with every step).
    """

    def __init__(self, *, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, feat_dim: int,
                 window: int, top_k: int, max_tokens: int, dtype=torch.bfloat16, chunk: int = 64,
                 device="cuda", score: str = "saliency", scope: str = "kv_head"):
        lib = load()
        self.cfg = make_config(batch, 0, n_q_heads, n_kv_heads, head_dim, feat_dim, window, chunk, top_k, dtype,
                               score, scope)
        nbytes = int(lib.still_cache_bytes(ctypes.byref(self.cfg), max_tokens))
        if nbytes == 0:
            raise StillError(-2, "still_cache_bytes")
        self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.c = Cache()
        _check(lib.still_cache_init(ctypes.byref(self.cfg), max_tokens, _ptr(self.buffer), nbytes,
                                    ctypes.byref(self.c), _stream()), "still_cache_init")
        ws = int(lib.still_decode_workspace_bytes(ctypes.byref(self.cfg), max_tokens))
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)

    @property
    def n_tokens(self) -> int:
        return int(self.c.n_tokens)

    def tensors(self):
        """Views of the device state (for inspection): dict of torch tensors."""
        c, cfg = self.c, self.cfg
        B, D, F = cfg.batch, cfg.head_dim, cfg.feat_dim
        H = cfg.n_q_heads if cfg.routing_scope == SCOPES["query_head"] else cfg.n_kv_heads  # heads that select
        dt = torch.bfloat16 if cfg.dtype == STILL_BF16 else torch.float32
        es = 2 if dt == torch.bfloat16 else 4
        base = self.buffer.data_ptr()

        def view(ptr, shape, dtype, esize):
            n = 1
            for x in shape:
                n *= x
            off = ptr - base
            return self.buffer[off:off + n * esize].view(dtype).view(*shape)

        cap = int(c.sel_capacity)
        nr = band_chunks(cfg.window) + 1  # ring slots
        return {
            "sel_k": view(c.sel_k, (B, H, cap, D), dt, es),
            "sel_v": view(c.sel_v, (B, H, cap // 64, D, 64), dt, es),
            "ring_k": view(c.ring_k, (B, H, nr, 64, D), dt, es),
            "ring_v": view(c.ring_v, (B, H, nr, 64, D), dt, es),
            "state_s": view(c.state_s, (B, H, F, D), torch.float32, 4),
            "state_z": view(c.state_z, (B, H, F), torch.float32, 4),
            "sel_mask": view(c.sel_mask, (B, H, nr), torch.int64, 8),
            "cur_saliency": view(c.cur_saliency, (B, H, 64), torch.float32, 4),
        }

    def step(self, q, k, v, w_phi, out=None, *, stream=None, events=None):
        """One token per sequence: q [B,Hq,D], k/v [B,Hkv,D] -> out [B,Hq,D]."""
        for t in (q, k, v, w_phi):
            if not (t.is_cuda and t.is_contiguous()):
                raise ValueError("tensors must be contiguous device tensors")
        if out is None:
            out = torch.empty_like(q)
        rc = load().still_decode_step_timed(ctypes.byref(self.cfg), ctypes.byref(self.c), _ptr(q), _ptr(k),
                                            _ptr(v), _ptr(w_phi), _ptr(out), _ptr(self.workspace),
                                            self.workspace.numel(), _stream(stream), events)
        _check(rc, "still_decode_step")
        return out

    def step_noalloc(self, q, k, v, w_phi, out, *, stream=None):
        """As step(), through still_decode_step_noalloc: no workspace, the library's own
        device scratch (out must be given: nothing is allocated)."""
        for t in (q, k, v, w_phi, out):
            if not (t.is_cuda and t.is_contiguous()):
                raise ValueError("tensors must be contiguous device tensors")
        rc = load().still_decode_step_noalloc(ctypes.byref(self.cfg), ctypes.byref(self.c), _ptr(q), _ptr(k),
                                              _ptr(v), _ptr(w_phi), _ptr(out), _stream(stream))
        _check(rc, "still_decode_step_noalloc")
        return out
