"""fp64 CPU oracle for one STILL intra-layer hybrid attention layer.

TEST INFRASTRUCTURE ONLY. This module is imported by the tests, by the smoke check and
by the CPU-baseline leg of the benchmark. The library (the HIP path behind the C ABI)
never imports, links or calls it, and it shares no code with that path.

Pages cited below (the method's only description):
  [P1] "仅0.04B！哈工深首创同层混合架构STILL，极低成本线性化LLM" (PaperWeekly repost),
       sections "Self-Saliency Score", "Norm-Preserved Feature Map（NP-Map）",
       "Chunk-Wise并行+延迟选择", and the paragraph before "STILL三大创新".
  [P2] "STILL: Content-Aware Intra-Layer Hybrid Attention Cuts Memory 80%, Speeds
       Prefill 83%" (picx.dev), summary and the 机器之心 excerpt.
  [P3] "STILL от HIT Shenzhen: гибридное внимание внутри слоя выбирает токены по
       содержанию" (news piece), section on why hybrids are called pseudo-hybrid.
  [P4] "STILL: Selecting Tokens for Intra-Layer Hybrid Attention to Linearize LLMs"
       (research-map summary), sections Problem and Approach.

Readings taken where the pages are silent (each is exercised by a test):
  * window W_i = {max(0, i-w+1), ..., i}: length w, causal, contains i itself;
  * logits a_ij = q_i . k_j / sqrt(D) for both the saliency and the softmax branch;
  * saliency s_i = KL(q_i || p_i) where p_i is the window softmax with the diagonal and
    q_i the one without it; this equals -log(1 - p_ii) = LSE(W_i) - LSE(W_i minus i),
    and is +inf when W_i = {i};
  * GQA: query head hq uses KV head hq // G (G = Hq / Hkv); routing is per KV head on the
    sum of the G query heads' saliency;
  * routing: in every complete chunk of C tokens the top_k largest saliencies are
    selected, ties to the lower index; a selection affects only queries of later chunks;
    tokens of an incomplete final chunk are never selected;
  * token j is in query i's softmax set iff j > i - w, or j lies in an earlier chunk and
    was selected; every other j <= i goes to linear attention;
  * NP-Map phi(x) = |x| * m / |m|,  m = elu(W_h x) + 1 (alpha = 1), W_h [d_f, D] per KV
    head, shared by queries and keys; phi(0) = 0;
  * fusion with one shared normaliser:
      o_i = (sum_SA e^{a_ij - M} v_j + e^{-M} sum_LA (phi(q_i).phi(k_j)) v_j)
            / (sum_SA e^{a_ij - M} + e^{-M} sum_LA phi(q_i).phi(k_j)),
    M = max over the softmax set (0 when that set is empty); o_i = 0 if the denominator is 0.

Parity pins: every function here is pinned in tests/test_oracle_pins.py against closed
forms, library routines (torch SDPA / ELU in fp64) and hand-derived cases. The backward
pass (attend_backward) is pinned against central finite differences of attend, against
an exact identity of the gradients, and against torch SDPA's gradients where the layer
reduces to causal softmax attention.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "lse", "saliency", "route", "route_margins", "np_map", "sa_mask_row", "brute",
    "brute_rows", "attend", "attend_backward", "future_attention_mass", "selection_overlap", "DecodeOracle",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def lse(a: np.ndarray, axis: int = -1) -> np.ndarray:
    """log(sum(exp(a))) along an axis; an all -inf (empty) slice gives -inf."""
    a = _f64(a)
    m = np.max(a, axis=axis, keepdims=True)
    finite = np.isfinite(m)
    m0 = np.where(finite, m, 0.0)
    with np.errstate(divide="ignore"):
        r = np.log(np.sum(np.exp(a - m0), axis=axis, keepdims=True)) + m0
    r = np.where(finite, r, -np.inf)
    return np.squeeze(r, axis=axis)


def _check_group(Hq: int, Hkv: int) -> int:
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("n_q_heads must be a positive multiple of n_kv_heads")
    return Hq // Hkv


# --------------------------------------------------------------------------------------
# Self-Saliency Score  ([P1] section "Self-Saliency Score"; [P4] section Approach)
# --------------------------------------------------------------------------------------

def _saliency_one_head(q: np.ndarray, k: np.ndarray, window: int) -> np.ndarray:
    """s_i for one query head: q [T,D], k [T,D] -> [T].

    Token i attends over its causal window once with and once without its own (diagonal)
    key; the divergence between the two window distributions is its saliency. In log-sum-
    exp form: s_i = LSE_{j in W_i} a_ij - LSE_{j in W_i, j != i} a_ij.
    """
    T, D = q.shape
    a = np.full((T, window), -np.inf)  # a[i, o] = a_{i, i-o}; o = 0 is the diagonal
    for o in range(min(window, T)):
        a[o:, o] = np.einsum("td,td->t", q[o:], k[: T - o]) / math.sqrt(D)
    with_diag = lse(a, axis=1)
    without_diag = lse(a[:, 1:], axis=1) if window > 1 else np.full(T, -np.inf)
    return with_diag - without_diag  # -inf subtracted -> +inf for a one-token window


def saliency(q, k, window: int):
    """Self-Saliency Score per query head and per KV head.

    q [B,T,Hq,D], k [B,T,Hkv,D] -> (s_kv [B,Hkv,T], s_q [B,Hq,T]); s_kv sums the G query
    heads of each group (reading for GQA, module header).
    """
    q, k = _f64(q), _f64(k)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = _check_group(Hq, Hkv)
    if window < 1:
        raise ValueError("saliency needs a window of at least one token")
    s_q = np.empty((B, Hq, T))
    for b in range(B):
        for hq in range(Hq):
            s_q[b, hq] = _saliency_one_head(q[b, :, hq], k[b, :, hq // G], window)
    s_kv = s_q.reshape(B, Hkv, G, T).sum(axis=2)
    return s_kv, s_q


def diagonal_score(q, k):
    """Routing score of the pages' ablation that routes by the diagonal attention alone
    ([P4] section "Surprising findings"): the raw diagonal logit q_i . k_i / sqrt(D) per
    query head, summed over each KV head's group as for the saliency. (The diagonal softmax
    weight p_ii itself would route exactly like the saliency, which grows with it.)

    q [B,T,Hq,D], k [B,T,Hkv,D] -> (s_kv [B,Hkv,T], s_q [B,Hq,T]).
    """
    q, k = _f64(q), _f64(k)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = _check_group(Hq, Hkv)
    kq = np.repeat(k, G, axis=2)  # query head hq reads KV head hq // G
    s_q = np.einsum("bthd,bthd->bht", q, kq) / np.sqrt(D)
    s_kv = s_q.reshape(B, Hkv, G, T).sum(axis=2)
    return s_kv, s_q


# --------------------------------------------------------------------------------------
# Chunk-wise routing  ([P1] section "Chunk-Wise并行+延迟选择"; [P4] section Approach)
# --------------------------------------------------------------------------------------

def route(s_kv, chunk: int, top_k: int):
    """Per complete chunk, select the top_k tokens by saliency (ties -> lower index).

    s_kv [B,Hkv,T] -> (sel_idx [B,Hkv,T//chunk,top_k] int64 ascending positions,
                       sel [B,Hkv,T] bool). Tokens of an incomplete last chunk stay False.
    """
    s_kv = _f64(s_kv)
    B, H, T = s_kv.shape
    if not (0 <= top_k <= chunk):
        raise ValueError("top_k must lie in [0, chunk]")
    n_full = T // chunk
    sel_idx = np.zeros((B, H, n_full, top_k), dtype=np.int64)
    sel = np.zeros((B, H, T), dtype=bool)
    idx = np.arange(chunk)
    for b in range(B):
        for h in range(H):
            for c in range(n_full):
                seg = s_kv[b, h, c * chunk:(c + 1) * chunk]
                order = np.lexsort((idx, -seg))  # saliency descending, then index ascending
                pick = np.sort(order[:top_k]) + c * chunk
                sel_idx[b, h, c] = pick
                sel[b, h, pick] = True
    return sel_idx, sel


def route_margins(s_kv, chunk: int, top_k: int) -> np.ndarray:
    """Per complete chunk, the gap between the k-th and (k+1)-th largest saliency.

    [B,Hkv,T//chunk]; +inf when top_k is 0 or chunk (no competing token), and 0 on ties.
    A selection whose margin exceeds a device's saliency error is unique on that device.
    """
    s_kv = _f64(s_kv)
    B, H, T = s_kv.shape
    n_full = T // chunk
    out = np.full((B, H, n_full), np.inf)
    if top_k == 0 or top_k == chunk:
        return out
    for b in range(B):
        for h in range(H):
            for c in range(n_full):
                seg = np.sort(s_kv[b, h, c * chunk:(c + 1) * chunk])[::-1]
                hi, lo = seg[top_k - 1], seg[top_k]
                if np.isinf(hi):
                    out[b, h, c] = 0.0 if np.isinf(lo) else np.inf
                else:
                    out[b, h, c] = hi - lo
    return out


# --------------------------------------------------------------------------------------
# NP-Map  ([P1] section "Norm-Preserved Feature Map（NP-Map）"; [P4] section Approach)
# --------------------------------------------------------------------------------------

def np_map(x, w) -> np.ndarray:
    """phi(x) = |x|_2 * m / |m|_2 with m = elu(W x) + 1.

    The map keeps the direction from a one-layer positive feature map and puts back the
    original vector's norm. x [..., D], w [d_f, D] -> [..., d_f]. m > 0 elementwise, so the
    division is always defined, and phi(0) = 0.
    """
    x, w = _f64(x), _f64(w)
    z = x @ w.T
    m = np.where(z > 0.0, z + 1.0, np.exp(np.minimum(z, 0.0)))  # elu(z) + 1, alpha = 1
    nx = np.linalg.norm(x, axis=-1, keepdims=True)
    nm = np.linalg.norm(m, axis=-1, keepdims=True)
    return nx * m / nm


# --------------------------------------------------------------------------------------
# Partition and fused output  ([P1] paragraph before "STILL三大创新" and section NP-Map;
# [P2] excerpt; [P3] on linear attention's fixed-size state)
# --------------------------------------------------------------------------------------

def sa_mask_row(i: int, window: int, chunk: int, sel_row: np.ndarray) -> np.ndarray:
    """Softmax-set membership of keys j = 0..i for query i (bool [i+1])."""
    j = np.arange(i + 1)
    in_window = j > i - window
    selected_past = (j // chunk < i // chunk) & sel_row[: i + 1]
    return in_window | selected_past


def _check_cfg(window: int, chunk: int, top_k: int):
    if window < 0 or chunk < 1 or not (0 <= top_k <= chunk):
        raise ValueError("bad window/chunk/top_k")
    if window == 0 and top_k != 0:
        raise ValueError("a zero window has no saliency, so top_k must be 0")


def _routing(q, k, window, chunk, top_k, sel):
    B, T, _, _ = q.shape
    Hkv = k.shape[2]
    if sel is not None:
        return np.asarray(sel, dtype=bool)
    if top_k == 0:
        return np.zeros((B, Hkv, T), dtype=bool)
    s_kv, _ = saliency(q, k, window)
    return route(s_kv, chunk, top_k)[1]


def _row(qi, phiq_i, kk, vv, phik, sa, D):
    """Output of one query row given its softmax-set mask over keys 0..i."""
    a = kk @ qi / math.sqrt(D)
    la = ~sa
    M = a[sa].max() if sa.any() else 0.0
    w_sa = np.exp(a[sa] - M)
    w_la = math.exp(-M) * (phik[la] @ phiq_i)
    num = w_sa @ vv[sa] + w_la @ vv[la]
    den = w_sa.sum() + w_la.sum()
    return num / den if den > 0.0 else np.zeros(vv.shape[1])


def brute(q, k, v, w_phi, window: int, chunk: int, top_k: int, sel=None) -> np.ndarray:
    """Literal per-query form: for every (i, j <= i) decide SA or LA, then fuse.

    q [B,T,Hq,D], k/v [B,T,Hkv,D], w_phi [Hkv,d_f,D] -> out [B,T,Hq,D] fp64.
    sel [B,Hkv,T] bool overrides the saliency routing when given.
    """
    _check_cfg(window, chunk, top_k)
    q, k, v, w_phi = _f64(q), _f64(k), _f64(v), _f64(w_phi)
    B, T, Hq, D = q.shape
    G = _check_group(Hq, k.shape[2])
    sel = _routing(q, k, window, chunk, top_k, sel)
    out = np.zeros_like(q)
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            phiq = np_map(q[b, :, hq], w_phi[h])
            phik = np_map(k[b, :, h], w_phi[h])
            for i in range(T):
                sa = sa_mask_row(i, window, chunk, sel[b, h])
                out[b, i, hq] = _row(q[b, i, hq], phiq[i], k[b, : i + 1, h], v[b, : i + 1, h],
                                     phik[: i + 1], sa, D)
    return out


def brute_rows(q, k, v, w_phi, window: int, chunk: int, sel, rows) -> np.ndarray:
    """The literal per-query form for selected rows only.

    rows: iterable of (b, hq, i). Returns [len(rows), D]. sel [B,Hkv,T] bool is required
    (compute it once with saliency + route for long sequences).
    """
    q, k, v, w_phi = _f64(q), _f64(k), _f64(v), _f64(w_phi)
    _, _, Hq, D = q.shape
    G = _check_group(Hq, k.shape[2])
    sel = np.asarray(sel, dtype=bool)
    res = []
    for (b, hq, i) in rows:
        h = hq // G
        phiq_i = np_map(q[b, i, hq], w_phi[h])
        phik = np_map(k[b, : i + 1, h], w_phi[h])
        sa = sa_mask_row(i, window, chunk, sel[b, h])
        res.append(_row(q[b, i, hq], phiq_i, k[b, : i + 1, h], v[b, : i + 1, h], phik, sa, D))
    return np.array(res)


def attend(q, k, v, w_phi, window: int, chunk: int, top_k: int, sel=None,
           heads=None, return_routing: bool = False):
    """Chunk-wise form of the same layer ([P1] section "Chunk-Wise并行+延迟选择").

    Queries are taken one chunk at a time. Keys lying before the first window position of
    the chunk (j <= i0 - w) are outside every window of the chunk: the selected ones join
    the softmax set, the others are summed once into the linear-attention state
    S = sum phi(k_j) v_j^T, z = sum phi(k_j). Keys from there up to the chunk's end get a
    per-query mask. Output as in brute(); the two agree to rounding.

    heads: optional list of query-head indices to compute (others are left zero).
    Returns out [B,T,Hq,D] (and (s_kv, sel) if return_routing).
    """
    _check_cfg(window, chunk, top_k)
    q, k, v, w_phi = _f64(q), _f64(k), _f64(v), _f64(w_phi)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = _check_group(Hq, Hkv)
    F = w_phi.shape[1]
    s_kv = None
    if sel is None and top_k > 0:
        s_kv, _ = saliency(q, k, window)
        sel = route(s_kv, chunk, top_k)[1]
    elif sel is None:
        sel = np.zeros((B, Hkv, T), dtype=bool)
    sel = np.asarray(sel, dtype=bool)
    out = np.zeros_like(q)
    n_chunks = -(-T // chunk)
    inv_sqrt_d = 1.0 / math.sqrt(D)
    for b in range(B):
        for hq in (range(Hq) if heads is None else heads):
            h = hq // G
            kk, vv = k[b, :, h], v[b, :, h]
            phik = np_map(kk, w_phi[h])
            sel_h = sel[b, h]
            S = np.zeros((F, D))
            z = np.zeros(F)
            folded = 0
            for c in range(n_chunks):
                i0, i1 = c * chunk, min(T, (c + 1) * chunk)
                far_end = max(0, i0 - window + 1)  # keys [0, far_end) are out of every window
                new = np.arange(folded, far_end)
                la_new = new[~sel_h[new]]
                S += phik[la_new].T @ vv[la_new]
                z += phik[la_new].sum(axis=0)
                folded = far_end
                sa_far = np.flatnonzero(sel_h[:far_end])
                near = np.arange(far_end, i1)
                Qc = q[b, i0:i1, hq]
                phiq = np_map(Qc, w_phi[h])
                I = np.arange(i0, i1)[:, None]
                J = near[None, :]
                visible = J <= I
                sa_near = visible & ((J > I - window) | ((J // chunk < c) & sel_h[near][None, :]))
                la_near = visible & ~sa_near
                a_far = Qc @ kk[sa_far].T * inv_sqrt_d
                a_near = np.where(sa_near, Qc @ kk[near].T * inv_sqrt_d, -np.inf)
                M = np.maximum(a_far.max(axis=1, initial=-np.inf), a_near.max(axis=1, initial=-np.inf))
                M = np.where(np.isfinite(M), M, 0.0)[:, None]
                e_far = np.exp(a_far - M)
                e_near = np.where(sa_near, np.exp(a_near - M), 0.0)
                lw_near = np.where(la_near, phiq @ phik[near].T, 0.0)
                scale_la = np.exp(-M)
                num = e_far @ vv[sa_far] + e_near @ vv[near] + scale_la * (phiq @ S + lw_near @ vv[near])
                den = (e_far.sum(axis=1) + e_near.sum(axis=1))[:, None] + \
                    scale_la * ((phiq @ z) + lw_near.sum(axis=1))[:, None]
                safe = den > 0.0
                out[b, i0:i1, hq] = np.where(safe, num / np.where(safe, den, 1.0), 0.0)
    if return_routing:
        return out, s_kv, sel
    return out


# --------------------------------------------------------------------------------------
# Local-global consistency of the saliency  ([P2] excerpt: the local score is meant to
# predict whether a token will still be attended once it is far history, with a reported
# overlap; [P1] section "Self-Saliency Score": selection accuracy close to global attention)
# --------------------------------------------------------------------------------------

def future_attention_mass(q, k, window: int, q_from: int = 0):
    """Attention each key receives from far-future queries under full causal softmax.

    For KV head h and key j: F_j = sum over the group's query heads g and over queries
    i >= j + max(window, 0) (j is outside i's window, i.e. far history for i) of
    p_ij = e^{a_ij} / sum_{l <= i} e^{a_il}, a_ij = q_i . k_j / sqrt(D).
    q_from: only queries i >= q_from are summed (the values of keys j >= q_from - window
    are then exact). Returns F [B, Hkv, T] fp64.
    """
    q, k = _f64(q), _f64(k)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = _check_group(Hq, Hkv)
    w = max(window, 0)
    F = np.zeros((B, Hkv, T))
    i = np.arange(q_from, T)[:, None]
    j = np.arange(T)[None, :]
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            a = q[b, q_from:, hq] @ k[b, :, h].T / math.sqrt(D)
            a = np.where(j <= i, a, -np.inf)
            p = np.exp(a - lse(a, axis=1)[:, None])
            F[b, h] += np.where(i >= j + w, p, 0.0).sum(axis=0)
    return F


def selection_overlap(sel_a, sel_b) -> np.ndarray:
    """Tokens two per-chunk selections have in common: sel_a, sel_b [B, Hkv, nC, k]
    -> counts [B, Hkv, nC]."""
    sel_a, sel_b = np.asarray(sel_a), np.asarray(sel_b)
    out = np.zeros(sel_a.shape[:3], dtype=np.int64)
    for idx in np.ndindex(*sel_a.shape[:3]):
        out[idx] = len(set(sel_a[idx].tolist()) & set(sel_b[idx].tolist()))
    return out


# --------------------------------------------------------------------------------------
# Backward pass with the routing held fixed  ([P1] section "Chunk-Wise并行+延迟选择" and
# [P4] section Approach: the same chunked layer is used for training)
# --------------------------------------------------------------------------------------

def _np_map_t(x, w):
    """NP-Map in torch fp64 (the same definition as np_map), for automatic differentiation."""
    import torch
    z = x @ w.T
    m = torch.where(z > 0.0, z + 1.0, torch.exp(torch.clamp(z, max=0.0)))
    return torch.linalg.vector_norm(x, dim=-1, keepdim=True) * m / torch.linalg.vector_norm(m, dim=-1, keepdim=True)


def attend_backward(q, k, v, w_phi, window: int, chunk: int, sel, dout, q_from: int = 0, rows=None):
    """Gradients of sum(out * dout) with respect to q, k, v and w_phi, for a fixed routing.

    The routing sel [B,Hkv,T] (bool) is an input: it is piecewise constant in q and k, so
    it contributes no gradient. The layer is written in its dense form (the SA and LA masks
    of every (i, j) pair, as in brute) with plain torch fp64 ops, and torch's reverse-mode
    differentiation takes the chain rule through the shared normaliser, both branches and
    the NP-Map. Rows whose normaliser is 0 have out = 0 and contribute nothing.
    q_from: only query rows i >= q_from enter the sum. Query row i affects out_i alone and key
    j only the rows i >= j, so the gradients of q rows and of k, v rows at positions >= q_from
    are then the full ones (the others are partial): a long sequence can be checked at its
    tail for the cost of its last rows.
    rows: alternatively, the query positions (distinct) whose rows enter the sum, in place of
    q_from. Where dout is zero on every other row, these are the whole loss, and every
    gradient returned (dq, dk, dv and dw_phi at every position) is the full one.
    Returns (dq, dk, dv, dw_phi) as fp64 arrays shaped like q, k, v and w_phi.
    """
    import torch
    _check_cfg(window, chunk, 0)
    qt, kt, vt, wt = (torch.tensor(_f64(x), requires_grad=True) for x in (q, k, v, w_phi))
    do = torch.tensor(_f64(dout))
    B, T, Hq, D = qt.shape
    G = _check_group(Hq, kt.shape[2])
    sel = torch.tensor(np.asarray(sel, dtype=bool))
    if rows is None:
        ridx = torch.arange(q_from, T)
    else:
        ridx = torch.tensor(np.asarray(rows, dtype=np.int64).reshape(-1))
        if ridx.numel() and (int(ridx.min()) < 0 or int(ridx.max()) >= T or ridx.unique().numel() != ridx.numel()):
            raise ValueError("rows must be distinct positions in [0, seq_len)")
    i = ridx[:, None]
    j = torch.arange(T)[None, :]
    causal = j <= i
    in_window = j > i - window
    earlier_chunk = (j // chunk) < (i // chunk)
    loss = torch.zeros((), dtype=torch.float64)
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            sa = causal & (in_window | (earlier_chunk & sel[b, h][None, :]))
            la = causal & ~sa
            qq, kk, vv = qt[b, ridx, hq], kt[b, :, h], vt[b, :, h]
            a = torch.where(sa, qq @ kk.T / math.sqrt(D), -math.inf)
            M = a.detach().amax(dim=1, keepdim=True)
            M = torch.where(torch.isfinite(M), M, torch.zeros_like(M))
            e_sa = torch.exp(a - M)
            lw = torch.where(la, _np_map_t(qq, wt[h]) @ _np_map_t(kk, wt[h]).T, 0.0) * torch.exp(-M)
            wgt = e_sa + lw
            den = wgt.sum(dim=1, keepdim=True)
            safe = den > 0.0
            o = torch.where(safe, (wgt @ vv) / torch.where(safe, den, torch.ones_like(den)), 0.0)
            loss = loss + (o * do[b, ridx, hq]).sum()
    loss.backward()
    return tuple(t.grad.numpy() for t in (qt, kt, vt, wt))


# --------------------------------------------------------------------------------------
# Decode with chunk-granular delayed selection  ([P1] section "Chunk-Wise并行+延迟选择";
# [P4] section Approach; [P3] on the fixed-size state of linear attention)
# --------------------------------------------------------------------------------------

class DecodeOracle:
    """Token-by-token replay of the layer with an explicit decode state.

    With L = max(1, ceil((window - 1) / chunk)) earlier chunks kept raw (every key of a
    token's window lies in them or in its own chunk), the state per (batch, KV head) for a
    token of chunk c is: a compact list of the selected tokens of chunks <= c-L-1 (the
    softmax cache), the raw keys/values of chunks c-L .. c (the ring), the selections of
    chunks c-L .. c-1, the running saliency of chunk c, and the linear-attention state
    (S, z) of every unselected token of chunks <= c-L-1. When chunk c completes, its top_k
    tokens are chosen, and chunk c-L is folded: its selected rows join the cache, the rest
    join (S, z). Needs window >= 1 (or window = 0 with top_k = 0).
    """

    def __init__(self, w_phi, n_q_heads: int, window: int, chunk: int, top_k: int):
        _check_cfg(window, chunk, top_k)
        self.w = _f64(w_phi)
        self.Hkv, self.F, self.D = self.w.shape
        self.Hq = n_q_heads
        self.G = _check_group(n_q_heads, self.Hkv)
        self.window, self.chunk, self.top_k = window, chunk, top_k
        self.L = max(1, -(-(window - 1) // chunk)) if window >= 1 else 1
        self.B = None
        self.t = 0

    def _init(self, B):
        H, D, F, C, L = self.Hkv, self.D, self.F, self.chunk, self.L
        self.B = B
        self.cache_k = [[np.zeros((0, D)) for _ in range(H)] for _ in range(B)]
        self.cache_v = [[np.zeros((0, D)) for _ in range(H)] for _ in range(B)]
        self.S = np.zeros((B, H, F, D))
        self.z = np.zeros((B, H, F))
        self.ring_k = np.zeros((B, H, L + 1, C, D))  # slot l holds chunk c - L + l
        self.ring_v = np.zeros((B, H, L + 1, C, D))
        self.ring_sel = np.zeros((B, H, L, C), dtype=bool)  # selections of chunks c-L .. c-1
        self.cur_s = np.zeros((B, H, C))
        self.sel_idx = []  # per completed chunk: [B,H,top_k] absolute positions

    def step(self, q_t, k_t, v_t) -> np.ndarray:
        """q_t [B,Hq,D], k_t/v_t [B,Hkv,D] for token i = self.t -> out [B,Hq,D]."""
        q_t, k_t, v_t = _f64(q_t), _f64(k_t), _f64(v_t)
        B = q_t.shape[0]
        if self.B is None:
            self._init(B)
        C, w, D, G, L = self.chunk, self.window, self.D, self.G, self.L
        i = self.t
        c, r = divmod(i, C)
        self.ring_k[:, :, L, r] = k_t
        self.ring_v[:, :, L, r] = v_t
        out = np.zeros((B, self.Hq, D))
        inv = 1.0 / math.sqrt(D)
        # ring keys in position order (chunks that exist, the current one up to i), their
        # positions, and which are selected tokens of earlier chunks
        slots = [l for l in range(L + 1) if c - L + l >= 0]
        pos = np.concatenate([(c - L + l) * C + np.arange(C if l < L else r + 1) for l in slots])
        for b in range(B):
            for h in range(self.Hkv):
                W = self.w[h]
                rk = np.concatenate([self.ring_k[b, h, l, : (C if l < L else r + 1)] for l in slots])
                rv = np.concatenate([self.ring_v[b, h, l, : (C if l < L else r + 1)] for l in slots])
                rsel = np.concatenate([self.ring_sel[b, h, l] if l < L else np.zeros(r + 1, dtype=bool)
                                       for l in slots])
                in_window = pos > i - w
                sa = in_window | rsel
                ck, cv = self.cache_k[b][h], self.cache_v[b][h]
                s_sum = 0.0
                for g in range(G):
                    qv = q_t[b, h * G + g]
                    # saliency of token i over its window (all inside the ring)
                    if w >= 1:
                        logits = rk[in_window] @ qv * inv  # the last entry is token i itself
                        rest = logits[:-1]
                        s_sum += lse(logits) - (lse(rest) if rest.size else -np.inf)
                    phiq = np_map(qv, W)
                    keys_sa = np.concatenate([ck, rk[sa]])
                    vals_sa = np.concatenate([cv, rv[sa]])
                    keys_la, vals_la = rk[~sa], rv[~sa]
                    a = keys_sa @ qv * inv
                    M = a.max() if a.size else 0.0
                    e = np.exp(a - M)
                    lw = np_map(keys_la, W) @ phiq if keys_la.size else np.zeros(0)
                    num = e @ vals_sa + math.exp(-M) * (phiq @ self.S[b, h] + lw @ vals_la)
                    den = e.sum() + math.exp(-M) * (phiq @ self.z[b, h] + lw.sum())
                    out[b, h * G + g] = num / den if den > 0.0 else 0.0
                self.cur_s[b, h, r] = s_sum
        self.t += 1
        if r == C - 1:
            self._complete_chunk(c)
        return out

    def _complete_chunk(self, c: int):
        C, k, L = self.chunk, self.top_k, self.L
        B, H = self.B, self.Hkv
        # fold chunk c-L: selected rows -> softmax cache, the rest -> (S, z)
        if c - L >= 0:
            for b in range(B):
                for h in range(H):
                    sel = self.ring_sel[b, h, 0]
                    pk, pv = self.ring_k[b, h, 0], self.ring_v[b, h, 0]
                    self.cache_k[b][h] = np.concatenate([self.cache_k[b][h], pk[sel]])
                    self.cache_v[b][h] = np.concatenate([self.cache_v[b][h], pv[sel]])
                    phik = np_map(pk[~sel], self.w[h])
                    self.S[b, h] += phik.T @ pv[~sel]
                    self.z[b, h] += phik.sum(axis=0)
        # select the top_k of chunk c by its saliency
        idx = np.arange(C)
        new_sel = np.zeros((B, H, C), dtype=bool)
        picks = np.zeros((B, H, k), dtype=np.int64)
        for b in range(B):
            for h in range(H):
                order = np.lexsort((idx, -self.cur_s[b, h]))
                pick = np.sort(order[:k])
                new_sel[b, h, pick] = True
                picks[b, h] = pick + c * C
        self.sel_idx.append(picks)
        # rotate: chunk c - L + l + 1 moves to slot l; slot L takes the next chunk
        self.ring_k[:, :, :L] = self.ring_k[:, :, 1:].copy()
        self.ring_v[:, :, :L] = self.ring_v[:, :, 1:].copy()
        self.ring_k[:, :, L] = 0.0
        self.ring_v[:, :, L] = 0.0
        self.ring_sel[:, :, : L - 1] = self.ring_sel[:, :, 1:].copy()
        self.ring_sel[:, :, L - 1] = new_sel
        self.cur_s[:] = 0.0
