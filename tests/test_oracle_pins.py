"""Pins of the fp64 oracle against closed forms, library routines and hand-derived cases.

Nothing here compares the oracle with itself: each check uses a different route to the
same number (an explicit KL sum, torch's SDPA / ELU in fp64, a dense textbook linear
attention, brute-force subset search, or an output worked out by hand).
"""

import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import still_oracle as O

RNG = np.random.default_rng(12345)


def _rand(*shape, scale=1.0, rng=RNG):
    return rng.standard_normal(shape) * scale


# ----------------------------------------------------------------------------- lse

def test_lse_matches_scipy():
    a = _rand(7, 13, scale=5.0)
    np.testing.assert_allclose(O.lse(a, axis=1), scipy.special.logsumexp(a, axis=1), rtol=0, atol=1e-12)
    b = np.full((3, 4), -np.inf)
    assert np.all(O.lse(b, axis=1) == -np.inf)


# ----------------------------------------------------------------------------- saliency

@pytest.mark.parametrize("window", [2, 3, 8, 16])
def test_saliency_equals_explicit_kl_sum(window):
    """s_i = sum_j qbar_j log(qbar_j / p_j): KL between the window softmax without and
    with the diagonal, summed term by term over the window."""
    T, D = 24, 8
    q = _rand(1, T, 1, D, scale=1.5)
    k = _rand(1, T, 1, D, scale=1.5)
    _, s_q = O.saliency(q, k, window)
    for i in range(T):
        lo = max(0, i - window + 1)
        a = np.array([q[0, i, 0] @ k[0, j, 0] / math.sqrt(D) for j in range(lo, i + 1)])
        if len(a) == 1:
            assert s_q[0, 0, i] == np.inf
            continue
        p = np.exp(a) / np.exp(a).sum()
        qbar = np.exp(a[:-1]) / np.exp(a[:-1]).sum()
        kl = float(np.sum(qbar * np.log(qbar / p[:-1])))
        assert abs(s_q[0, 0, i] - kl) < 1e-12
        # and the one-line closed form -log(1 - p_ii)
        assert abs(s_q[0, 0, i] + math.log1p(-p[-1])) < 1e-12


def test_saliency_special_values():
    """Equal logits (q = 0): a window of n tokens gives log(n/(n-1)); one token gives +inf."""
    T, D, w = 20, 4, 6
    q = np.zeros((1, T, 1, D))
    k = _rand(1, T, 1, D)
    _, s = O.saliency(q, k, w)
    for i in range(T):
        n = min(i + 1, w)
        want = np.inf if n == 1 else math.log(n / (n - 1))
        assert s[0, 0, i] == want or abs(s[0, 0, i] - want) < 1e-14
    _, s1 = O.saliency(_rand(1, T, 1, D), k, 1)
    assert np.all(np.isinf(s1)) and np.all(s1 > 0)


def test_saliency_dominant_diagonal():
    """A token whose own logit dwarfs the others has s close to a_ii - LSE(rest)."""
    D, w = 4, 4
    k = _rand(1, 8, 1, D, scale=0.1)
    q = _rand(1, 8, 1, D, scale=0.1)
    k[0, 6, 0] = np.array([10.0, 0, 0, 0])
    q[0, 6, 0] = np.array([10.0, 0, 0, 0])  # a_66 = 100/2 = 50
    _, s = O.saliency(q, k, w)
    rest = np.array([q[0, 6, 0] @ k[0, j, 0] / 2.0 for j in (3, 4, 5)])
    assert abs(s[0, 0, 6] - (50.0 - scipy.special.logsumexp(rest))) < 1e-9


def test_saliency_group_sum_and_identical_heads():
    B, T, D, G = 2, 30, 8, 3
    q1 = _rand(B, T, 1, D)
    k = _rand(B, T, 1, D)
    q = np.repeat(q1, G, axis=2)
    s_kv, s_q = O.saliency(q, k, 5)
    s_single, _ = O.saliency(q1, k, 5)
    np.testing.assert_allclose(s_kv, G * s_single, rtol=1e-14, atol=0)
    # identical heads route exactly like the single head (scaling keeps the order)
    a = O.route(s_kv, 10, 3)[0]
    b = O.route(s_single, 10, 3)[0]
    assert np.array_equal(a, b)


def test_diagonal_score_brute_force_and_group_sum():
    """The diagonal-logit routing score: an explicit per-token dot product (math.fsum over
    the head dimension), and the sum over identical heads of a group."""
    B, T, Hq, Hkv, D = 1, 9, 4, 2, 5
    q = _rand(B, T, Hq, D)
    k = _rand(B, T, Hkv, D)
    s_kv, s_q = O.diagonal_score(q, k)
    G = Hq // Hkv
    for hq in range(Hq):
        for i in range(T):
            want = math.fsum(q[0, i, hq, d] * k[0, i, hq // G, d] for d in range(D)) / math.sqrt(D)
            assert abs(s_q[0, hq, i] - want) < 1e-14
    q1 = _rand(B, T, 1, D)
    s_rep, _ = O.diagonal_score(np.repeat(q1, 3, axis=2), k[:, :, :1])
    s_one, _ = O.diagonal_score(q1, k[:, :, :1])
    np.testing.assert_allclose(s_rep, 3 * s_one, rtol=1e-14, atol=0)


def test_diagonal_score_against_saliency_closed_form():
    """With a window of two tokens and every query orthogonal to the previous key, the
    saliency is -log(1 - p_ii) = softplus(a_ii - 0): a monotone function of the diagonal
    logit, so the two scores agree through that closed form (and route alike)."""
    T, D = 65, 2
    x, y = _rand(T), _rand(T)
    q = np.zeros((1, T, 1, D))
    k = np.zeros((1, T, 1, D))
    for i in range(T):  # token i lives in dimension i % 2 only
        q[0, i, 0, i % 2] = 3.0 * x[i]
        k[0, i, 0, i % 2] = y[i]
    s, _ = O.saliency(q, k, 2)
    d, _ = O.diagonal_score(q, k)
    np.testing.assert_allclose(s[0, 0, 1:], np.logaddexp(0.0, d[0, 0, 1:]), rtol=1e-12, atol=1e-15)
    assert math.isinf(s[0, 0, 0])  # a one-token window
    # positions 1..64 as one chunk: both scores pick the same five
    assert np.array_equal(O.route(s[:, :, 1:], 64, 5)[0], O.route(d[:, :, 1:], 64, 5)[0])


# ----------------------------------------------------------------------------- routing

def _brute_topk(seg, k):
    """The unique subset whose every member beats every non-member on (s, -index)."""
    n = len(seg)
    found = []
    for sub in itertools.combinations(range(n), k):
        rest = [j for j in range(n) if j not in sub]
        if all((seg[a] > seg[r]) or (seg[a] == seg[r] and a < r) for a in sub for r in rest):
            found.append(sub)
    assert len(found) == 1
    return list(found[0])


@pytest.mark.parametrize("k", [0, 1, 2, 3, 6])
def test_route_equals_bruteforce_subset_search(k):
    C = 6
    rng = np.random.default_rng(7 + k)
    s = rng.integers(0, 4, size=(2, 3, 20)).astype(float)  # many ties
    s[0, 0, 3] = np.inf
    s[1, 2, 7] = np.inf
    s[1, 2, 8] = np.inf
    sel_idx, sel = O.route(s, C, k)
    assert sel_idx.shape == (2, 3, 3, k)
    for b in range(2):
        for h in range(3):
            for c in range(3):
                want = [c * C + j for j in _brute_topk(s[b, h, c * C:(c + 1) * C], k)]
                assert list(sel_idx[b, h, c]) == want
            assert not sel[b, h, 18:].any()  # incomplete chunk never selected
            assert sel[b, h].sum() == 3 * k


def test_route_margins():
    s = np.array([[[5.0, 1.0, 3.0, 3.0, 0.0, 2.0, np.inf, np.inf]]])
    m = O.route_margins(s, 4, 2)
    assert m[0, 0, 0] == 0.0  # 3 vs 3 tie at the boundary
    assert m[0, 0, 1] == np.inf  # both infinities selected, the next is finite
    m1 = O.route_margins(s, 4, 1)
    assert m1[0, 0, 0] == 2.0 and m1[0, 0, 1] == 0.0  # inf vs inf tie


# ----------------------------------------------------------------------------- NP-Map

def test_np_map_invariants():
    x = _rand(50, 16, scale=3.0)
    w = _rand(24, 16, scale=0.4)
    phi = O.np_map(x, w)
    np.testing.assert_allclose(np.linalg.norm(phi, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    assert np.all(phi >= 0)
    assert np.all(O.np_map(np.zeros((3, 16)), w) == 0.0)
    # W = 0: m = 1 everywhere, so phi(x) = |x|/sqrt(d_f) * 1 and phi(q).phi(k) = |q||k|
    phi0 = O.np_map(x, np.zeros((24, 16)))
    np.testing.assert_allclose(phi0, np.linalg.norm(x, axis=1, keepdims=True) / math.sqrt(24) * np.ones((1, 24)),
                               rtol=1e-14)


def test_np_map_direction_uses_library_elu():
    """Direction of phi equals the direction of torch's ELU(Wx) + 1 (alpha = 1)."""
    x = _rand(40, 8, scale=2.0)
    w = _rand(12, 8)
    m = torch.nn.functional.elu(torch.from_numpy(x @ w.T), alpha=1.0).numpy() + 1.0
    phi = O.np_map(x, w)
    want = m / np.linalg.norm(m, axis=1, keepdims=True) * np.linalg.norm(x, axis=1, keepdims=True)
    np.testing.assert_allclose(phi, want, rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------------------- special cases

def _case(B, T, Hq, Hkv, D, F, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hq, D)) * scale
    k = rng.standard_normal((B, T, Hkv, D)) * scale
    v = rng.standard_normal((B, T, Hkv, D))
    w = rng.standard_normal((Hkv, F, D)) / math.sqrt(D)
    return q, k, v, w


def _sdpa_causal(q, k, v):
    """torch SDPA (fp64, CPU, is_causal) with KV heads expanded for GQA."""
    B, T, Hq, D = q.shape
    G = Hq // k.shape[2]
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(np.repeat(k, G, axis=2)).permute(0, 2, 1, 3)
    tv = torch.from_numpy(np.repeat(v, G, axis=2)).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("T,C", [(40, 8), (37, 8), (5, 8)])
def test_topk_chunk_reduces_to_causal_softmax(T, C):
    q, k, v, w = _case(2, T, 4, 2, 8, 6, seed=T)
    want = _sdpa_causal(q, k, v)
    for fn in (O.brute, O.attend):
        got = fn(q, k, v, w, window=C, chunk=C, top_k=C)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # a window covering the whole sequence does the same with no selection
    got = O.attend(q, k, v, w, window=T, chunk=C, top_k=0)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def _textbook_causal_la(q, k, v, w):
    B, T, Hq, D = q.shape
    G = Hq // k.shape[2]
    out = np.zeros_like(q)
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            pq = O.np_map(q[b, :, hq], w[h])
            pk = O.np_map(k[b, :, h], w[h])
            A = np.tril(pq @ pk.T)
            out[b, :, hq] = (A @ v[b, :, h]) / A.sum(axis=1, keepdims=True)
    return out


@pytest.mark.parametrize("T,C", [(33, 8), (16, 16)])
def test_zero_window_zero_topk_is_causal_linear_attention(T, C):
    q, k, v, w = _case(1, T, 2, 1, 8, 12, seed=3)
    want = _textbook_causal_la(q, k, v, w)
    for fn in (O.brute, O.attend):
        np.testing.assert_allclose(fn(q, k, v, w, window=0, chunk=C, top_k=0), want, rtol=0, atol=1e-12)


def test_constant_values_and_linearity():
    q, k, v, w = _case(1, 45, 2, 1, 8, 8, seed=9)
    const = np.broadcast_to(np.arange(8.0), v.shape).copy()
    out = O.attend(q, k, const, w, window=4, chunk=8, top_k=2)
    np.testing.assert_allclose(out, np.broadcast_to(np.arange(8.0), out.shape), atol=1e-12)
    v2 = np.random.default_rng(1).standard_normal(v.shape)
    o1 = O.attend(q, k, v, w, 4, 8, 2)
    o2 = O.attend(q, k, v2, w, 4, 8, 2)
    o12 = O.attend(q, k, v + 2 * v2, w, 4, 8, 2)
    np.testing.assert_allclose(o12, o1 + 2 * o2, atol=1e-12)


def test_hand_case_shared_normaliser():
    """T=2, window 1, no complete chunk. W = 0 makes phi(q).phi(k) = |q||k|.
    Query 1: softmax set {1} with a_11 = ln 2 + 3, linear set {0} with |q1||k0| = e^3.
    With M = a_11 the weights are 1 (softmax) and e^3 e^-M = 1/2 (linear), so
    o_1 = (v_1 + v_0/2) / (3/2) = (2 v_1 + v_0) / 3; query 0 sees only itself: o_0 = v_0."""
    D, F = 4, 3
    a11 = math.log(2.0) + 3.0
    k1 = np.array([1.0, 0, 0, 0])
    q1 = np.array([2.0 * a11, 0, 0, 0])  # q1.k1 / sqrt(4) = a11
    k0 = np.array([0, math.exp(3.0) / np.linalg.norm(q1), 0, 0])
    q0 = np.array([0.3, -0.2, 0.1, 0.5])
    q = np.stack([q0, q1])[None, :, None, :]
    k = np.stack([k0, k1])[None, :, None, :]
    v = np.array([[1.0, 2.0, 3.0, 4.0], [-1.0, 0.5, 7.0, 2.0]])[None, :, None, :]
    w = np.zeros((1, F, D))
    for fn in (O.brute, O.attend):
        out = fn(q, k, v, w, window=1, chunk=4, top_k=0)
        np.testing.assert_allclose(out[0, 1, 0], (2 * v[0, 1, 0] + v[0, 0, 0]) / 3, atol=1e-13)
        np.testing.assert_allclose(out[0, 0, 0], v[0, 0, 0], atol=1e-15)


def test_hand_case_delayed_selection():
    """Chunk 2, window 1, top_k 1, q = 0 (so every softmax weight is 1 and every linear
    weight phi(0).phi(k) is 0). Window 1 makes every saliency +inf, so ties pick the first
    token of each chunk: 0 and 2. Worked by hand from the partition rule:
      o_0 = v0, o_1 = v1 (chunk 0's choice only helps later chunks),
      o_2 = (v2 + v0)/2, o_3 = (v3 + v0)/2 (token 2 is in the query's own chunk),
      o_4 = (v4 + v0 + v2)/3."""
    T, D = 5, 4
    rng = np.random.default_rng(5)
    q = np.zeros((1, T, 1, D))
    k = rng.standard_normal((1, T, 1, D))
    v = rng.standard_normal((1, T, 1, D))
    w = rng.standard_normal((1, 6, D))
    V = v[0, :, 0]
    want = np.stack([V[0], V[1], (V[2] + V[0]) / 2, (V[3] + V[0]) / 2, (V[4] + V[0] + V[2]) / 3])
    for fn in (O.brute, O.attend):
        np.testing.assert_allclose(fn(q, k, v, w, window=1, chunk=2, top_k=1)[0, :, 0], want, atol=1e-14)
    dec = O.DecodeOracle(w, 1, 1, 2, 1)
    outs = np.stack([dec.step(q[:, t], k[:, t], v[:, t]) for t in range(T)])
    np.testing.assert_allclose(outs[:, 0, 0], want, atol=1e-14)


def test_empty_softmax_set_zero_query():
    """window 0 and top_k 0 with q = 0: the denominator is 0 and the output is defined as 0."""
    q, k, v, w = _case(1, 10, 1, 1, 4, 4, seed=2)
    q[0, 3, 0] = 0.0
    for fn in (O.brute, O.attend):
        out = fn(q, k, v, w, window=0, chunk=4, top_k=0)
        assert np.all(out[0, 3, 0] == 0.0)
        assert np.all(np.isfinite(out))


# ----------------------------------------------------------------------------- forms agree

@pytest.mark.parametrize("T,Hq,Hkv,w,C,k", [
    (64, 2, 1, 8, 8, 2), (61, 4, 2, 8, 8, 3), (50, 2, 2, 3, 8, 1), (40, 1, 1, 1, 8, 4),
    (45, 3, 1, 12, 8, 2), (30, 2, 1, 8, 8, 8), (7, 2, 1, 8, 8, 2), (1, 2, 1, 4, 4, 1),
    # windows longer than a chunk: one key past it, two chunks, past two chunks
    (40, 2, 1, 9, 8, 1), (52, 2, 1, 16, 8, 2), (60, 2, 1, 17, 8, 3),
])
def test_chunked_equals_brute(T, Hq, Hkv, w, C, k):
    q, k_, v, wp = _case(2, T, Hq, Hkv, 8, 6, seed=T + k, scale=1.7)
    a = O.attend(q, k_, v, wp, w, C, k)
    b = O.brute(q, k_, v, wp, w, C, k)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_brute_rows_match_brute():
    q, k, v, w = _case(1, 40, 2, 1, 8, 8, seed=4, scale=1.5)
    s_kv, _ = O.saliency(q, k, 8)
    _, sel = O.route(s_kv, 8, 2)
    full = O.brute(q, k, v, w, 8, 8, 2, sel=sel)
    rows = [(0, 1, 39), (0, 0, 17), (0, 1, 0)]
    got = O.brute_rows(q, k, v, w, 8, 8, sel, rows)
    for r, (b, hq, i) in enumerate(rows):
        np.testing.assert_allclose(got[r], full[b, i, hq], atol=1e-14)


@pytest.mark.parametrize("T,w,C,k,G", [(70, 8, 8, 2, 2), (33, 4, 8, 3, 1), (24, 8, 8, 8, 1), (20, 0, 8, 0, 2),
                                       (61, 12, 8, 2, 2), (50, 16, 8, 3, 1), (45, 9, 8, 8, 1), (40, 20, 8, 2, 1)])
def test_decode_replay_equals_prefill(T, w, C, k, G):
    q, k_, v, wp = _case(2, T, G, 1, 8, 6, seed=11, scale=1.5)
    want, s_kv, sel = O.attend(q, k_, v, wp, w, C, k, return_routing=True)
    dec = O.DecodeOracle(wp, G, w, C, k)
    outs = np.stack([dec.step(q[:, t], k_[:, t], v[:, t]) for t in range(T)], axis=1)
    np.testing.assert_allclose(outs, want, rtol=0, atol=1e-12)
    if k > 0:
        got_idx = np.stack(dec.sel_idx, axis=2) if dec.sel_idx else np.zeros((2, 1, 0, k))
        want_idx = O.route(s_kv, C, k)[0]
        assert np.array_equal(got_idx, want_idx)


# ----------------------------------------------------------------------------- backward

def _fixed_routing(q, k, w, C, top_k, B, Hkv, T):
    if top_k == 0:
        return np.zeros((B, Hkv, T), dtype=bool)
    s_kv, _ = O.saliency(q, k, w)
    return O.route(s_kv, C, top_k)[1]


@pytest.mark.parametrize("T,Hq,Hkv,w,C,k", [(37, 2, 1, 8, 8, 2), (20, 2, 2, 0, 8, 0), (30, 4, 2, 3, 8, 3),
                                            (26, 2, 1, 8, 8, 8)])
def test_backward_matches_finite_differences(T, Hq, Hkv, w, C, k):
    """attend_backward (torch reverse mode over the dense form) against central differences
    of attend (the chunked NumPy form) at random coordinates of every input."""
    q, k_, v, wp = _case(1, T, Hq, Hkv, 8, 6, seed=T + w, scale=1.5)
    sel = _fixed_routing(q, k_, w, C, k, 1, Hkv, T)
    dout = np.random.default_rng(T).standard_normal(q.shape)
    grads = O.attend_backward(q, k_, v, wp, w, C, sel, dout)
    inputs = [q, k_, v, wp]
    rng = np.random.default_rng(w + 100 * k)
    h = 1e-5

    def loss(xs):
        return float(np.sum(O.attend(*xs, w, C, k, sel=sel) * dout))

    for t, (x, g) in enumerate(zip(inputs, grads)):
        assert g.shape == x.shape
        for _ in range(6):
            idx = tuple(int(rng.integers(n)) for n in x.shape)
            plus = [a.copy() for a in inputs]
            minus = [a.copy() for a in inputs]
            plus[t][idx] += h
            minus[t][idx] -= h
            fd = (loss(plus) - loss(minus)) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-7 * (1.0 + abs(fd)), (t, idx, fd, g[idx])


def test_backward_value_gradients_sum_to_output_gradients():
    """Every row's weights sum to 1, so the value gradients of a KV head sum (over
    positions) to the output gradients of its query heads, exactly."""
    T, Hq, Hkv, w, C, k = 45, 4, 2, 8, 8, 2
    q, k_, v, wp = _case(2, T, Hq, Hkv, 8, 6, seed=5, scale=1.5)
    sel = _fixed_routing(q, k_, w, C, k, 2, Hkv, T)
    dout = np.random.default_rng(1).standard_normal(q.shape)
    _, _, dv, _ = O.attend_backward(q, k_, v, wp, w, C, sel, dout)
    G = Hq // Hkv
    want = dout.reshape(2, T, Hkv, G, 8).sum(axis=(1, 3))
    np.testing.assert_allclose(dv.sum(axis=1), want, rtol=0, atol=1e-10)


def test_backward_reduces_to_causal_softmax_gradients():
    """With window = chunk = top_k every past token is in the softmax set: the gradients are
    those of causal softmax attention (torch SDPA, fp64), and the NP-Map gets none."""
    T, Hq, Hkv, C = 29, 4, 2, 8
    q, k_, v, wp = _case(1, T, Hq, Hkv, 8, 6, seed=8, scale=1.5)
    sel = np.ones((1, Hkv, T), dtype=bool)
    dout = np.random.default_rng(2).standard_normal(q.shape)
    dq, dk, dv, dw = O.attend_backward(q, k_, v, wp, C, C, sel, dout)
    G = Hq // Hkv
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k_, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(0, 2, 1, 3), tk.repeat_interleave(G, dim=2).permute(0, 2, 1, 3),
        tv.repeat_interleave(G, dim=2).permute(0, 2, 1, 3), is_causal=True)
    (o.permute(0, 2, 1, 3) * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)
    assert np.all(dw == 0.0)


def test_backward_tail_rows_equal_full_gradients():
    """attend_backward(q_from=t0) gives the full gradients of q, k and v rows at t0 and after."""
    T, Hq, Hkv, w, C, k = 40, 2, 1, 8, 8, 2
    q, k_, v, wp = _case(1, T, Hq, Hkv, 8, 6, seed=12, scale=1.5)
    sel = _fixed_routing(q, k_, w, C, k, 1, Hkv, T)
    dout = np.random.default_rng(3).standard_normal(q.shape)
    full = O.attend_backward(q, k_, v, wp, w, C, sel, dout)
    tail = O.attend_backward(q, k_, v, wp, w, C, sel, dout, q_from=27)
    for a, b in zip(full[:3], tail[:3]):
        np.testing.assert_allclose(b[:, 27:], a[:, 27:], rtol=0, atol=1e-12)
    assert np.abs(tail[1][:, :27]).max() > 0  # earlier keys get only part of their gradient


def test_backward_row_list_equals_masked_output_gradient():
    """attend_backward(rows=R) equals the full-loss gradients when dout is zero outside the
    rows R (rows unsorted, with gaps, the first and the last among them): every gradient is
    then exact at every position, dW included."""
    T, Hq, Hkv, w, C, k = 43, 4, 2, 8, 8, 3
    q, k_, v, wp = _case(1, T, Hq, Hkv, 8, 6, seed=14, scale=1.5)
    sel = _fixed_routing(q, k_, w, C, k, 1, Hkv, T)
    rows = np.array([30, 0, 17, 42, 9, 8, 25])
    dout = np.random.default_rng(4).standard_normal(q.shape)
    masked = np.zeros_like(dout)
    masked[:, rows] = dout[:, rows]
    full = O.attend_backward(q, k_, v, wp, w, C, sel, masked)
    part = O.attend_backward(q, k_, v, wp, w, C, sel, dout, rows=rows)
    for a, b in zip(full, part):
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)
    assert np.all(part[0][:, np.setdiff1d(np.arange(T), rows)] == 0.0)
    assert np.abs(part[1]).max() > 0 and np.abs(part[3]).max() > 0
    with pytest.raises(ValueError):
        O.attend_backward(q, k_, v, wp, w, C, sel, dout, rows=[3, 3])


# ----------------------------------------------------------------------------- local-global consistency

def test_future_attention_mass_brute_force():
    """Double loop over (query, key) with explicit softmax rows."""
    T, Hq, Hkv, D, w = 11, 4, 2, 8, 3
    q, k, _, _ = _case(1, T, Hq, Hkv, D, 4, seed=21, scale=1.3)
    got = O.future_attention_mass(q, k, w)
    want = np.zeros((1, Hkv, T))
    for hq in range(Hq):
        h = hq // (Hq // Hkv)
        for i in range(T):
            logits = [float(np.dot(q[0, i, hq], k[0, j, h])) / math.sqrt(D) for j in range(i + 1)]
            zs = sum(math.exp(x) for x in logits)
            for j in range(i + 1):
                if i - j >= w:
                    want[0, h, j] += math.exp(logits[j]) / zs
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_future_attention_mass_uniform_closed_form():
    """q = 0 makes every causal row uniform, p_ij = 1/(i+1), so F_j = G (H_T - H_{j+w}) with
    H_n the harmonic numbers."""
    T, Hq, Hkv, w = 40, 3, 1, 5
    _, k, _, _ = _case(1, T, Hq, Hkv, 8, 4, seed=2)
    q = np.zeros((1, T, Hq, 8))
    got = O.future_attention_mass(q, k, w)[0, 0]
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, T + 1))])
    want = np.array([Hq * (H[T] - H[min(j + w, T)]) for j in range(T)])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_future_attention_mass_tail_rows():
    T, w = 30, 4
    q, k, _, _ = _case(1, T, 2, 1, 8, 4, seed=6, scale=1.5)
    full = O.future_attention_mass(q, k, w)
    tail = O.future_attention_mass(q, k, w, q_from=20)
    np.testing.assert_allclose(tail[..., 20 - w:], full[..., 20 - w:], rtol=0, atol=1e-13)


def test_selection_overlap_counts():
    a = np.array([[[[0, 1, 2], [64, 70, 80]]]])
    b = np.array([[[[1, 2, 5], [64, 70, 80]]]])
    assert O.selection_overlap(a, b).tolist() == [[[2, 3]]]
