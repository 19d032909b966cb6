"""CPU checks of the row-wise output check the full-size GPU tests use: it must reject the
outputs of a wrong key partition (planted in the oracle) on the very rows and inputs those
tests sample, and must accept the oracle's own output rounded to bf16."""

import numpy as np
import pytest

import parity_check as PC
from linear_attention_saliency_amd import synth
from oracle import still_oracle as O


@pytest.mark.parametrize("stress", [False, True], ids=["bench-draw", "stress"])
def test_row_check_rejects_partition_mutants(stress):
    """The 16K Llama-3.2-1B-shaped layer: every planted partition mistake fails the check on
    the sampled rows (under the benchmark draw the outputs are small enough that the
    absolute bar alone passes some of them; the relative bar does not)."""
    wl = synth.L1B_16K.replace(qk_scale=1.0) if stress else synth.L1B_16K
    q, k, v, wp = synth.make_inputs(wl)
    s = PC.group_scores(O, q, k, wl.window, range(wl.n_kv_heads))
    _, sel = O.route(s, wl.chunk, wl.top_k)
    rows = PC.sample_rows(np.random.default_rng(5), 1, wl.seq_len, wl.n_q_heads, 64)
    assert len(rows) >= 64 and rows[0][2] == 0 and rows[-1][2] == wl.seq_len - 1
    ref = O.brute_rows(q, k, v, wp, wl.window, wl.chunk, sel, rows)
    # the oracle's own rows, rounded as the device stores them, pass
    ok, ea, er, _ = PC.check_rows(synth.round_bf16(ref.astype(np.float32)), ref, "bf16")
    assert ok and er <= 2.0 ** -8, er
    absolute_only_misses = 0
    for kind in PC.MUTANTS:
        mut = PC.mutant_rows(O, q, k, v, wp, wl.window, wl.chunk, sel, rows, kind)
        ok, ea, er, nbad = PC.check_rows(mut, ref, "bf16")
        assert not ok, (kind, ea, er)
        absolute_only_misses += ea <= PC.ABS_TOL["bf16"]
    if not stress:
        assert absolute_only_misses >= 1  # why the relative bar is there


def test_row_check_bars():
    ref = np.array([[0.5, -0.25], [1e-3, 2e-3]])
    assert PC.check_rows(ref * (1 + 4e-3), ref, "bf16")[0]
    assert not PC.check_rows(ref + np.array([[0.0, 0.0], [0.0, 3e-5]]), ref, "bf16")[0]  # 1.5% of row 2
    assert not PC.check_rows(ref + np.array([[0.021, 0.0], [0.0, 0.0]]), ref, "bf16")[0]  # absolute bar
    assert PC.check_rows(np.zeros((1, 3)), np.zeros((1, 3)), "f32")[0]
    assert not PC.check_rows(np.full((1, 3), 1e-9), np.zeros((1, 3)), "f32")[0]


def _grads_far_selected_pairs_dropped(q, k, v, w, window, chunk, sel, dout, rows):
    """The oracle's backward with one planted mistake: no gradient reaches k and v through the
    softmax pairs of selected keys from queries two or more chunks later (the pairs a broken
    selected-key kernel would lose). Same dense form as attend_backward otherwise."""
    import math

    import torch

    qt, kt, vt, wt = (torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True) for x in (q, k, v, w))
    do = torch.tensor(np.asarray(dout, dtype=np.float64))
    B, T, Hq, D = qt.shape
    G = Hq // kt.shape[2]
    selt = torch.tensor(sel)
    i = torch.tensor(rows)[:, None]
    j = torch.arange(T)[None, :]
    loss = torch.zeros((), dtype=torch.float64)
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            far_sel = (j // chunk <= i // chunk - 2) & selt[b, h][None, :]
            sa = (j <= i) & ((j > i - window) | ((j // chunk < i // chunk) & selt[b, h][None, :]))
            la = (j <= i) & ~sa
            qq, kk, vv = qt[b, rows, hq], kt[b, :, h], vt[b, :, h]
            kd, vd = kk.detach(), vv.detach()
            a = torch.where(far_sel, qq @ kd.T, qq @ kk.T) / math.sqrt(D)
            a = torch.where(sa, a, -math.inf)
            M = a.detach().amax(dim=1, keepdim=True)
            e = torch.exp(a - M)
            lw = torch.where(la, O._np_map_t(qq, wt[h]) @ O._np_map_t(kk, wt[h]).T, 0.0) * torch.exp(-M)
            wgt = e + lw
            num = torch.where(far_sel, e, 0.0) @ vd + torch.where(far_sel, 0.0, e) @ vv + lw @ vv
            o = num / wgt.sum(dim=1, keepdim=True)
            loss = loss + (o * do[b, rows, hq]).sum()
    loss.backward()
    return kt.grad.numpy(), vt.grad.numpy()


def test_backward_bar_sees_missing_far_key_gradients():
    """The full-size backward tests compare every gradient within 3e-2 of its largest entry,
    with dout zero outside about 70 sampled rows. On the routing-stress draw that bar rejects
    dk and dv without the gradients of the selected keys' far pairs (the benchmark draw
    alone would not: there those are under 1.2% of the largest entry)."""
    wl = synth.L1B_16K.replace(seq_len=4096, n_q_heads=8, n_kv_heads=2, qk_scale=1.0, n_planted=41)
    q, k, v, wp = synth.make_inputs(wl)
    s = PC.group_scores(O, q, k, wl.window, range(wl.n_kv_heads))
    _, sel = O.route(s, wl.chunk, wl.top_k)
    rows = np.array(sorted({i for (_, _, i) in PC.sample_rows(np.random.default_rng(7), 1, 4096, 1, 64)}))
    dout = synth.make_grad_out(wl)
    _, dk, dv, _ = O.attend_backward(q, k, v, wp, wl.window, wl.chunk, sel, dout, rows=rows)
    mk, mv = _grads_far_selected_pairs_dropped(q, k, v, wp, wl.window, wl.chunk, sel, dout, rows)
    rel = lambda g, r: float(np.abs(g - r).max() / np.abs(r).max())  # noqa: E731
    assert rel(mk, dk) > 3e-2 and rel(mv, dv) > 3e-2, (rel(mk, dk), rel(mv, dv))
