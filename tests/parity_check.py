"""Row-wise output check shared by the full-size GPU parity tests and the CPU test that shows
it can fail.

A full-size layer is checked on sampled output rows against the oracle's per-query form
(oracle.still_oracle.brute_rows). A row passes when its largest absolute error is within
the absolute bar (1e-4 fp32, 2e-2 bf16) and within a relative bar of that row's largest
oracle entry (REL_TOL). The relative bar is what makes the check sensitive: under the
benchmark distribution most outputs are far below the absolute bar, so a wrong key
partition would pass it; relative to each row's own size it does not (the CPU test
test_row_check_rejects_partition_mutants runs this function on such mistakes).

Relative bars: bf16 outputs are rounded to 2^-9 relative, and the probabilities, the
NP-Map features and the chunk states enter the MFMA products rounded to bf16 (each weight
off by up to 2^-9 of itself), so a row is off by a few 2^-9 of its size; 1e-2 leaves room
for that and no room for a misrouted key set. (Scores are exact fp32 sums of the stored
bf16 products, scaled in fp32: keys pre-multiplied by the logit scale and rounded to bf16
would put 2^-9 of the logit into every weight's exponent, which at the stress draw's
logits of 10 to 20 log2 units alone reaches 1.1e-2 to 1.7e-2 of a row.) fp32 rows are
off by about 1e-6 of their size (fp32 MFMA sums, hardware exp2 and reciprocal); 1e-3 is
the bar.
"""

from __future__ import annotations

import numpy as np

ABS_TOL = {"f32": 1e-4, "bf16": 2e-2}
REL_TOL = {"f32": 1e-3, "bf16": 1e-2}


def sample_rows(rng, B: int, T: int, Hq: int, n: int = 64, chunk: int = 64):
    """About n (b, hq, i) rows spread over the sequence: one random position in each of n
    equal segments, plus the first and last rows of the first two chunks and of the last
    chunk. Batch and head are drawn at random for each row."""
    pos = []
    for s in range(n):
        lo, hi = (s * T) // n, ((s + 1) * T) // n
        if hi > lo:
            pos.append(int(rng.integers(lo, hi)))
    last = ((T - 1) // chunk) * chunk
    pos += [0, chunk - 1, chunk, 2 * chunk - 1, last, T - 1]
    pos = sorted({p for p in pos if 0 <= p < T})
    return [(int(rng.integers(B)), int(rng.integers(Hq)), p) for p in pos]


def row_errors(got: np.ndarray, ref: np.ndarray):
    """Per row: (largest absolute error, that error over the row's largest oracle entry)."""
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref).reshape(len(ref), -1).max(axis=1)
    size = np.abs(ref).reshape(len(ref), -1).max(axis=1)
    rel = np.where(size > 0, err / np.where(size > 0, size, 1.0), np.where(err > 0, np.inf, 0.0))
    return err, rel


def check_rows(got, ref, dtype: str):
    """(passed, worst absolute error, worst relative error, number of failing rows)."""
    err, rel = row_errors(got, ref)
    bad = (err > ABS_TOL[dtype]) | (rel > REL_TOL[dtype])
    return (not bool(bad.any())), float(err.max(initial=0.0)), float(rel.max(initial=0.0)), int(bad.sum())


# ---- planted mistakes (CPU only): the same rows computed with a wrong key partition ------

MUTANTS = ("selected_to_linear", "far_selected_dropped", "state_dropped", "previous_chunk_selection_ignored")


def mutant_rows(O, q, k, v, w_phi, window: int, chunk: int, sel, rows, kind: str) -> np.ndarray:
    """Rows of the layer with one plausible kernel mistake planted in the oracle's per-query
    form (O is the oracle module):
      selected_to_linear               selected keys of earlier chunks go to linear attention
                                       (as a broken compact-cache loop would leave them);
      far_selected_dropped             selected keys of chunks <= c-2 are left out entirely
                                       (compact tiles skipped);
      state_dropped                    linear keys of chunks <= c-2 are left out (prefix
                                       state not read);
      previous_chunk_selection_ignored chunk c-1's selection is not applied (its selected
                                       keys outside the window go to linear attention)."""
    q, k, v, w_phi = (np.asarray(x, dtype=np.float64) for x in (q, k, v, w_phi))
    _, _, Hq, D = q.shape
    G = Hq // k.shape[2]
    sel = np.asarray(sel, dtype=bool)
    res = []
    for (b, hq, i) in rows:
        h = hq // G
        j = np.arange(i + 1)
        c = i // chunk
        in_window = j > i - window
        earlier = (j // chunk < c) & sel[b, h, : i + 1]
        far = j // chunk <= c - 2
        sa = in_window | earlier
        keep = np.ones(i + 1, dtype=bool)
        if kind == "selected_to_linear":
            sa = in_window.copy()
        elif kind == "far_selected_dropped":
            keep = ~(earlier & far & ~in_window)
        elif kind == "state_dropped":
            keep = ~(far & ~sa)
        elif kind == "previous_chunk_selection_ignored":
            sa = in_window | (earlier & far)
        else:
            raise ValueError(kind)
        phiq = O.np_map(q[b, i, hq], w_phi[h])
        phik = O.np_map(k[b, : i + 1, h][keep], w_phi[h])
        res.append(O._row(q[b, i, hq], phiq, k[b, : i + 1, h][keep], v[b, : i + 1, h][keep], phik, sa[keep], D))
    return np.array(res)


def decided_fraction(margins: np.ndarray, margin: float = 1e-3) -> float:
    m = np.asarray(margins)
    return float((m > margin).sum()) / max(1, m.size)


__all__ = ["ABS_TOL", "REL_TOL", "sample_rows", "row_errors", "check_rows", "MUTANTS", "mutant_rows",
           "decided_fraction", "group_scores"]


def group_scores(O, q, k, window: int, heads, score: str = "saliency", threads: int = 8) -> np.ndarray:
    """The oracle's group-summed routing score for the KV heads `heads` only ([B, len(heads),
    T]), one KV head per thread (each head's query group is independent of the others)."""
    from concurrent.futures import ThreadPoolExecutor

    G = q.shape[2] // k.shape[2]

    def one(h):
        qg, kg = q[:, :, h * G:(h + 1) * G], k[:, :, h:h + 1]
        s = O.saliency(qg, kg, window)[0] if score == "saliency" else O.diagonal_score(qg, kg)[0]
        return s[:, 0]

    with ThreadPoolExecutor(max_workers=max(1, min(threads, len(heads)))) as ex:
        return np.stack(list(ex.map(one, heads)), axis=1)
