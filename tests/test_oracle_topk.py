"""Pins for the oracle's top-k token selection: brute-force full sort by
(score descending, index ascending), the hand example, ties, NaN, padding."""
import json
import os

import numpy as np

from oracle import topk_select, topk_select_row


def _brute(row, k, n_cand):
    v = np.asarray(row[:n_cand], np.float64)
    # rank key: NaN lowest; -0 == +0
    key = np.where(np.isnan(v), -np.inf, v)
    nanflag = np.isnan(v).astype(int)
    order = np.lexsort((np.arange(n_cand), -key, nanflag))  # non-NaN first, score desc, index asc
    keep = np.sort(order[: min(k, n_cand)])
    out = np.full(k, -1)
    out[: keep.size] = keep
    return out


def test_bruteforce_many_seeds():
    rng = np.random.default_rng(1)
    for trial in range(600):
        L = int(rng.integers(1, 65))
        k = int(rng.integers(1, 70))
        n_cand = int(rng.integers(0, L + 1))
        kind = trial % 4
        if kind == 0:
            row = rng.normal(size=L)
        elif kind == 1:  # heavy ties, zeros of both signs
            row = rng.integers(-2, 3, size=L).astype(float) * 0.5
            row[rng.random(L) < 0.3] = -0.0
        elif kind == 2:  # all equal
            row = np.full(L, 0.25)
        else:  # NaNs and infinities mixed in
            row = rng.normal(size=L)
            row[rng.random(L) < 0.2] = np.nan
            row[rng.random(L) < 0.1] = -np.inf
            row[rng.random(L) < 0.05] = np.inf
        got = topk_select_row(row, k, n_cand)
        ref = _brute(row, k, n_cand)
        assert np.array_equal(got, ref), (trial, row, k, n_cand, got, ref)


def test_hand_example(golden_dir):
    with open(os.path.join(golden_dir, "hand_4tok_index.json")) as f:
        g = json.load(f)
    S = np.array([[-np.inf if v is None else v for v in row] for row in g["scores"]])[None]
    for k, exp in g["topk"].items():
        got = topk_select(S, int(k), q_offset=0)[0]
        assert np.array_equal(got, np.array(exp)), (k, got)


def test_causal_range_and_padding():
    row = np.arange(10, dtype=float)  # later tokens score higher
    got = topk_select(row[None, None], 4, q_offset=2)[0, 0]  # t=0 at position 2 sees 0..2
    assert list(got) == [0, 1, 2, -1]


def test_zero_ties_lower_index_wins():
    row = np.array([0.0, -0.0, 3.0, 0.0, -0.0, 1.0])
    assert list(topk_select_row(row, 4, 6)) == [0, 1, 2, 5]
