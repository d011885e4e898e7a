"""Pins for the oracle's lightning-indexer scores."""
import json
import os

import numpy as np
import torch

from oracle import index_scores, e4m3_encode


def _hand(golden_dir):
    with open(os.path.join(golden_dir, "hand_4tok_index.json")) as f:
        return json.load(f)


def test_hand_example_exact(golden_dir):
    g = _hand(golden_dir)
    K = np.array(g["keys"], np.float64)
    Q = np.array(g["queries"], np.float64)
    w = np.array(g["w"], np.float64)
    # as raw floats
    I = index_scores(Q[None], K[None], w[None], q_offset=0)[0]
    exp = np.array([[-np.inf if v is None else v for v in row] for row in g["scores"]])
    assert np.array_equal(I, exp)
    # as FP8 codes with unit scales: identical
    qc, kc = e4m3_encode(Q), e4m3_encode(K)
    I8 = index_scores(qc[None], kc[None], w[None], 0,
                      q_scale=np.ones((1, 4, 2)), k_scale=np.ones((1, 4)))[0]
    assert np.array_equal(I8, exp)


def test_fp8_dot_equals_integer_dot():
    """H_I = 1, w = 1, unit scales: I = ReLU(q.k) and q.k is exact.  Check it
    against an int64 dot of the codes' values times 2^9 (decoded by torch)."""
    rng = np.random.default_rng(3)
    T, N, d = 6, 50, 128
    qc = rng.integers(0, 256, (1, T, 1, d), dtype=np.uint8)
    kc = rng.integers(0, 256, (1, N, d), dtype=np.uint8)
    qc[(qc & 0x7F) == 0x7F] = 0x3F
    kc[(kc & 0x7F) == 0x7F] = 0x41
    I = index_scores(qc, kc, np.ones((1, T, 1)), q_offset=N, q_scale=np.ones((1, T, 1)),
                     k_scale=np.ones((1, N)))[0]
    tq = (torch.from_numpy(qc).view(torch.float8_e4m3fn).double() * 512).long()[0, :, 0]
    tk = (torch.from_numpy(kc).view(torch.float8_e4m3fn).double() * 512).long()[0]
    dot = (tq[:, None, :] * tk[None, :, :]).sum(-1)  # int64, exact
    ref = torch.clamp(dot, min=0).double().numpy() / 2.0 ** 18
    assert np.array_equal(I, ref)


def test_brute_force_python_loops():
    rng = np.random.default_rng(11)
    B, T, N, H, d, off = 2, 5, 9, 3, 4, 3
    q = rng.normal(size=(B, T, H, d))
    k = rng.normal(size=(B, N, d))
    w = rng.uniform(-1, 1, size=(B, T, H))  # negative weights allowed
    I = index_scores(q, k, w, off)
    for b in range(B):
        for t in range(T):
            for s in range(N):
                if s > off + t:
                    assert I[b, t, s] == -np.inf
                    continue
                acc = 0.0
                for j in range(H):
                    dot = 0.0
                    for c in range(d):
                        dot += q[b, t, j, c] * k[b, s, c]
                    acc += w[b, t, j] * max(0.0, dot)
                assert abs(I[b, t, s] - acc) <= 1e-12 * (1 + abs(acc))


def test_scales_fold_through_relu():
    """Positive per-token scales multiply the score: I(qs, ks) = qs*ks*I(1, 1)."""
    rng = np.random.default_rng(5)
    T, N, H, d = 4, 12, 8, 128
    qc = e4m3_encode(rng.normal(0, 60, (1, T, H, d)))
    kc = e4m3_encode(rng.normal(0, 60, (1, N, d)))
    w = rng.uniform(0, 1, (1, T, H))
    qs = rng.uniform(0.001, 0.01, (1, T))
    ks = rng.uniform(0.001, 0.01, (1, N))
    I1 = index_scores(qc, kc, w, N, q_scale=np.ones((1, T, H)), k_scale=np.ones((1, N)))
    Is = index_scores(qc, kc, w, N, q_scale=np.repeat(qs[..., None], H, -1), k_scale=ks)
    ref = I1 * qs[..., None] * ks[:, None, :]
    assert np.allclose(Is, ref, rtol=1e-13, atol=0)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(9)
    q = rng.normal(size=(2, 6, 2, 8))
    k = rng.normal(size=(2, 10, 8))
    w = rng.uniform(size=(2, 6, 2))
    full = index_scores(q, k, w, 4)
    rows = [(1, 5), (0, 0), (1, 2)]
    sub = index_scores(q, k, w, 4, rows=rows)
    for r, (b, t) in enumerate(rows):
        assert np.array_equal(sub[r], full[b, t])
