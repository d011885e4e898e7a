"""Pins for the oracle's indexer KL objective (dense warm-up and the form
restricted to the selected set): torch's kl_div with float64 autograd, the
p = softmax(I) and one-hot closed forms, central finite differences, shift
invariance, non-negativity, and the sparse form over every candidate equal
to the dense form."""
import math

import numpy as np
import torch

import oracle


def _row(seed, n):
    rng = np.random.default_rng(seed)
    I = rng.normal(0, 3, n)
    p = rng.dirichlet(np.full(n, 0.3))
    p[rng.random(n) < 0.2] = 0.0            # exact zeros in the target
    return I, p / p.sum()


def test_matches_torch_kl_div_and_autograd():
    for seed, n in [(1, 7), (2, 100), (3, 1000)]:
        I, p = _row(seed, n)
        loss, grad = oracle.indexer_kl_dense_row(I, p, n)
        It = torch.tensor(I, dtype=torch.float64, requires_grad=True)
        pt = torch.tensor(p, dtype=torch.float64)
        lt = torch.nn.functional.kl_div(torch.log_softmax(It, 0), pt, reduction="sum")
        lt.backward()
        assert abs(loss - lt.item()) <= 1e-12 * max(1.0, abs(lt.item()))
        assert np.allclose(grad, It.grad.numpy(), rtol=0, atol=1e-14)


def test_target_equal_to_softmax_gives_zero():
    I, _ = _row(4, 50)
    q = np.exp(I - I.max())
    q /= q.sum()
    loss, grad = oracle.indexer_kl_dense_row(I, q, 50)
    assert abs(loss) < 1e-13 and np.max(np.abs(grad)) < 1e-15


def test_one_hot_target_closed_form():
    I, _ = _row(5, 30)
    p = np.zeros(30)
    p[11] = 1.0
    loss, grad = oracle.indexer_kl_dense_row(I, p, 30)
    lse = math.log(sum(math.exp(v) for v in I))      # plain Python sum
    assert abs(loss - (lse - I[11])) < 1e-12
    q = [math.exp(v - lse) for v in I]
    assert all(abs(grad[s] - (q[s] - (s == 11))) < 1e-14 for s in range(30))


def test_finite_differences():
    I, p = _row(6, 12)
    _, grad = oracle.indexer_kl_dense_row(I, p, 12)
    h = 1e-6
    for s in range(12):
        e = np.zeros(12)
        e[s] = h
        up, _ = oracle.indexer_kl_dense_row(I + e, p, 12)
        dn, _ = oracle.indexer_kl_dense_row(I - e, p, 12)
        assert abs((up - dn) / (2 * h) - grad[s]) < 1e-8


def test_shift_invariance_and_non_negative():
    I, p = _row(7, 200)
    l0, g0 = oracle.indexer_kl_dense_row(I, p, 200)
    l1, g1 = oracle.indexer_kl_dense_row(I + 123.5, p, 200)
    assert l0 >= 0 and abs(l0 - l1) < 1e-10 and np.max(np.abs(g0 - g1)) < 1e-12


def test_causal_range_and_unnormalised_target():
    I, p = _row(8, 40)
    p = p * 3.0                                   # P = 3: gradient P q - p
    loss, grad = oracle.indexer_kl_dense_row(I, p, 25)
    assert np.all(grad[25:] == 0)
    q = np.exp(I[:25] - I[:25].max())
    q /= q.sum()
    P = p[:25].sum()
    assert np.allclose(grad[:25], P * q - p[:25], atol=1e-15)
    pos = p[:25] > 0
    assert abs(loss - np.sum(p[:25][pos] * np.log(p[:25][pos] / q[pos]))) < 1e-12


def test_sparse_over_all_candidates_equals_dense():
    rng = np.random.default_rng(9)
    B, T, N, q_off = 2, 3, 20, 17
    scores = rng.normal(0, 2, (B, T, N))
    p = rng.random((B, T, N))
    ld, gd = oracle.indexer_kl(scores, p, q_off)
    k = N
    idx = np.full((B, T, k), -1)
    ps = np.zeros((B, T, k))
    for b in range(B):
        for t in range(T):
            n = min(N, q_off + t + 1)
            perm = rng.permutation(n)             # slot order must not matter
            idx[b, t, :n] = perm
            ps[b, t, :n] = p[b, t, perm]
    ls, gs = oracle.indexer_kl(scores, ps, q_off, idx=idx)
    assert np.allclose(ls, ld, rtol=1e-12, atol=1e-12)
    for b in range(B):
        for t in range(T):
            n = min(N, q_off + t + 1)
            assert np.allclose(gs[b, t, :n], gd[b, t, idx[b, t, :n]], atol=1e-14)
            assert np.all(gs[b, t, n:] == 0)
