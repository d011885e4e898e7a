"""Pins for the oracle's sparse MQA attention backward: central finite
differences of the (pinned) forward, float64 autograd through torch's
scaled_dot_product_attention when every causal token is selected, an
identity that ties the query and latent gradients together, and closed forms
for repeated and empty selections."""
import numpy as np
import torch

import oracle
from oracle import sparse_mqa_attention, topk_select, index_scores


def _loss(q, kv, idx, do, d_v, scale):
    out, _ = sparse_mqa_attention(q, kv, idx, d_v, scale)
    return float(np.sum(out * do))


def test_central_finite_differences():
    rng = np.random.default_rng(11)
    B, T, N, H, dqk, dv, scale = 1, 3, 9, 3, 7, 5, 0.41
    q = rng.normal(size=(B, T, H, dqk))
    kv = rng.normal(size=(B, N, dqk))
    do = rng.normal(size=(B, T, H, dv))
    # a duplicate, an empty slot and an out-of-range slot
    idx = np.array([[[0, 4, 4, 8, -1, 2], [1, 3, 5, 7, 9, 0], [6, 2, 2, 2, 8, -1]]])
    dq, dkv = oracle.sparse_mqa_attention_bwd(q, kv, idx, do, dv, scale)
    eps = 1e-6
    for arr, grad in ((q, dq), (kv, dkv)):
        num = np.zeros_like(arr)
        for pos in np.ndindex(arr.shape):
            keep = arr[pos]
            arr[pos] = keep + eps
            lp = _loss(q, kv, idx, do, dv, scale)
            arr[pos] = keep - eps
            lm = _loss(q, kv, idx, do, dv, scale)
            arr[pos] = keep
            num[pos] = (lp - lm) / (2 * eps)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-8)
    assert np.all(dkv[0, [1, 3, 5, 7]] != 0)


def test_k_ge_L_equals_torch_autograd_of_dense_causal():
    rng = np.random.default_rng(12)
    B, L, H, dqk, dv, scale = 2, 13, 4, 10, 6, 0.29
    q = rng.normal(size=(B, L, H, dqk))
    kv = rng.normal(size=(B, L, dqk))
    do = rng.normal(size=(B, L, H, dv))
    scores = index_scores(rng.normal(size=(B, L, 2, 4)), rng.normal(size=(B, L, 4)),
                          rng.uniform(size=(B, L, 2)), 0)
    idx = topk_select(scores, L + 2, 0)
    dq, dkv = oracle.sparse_mqa_attention_bwd(q, kv, idx, do, dv, scale)

    qt = torch.from_numpy(q).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    kvt = torch.from_numpy(kv).requires_grad_(True)
    k = kvt[:, None].expand(B, H, L, dqk)
    v = kvt[:, None, :, :dv].expand(B, H, L, dv)
    o = torch.nn.functional.scaled_dot_product_attention(qt, k, v, is_causal=True, scale=scale)
    o.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    assert np.allclose(dq, qt.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dkv, kvt.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_query_and_latent_gradients_identity():
    # o depends on q and the key part only through z = scale q.c, so
    # sum_h dq[h].q[h] = sum_i dz[h,i] z[h,i] = (key part of) sum_s dkv[s].kv[s];
    # the value part adds sum_h do[h].o[h].
    rng = np.random.default_rng(13)
    B, T, N, H, dqk, dv, k = 2, 5, 40, 6, 12, 8, 16
    q = rng.normal(size=(B, T, H, dqk))
    kv = rng.normal(size=(B, N, dqk))
    do = rng.normal(size=(B, T, H, dv))
    idx = rng.integers(-3, N + 3, size=(B, T, k))
    idx[0, 0, :4] = 17  # a token selected four times
    dq, dkv = oracle.sparse_mqa_attention_bwd(q, kv, idx, do, dv, 0.7)
    out, _ = sparse_mqa_attention(q, kv, idx, dv, 0.7)
    lhs = np.sum(dq * q)
    rhs = np.sum(dkv * kv) - np.sum(do * out)
    assert abs(lhs - rhs) <= 1e-10 * (abs(lhs) + 1)


def test_one_distinct_token_closed_form():
    # every valid slot holds token a: o = c_a[:d_v] whatever q is, so dq = 0
    # and dkv[a] = (sum_h do[h], 0)
    rng = np.random.default_rng(14)
    H, dqk, dv, N = 5, 9, 6, 12
    q = rng.normal(size=(1, 1, H, dqk))
    kv = rng.normal(size=(1, N, dqk))
    do = rng.normal(size=(1, 1, H, dv))
    idx = np.array([[[7, -1, 7, N + 3, 7]]])
    dq, dkv = oracle.sparse_mqa_attention_bwd(q, kv, idx, do, dv, 0.9)
    assert np.allclose(dq, 0, atol=1e-14)
    ref = np.zeros((1, N, dqk))
    ref[0, 7, :dv] = do[0, 0].sum(0)
    assert np.allclose(dkv, ref, atol=1e-13)


def test_empty_selection_gives_zero():
    rng = np.random.default_rng(15)
    q = rng.normal(size=(1, 2, 3, 8))
    kv = rng.normal(size=(1, 5, 8))
    do = rng.normal(size=(1, 2, 3, 4))
    idx = np.array([[[-1, 5, 9], [-1, -1, -7]]])
    dq, dkv = oracle.sparse_mqa_attention_bwd(q, kv, idx, do, 4, 1.0)
    assert not dq.any() and not dkv.any()
