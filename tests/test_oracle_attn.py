"""Pins for the oracle's sparse MQA attention: dense causal attention from
torch's scaled_dot_product_attention when k >= L, and closed forms."""
import numpy as np
import torch

from oracle import sparse_mqa_attention, topk_select, index_scores


def _dense_causal(q, kv, d_v, scale):
    """torch SDPA in float64, one shared KV broadcast to every head."""
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)  # B,H,T,D
    B, H, T, D = qt.shape
    k = torch.from_numpy(kv)[:, None].expand(B, H, kv.shape[1], D)
    v = torch.from_numpy(kv[..., :d_v])[:, None].expand(B, H, kv.shape[1], d_v)
    o = torch.nn.functional.scaled_dot_product_attention(qt, k, v, is_causal=True, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def test_k_ge_L_equals_dense_causal():
    rng = np.random.default_rng(2)
    B, L, H, dqk, dv = 2, 23, 5, 12, 8
    q = rng.normal(size=(B, L, H, dqk))
    kv = rng.normal(size=(B, L, dqk))
    scores = index_scores(rng.normal(size=(B, L, 2, 4)), rng.normal(size=(B, L, 4)),
                          rng.uniform(size=(B, L, 2)), 0)
    idx = topk_select(scores, L + 3, 0)   # k >= L keeps every causal token
    out, lse = sparse_mqa_attention(q, kv, idx, dv, 0.37)
    ref = _dense_causal(q, kv, dv, 0.37)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    # lse against a direct log-sum-exp of the causal logits
    z = 0.37 * np.einsum("bthd,bsd->bhts", q, kv)
    mask = np.arange(L)[None, :] > np.arange(L)[:, None]
    z[:, :, mask] = -np.inf
    ref_lse = np.logaddexp.reduce(z, axis=-1).transpose(0, 2, 1)
    assert np.allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(4)
    kv = rng.normal(size=(1, 30, 10))
    idx = np.array([[[3, 7, 7, 20, -1, 29]]])
    out, lse = sparse_mqa_attention(np.zeros((1, 1, 3, 10)), kv, idx, 6, 1.0)
    ref = kv[0, [3, 7, 7, 20, 29], :6].mean(0)
    assert np.allclose(out[0, 0], ref[None], atol=1e-14)
    assert np.allclose(lse, np.log(5.0), atol=1e-14)


def test_single_index_gives_that_value_row():
    rng = np.random.default_rng(6)
    q = rng.normal(size=(1, 1, 4, 9))
    kv = rng.normal(size=(1, 11, 9))
    idx = np.array([[[-1, -1, 8, -1]]])
    out, lse = sparse_mqa_attention(q, kv, idx, 5, 0.5)
    assert np.array_equal(out[0, 0], np.repeat(kv[0, 8, :5][None], 4, 0))
    assert np.allclose(lse[0, 0], 0.5 * q[0, 0] @ kv[0, 8], atol=1e-14)


def test_permutation_invariance_and_duplicates():
    rng = np.random.default_rng(8)
    q = rng.normal(size=(1, 1, 6, 16))
    kv = rng.normal(size=(1, 40, 16))
    idx = rng.choice(40, 12, replace=False)
    o1, l1 = sparse_mqa_attention(q, kv, idx[None, None], 10, 0.25)
    o2, l2 = sparse_mqa_attention(q, kv, rng.permutation(idx)[None, None], 10, 0.25)
    assert np.allclose(o1, o2, atol=1e-14) and np.allclose(l1, l2, atol=1e-14)
    # a duplicated index weighs twice: same as adding log 2 to its logit
    dup = np.concatenate([idx, idx[:1]])
    o3, l3 = sparse_mqa_attention(q, kv, dup[None, None], 10, 0.25)
    z = 0.25 * q[0, 0] @ kv[0, idx].T
    z[:, 0] += np.log(2.0)
    p = np.exp(z - z.max(1, keepdims=True))
    ref = (p @ kv[0, idx, :10]) / p.sum(1, keepdims=True)
    assert np.allclose(o3[0, 0], ref, atol=1e-13)


def test_empty_row():
    out, lse = sparse_mqa_attention(np.ones((1, 1, 2, 4)), np.ones((1, 3, 4)),
                                    np.array([[[-1, -1]]]), 3, 1.0)
    assert np.all(out == 0) and np.all(lse == -np.inf)
