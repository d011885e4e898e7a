"""Pins for the oracle's sparse MLA attention in MHA mode (per-head keys and
values up-projected from the latent entries).

* Absorption: the per-head products equal MQA mode on the latent entries
  with the key up-projection folded into the query and the value
  up-projection applied to the output (q . [W_UK c ; r] = [W_UK^T q_n ; q_r]
  . [c ; r] and sum_i p_i W_UV c_i = W_UV sum_i p_i c_i), checked against the
  separately pinned MQA-mode oracle.
* k >= L: dense causal multi-head attention from torch's
  scaled_dot_product_attention in float64, each head with its own keys and
  values built by explicit per-head matrix products.
* A single selected token gives that head's value row exactly.
"""
import numpy as np
import torch

from oracle import (index_scores, mha_keys_values, sparse_mha_attention, sparse_mqa_attention,
                    topk_select)

D_C, D_R, D_N, D_VH = 16, 6, 8, 5


def _inputs(seed, B=2, T=9, N=21, H=4):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(B, T, H, D_N + D_R))
    kv = rng.normal(size=(B, N, D_C + D_R))
    w_uk = rng.normal(size=(H, D_N, D_C)) / np.sqrt(D_C)
    w_uv = rng.normal(size=(H, D_VH, D_C)) / np.sqrt(D_C)
    idx = np.stack([np.stack([rng.permutation(N)[:7] for _ in range(T)]) for _ in range(B)])
    if B > 1 and T > 4:
        idx[0, 1, 3] = -1             # an empty slot
        idx[1, 2, :3] = idx[1, 2, 3]  # a token in four slots
        idx[1, 4, 0] = N + 5          # out of range: skipped
    return q, kv, w_uk, w_uv, idx


def test_absorption_equals_mqa_mode():
    q, kv, w_uk, w_uv, idx = _inputs(1)
    scale = 0.41
    out, lse = sparse_mha_attention(q, kv, w_uk, w_uv, idx, scale, D_C)
    # MQA mode on the latent entries: query [W_UK[h]^T q_nope ; q_rope]
    q_abs = np.concatenate([np.einsum("hdc,bthd->bthc", w_uk, q[..., :D_N]), q[..., D_N:]], axis=-1)
    o_lat, lse_mqa = sparse_mqa_attention(q_abs, kv, idx, D_C, scale)
    out_abs = np.einsum("hvc,bthc->bthv", w_uv, o_lat)
    assert np.allclose(out, out_abs, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, lse_mqa, rtol=1e-12, atol=1e-12)


def _dense_mha_causal(q, kv, w_uk, w_uv, scale):
    """torch SDPA in float64 with per-head keys and values, each built by a
    matrix product of that head's up-projection with the latent part."""
    B, T, H, _ = q.shape
    c = torch.from_numpy(kv[..., :D_C])
    r = torch.from_numpy(kv[..., D_C:])
    ks, vs = [], []
    for h in range(H):
        ks.append(torch.cat([c @ torch.from_numpy(w_uk[h]).T, r], dim=-1))
        vs.append(c @ torch.from_numpy(w_uv[h]).T)
    k = torch.stack(ks, dim=1)  # B,H,N,D
    v = torch.stack(vs, dim=1)
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(qt, k, v, is_causal=True, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def test_k_ge_L_equals_dense_causal_mha():
    rng = np.random.default_rng(3)
    B, L, H = 2, 17, 3
    q = rng.normal(size=(B, L, H, D_N + D_R))
    kv = rng.normal(size=(B, L, D_C + D_R))
    w_uk = rng.normal(size=(H, D_N, D_C)) / 4
    w_uv = rng.normal(size=(H, D_VH, D_C)) / 4
    scores = index_scores(rng.normal(size=(B, L, 2, 4)), rng.normal(size=(B, L, 4)),
                          rng.uniform(size=(B, L, 2)), 0)
    idx = topk_select(scores, L + 2, 0)
    out, lse = sparse_mha_attention(q, kv, w_uk, w_uv, idx, 0.3, D_C)
    ref = _dense_mha_causal(q, kv, w_uk, w_uv, 0.3)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    assert np.all(np.isfinite(lse))


def test_single_index_gives_that_heads_value_row():
    q, kv, w_uk, w_uv, _ = _inputs(5, B=1, T=1)
    idx = np.array([[[-1, 11, -1]]])
    out, lse = sparse_mha_attention(q, kv, w_uk, w_uv, idx, 0.7, D_C)
    for h in range(q.shape[2]):
        v = w_uv[h] @ kv[0, 11, :D_C]
        k = np.concatenate([w_uk[h] @ kv[0, 11, :D_C], kv[0, 11, D_C:]])
        assert np.allclose(out[0, 0, h], v, rtol=1e-14, atol=1e-14)
        assert np.isclose(lse[0, 0, h], 0.7 * q[0, 0, h] @ k, rtol=1e-14, atol=1e-14)


def test_keys_values_shapes_and_shared_rope():
    _, kv, w_uk, w_uv, _ = _inputs(7, B=1)
    K, V = mha_keys_values(kv[0], w_uk, w_uv, D_C)
    assert K.shape == (kv.shape[1], w_uk.shape[0], D_N + D_R) and V.shape == (kv.shape[1], w_uk.shape[0], D_VH)
    assert np.array_equal(K[:, 0, D_N:], K[:, -1, D_N:])  # one rope key for every head
    assert np.array_equal(K[:, 2, D_N:], kv[0, :, D_C:])


def test_empty_row_gives_zero_and_minus_inf():
    q, kv, w_uk, w_uv, _ = _inputs(9, B=1, T=1)
    out, lse = sparse_mha_attention(q, kv, w_uk, w_uv, np.full((1, 1, 4), -1), 1.0, D_C)
    assert np.all(out == 0) and np.all(lse == -np.inf)
