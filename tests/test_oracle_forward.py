"""Pins for the oracle's composed path."""
import numpy as np

from oracle import dsa_forward, e4m3_encode, sparse_mqa_attention
from test_oracle_attn import _dense_causal


def _inputs(rng, B, L, HI=8, dI=128, H=4, dqk=24, dv=16):
    qc = e4m3_encode(rng.normal(0, 50, (B, L, HI, dI)))
    kc = e4m3_encode(rng.normal(0, 50, (B, L, dI)))
    qs = np.repeat(rng.uniform(0.001, 0.01, (B, L, 1)), HI, -1)
    ks = rng.uniform(0.001, 0.01, (B, L))
    w = rng.uniform(0, 0.125, (B, L, HI))
    q = rng.normal(size=(B, L, H, dqk))
    kv = rng.normal(size=(B, L, dqk))
    return qc, qs, kc, ks, w, q, kv


def test_chunked_prefill_equals_tail_of_full_prefill():
    rng = np.random.default_rng(12)
    B, L, T, k = 2, 40, 9, 7
    qc, qs, kc, ks, w, q, kv = _inputs(rng, B, L)
    full = dsa_forward(qc, kc, w, q, kv, k=k, q_offset=0, d_v=16, sm_scale=0.2,
                       q_scale=qs, k_scale=ks)
    off = L - T
    chunk = dsa_forward(qc[:, off:], kc, w[:, off:], q[:, off:], kv, k=k, q_offset=off,
                        d_v=16, sm_scale=0.2, q_scale=qs[:, off:], k_scale=ks)
    rows_full = [r for r, (b, t) in enumerate(full["rows"]) if t >= off]
    assert np.array_equal(chunk["idx"], full["idx"][rows_full])
    assert np.array_equal(chunk["out"], full["out"][rows_full])
    assert np.array_equal(chunk["scores"], full["scores"][rows_full])


def test_forward_with_k_ge_L_is_dense_causal():
    rng = np.random.default_rng(13)
    B, L = 1, 17
    qc, qs, kc, ks, w, q, kv = _inputs(rng, B, L)
    res = dsa_forward(qc, kc, w, q, kv, k=32, q_offset=0, d_v=16, sm_scale=0.3,
                      q_scale=qs, k_scale=ks)
    ref = _dense_causal(q, kv, 16, 0.3)
    assert np.allclose(res["out"].reshape(ref.shape), ref, rtol=1e-12, atol=1e-12)


def test_selected_set_is_the_top_scores():
    rng = np.random.default_rng(14)
    qc, qs, kc, ks, w, q, kv = _inputs(rng, 1, 60)
    res = dsa_forward(qc, kc, w, q, kv, k=10, q_offset=0, d_v=16, sm_scale=0.3,
                      q_scale=qs, k_scale=ks)
    for r, (b, t) in enumerate(res["rows"]):
        sel = res["idx"][r][res["idx"][r] >= 0]
        assert sel.size == min(10, t + 1)
        s = res["scores"][r][: t + 1]
        if t + 1 > 10:
            others = np.setdiff1d(np.arange(t + 1), sel)
            assert s[sel].min() >= s[others].max()
        o, _ = sparse_mqa_attention(q[b:b + 1, t:t + 1], kv[b:b + 1], sel[None, None], 16, 0.3)
        assert np.allclose(o[0, 0], res["out"][r], atol=1e-14)
