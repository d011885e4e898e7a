"""Debug validation of caller indices (environment DSA_VALIDATE=1): entry
points that take token indices or cache positions refuse out-of-range ones
with DSA_ERR_BAD_INDEX and launch nothing else; without it they skip them."""
import numpy as np
import pytest
import torch

import long_context_02_amd as dsa
from dsa_parity import gpu_device

pytestmark = pytest.mark.gpu

BAD_INDEX = 4


def _attn_inputs(dev, N=300, T=3, k=64, seed=0):
    g = torch.Generator(device=dev).manual_seed(seed)
    q = torch.randn(1, T, 128, 576, generator=g, device=dev, dtype=torch.bfloat16)
    kv = torch.randn(1, N, 576, generator=g, device=dev, dtype=torch.bfloat16)
    rng = np.random.default_rng(seed)
    idx = np.full((1, T, k), -1, dtype=np.int32)
    for t in range(T):
        idx[0, t, :k // 2] = np.sort(rng.choice(N, k // 2, replace=False))
    return q, kv, idx


def _expect_bad(fn):
    with pytest.raises(dsa.DSAError) as e:
        fn()
    assert e.value.status == BAD_INDEX


def test_attention_forward_and_backward(monkeypatch):
    dev = gpu_device()
    q, kv, idx = _attn_inputs(dev)
    N = kv.shape[1]
    good = torch.from_numpy(idx).to(dev)
    print("[validate] attention", flush=True)
    ref_o, ref_l = dsa.sparse_mla_attn(q, kv, good, 512, 0.04)
    monkeypatch.setenv("DSA_VALIDATE", "1")
    o, l = dsa.sparse_mla_attn(q, kv, good, 512, 0.04)   # -1 padding is valid
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
    for bad_value in (N, N + 5, -2, -(1 << 31)):
        bad = idx.copy()
        bad[0, 1, 3] = bad_value
        bad_t = torch.from_numpy(bad).to(dev)
        out = torch.full_like(ref_o, 7.0)
        _expect_bad(lambda: dsa.sparse_mla_attn(q, kv, bad_t, 512, 0.04, out=out))
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())                  # nothing else ran
        dout = torch.ones_like(ref_o)
        _expect_bad(lambda: dsa.sparse_mla_attn_bwd(q, kv, bad_t, ref_o, ref_l, dout, 0.04))
    # without validation an out-of-range slot is skipped
    monkeypatch.delenv("DSA_VALIDATE")
    bad = idx.copy()
    bad[0, 1, 40] = N + 5                                # a padding slot made out of range
    o2, _ = dsa.sparse_mla_attn(q, kv, torch.from_numpy(bad).to(dev), 512, 0.04)
    torch.cuda.synchronize()
    assert torch.equal(o2, ref_o)


def test_indexer_kl_selected_set(monkeypatch):
    dev = gpu_device()
    N, k = 500, 32
    scores = torch.randn(1, 2, N, device=dev)
    p = torch.full((1, 2, k), 1.0 / k, device=dev)
    idx = torch.arange(k, device=dev, dtype=torch.int32).repeat(1, 2, 1)
    monkeypatch.setenv("DSA_VALIDATE", "1")
    print("[validate] indexer kl", flush=True)
    dsa.indexer_kl(scores, p, idx=idx)
    idx[0, 1, 5] = N
    _expect_bad(lambda: dsa.indexer_kl(scores, p, idx=idx))


def test_cache_append_positions(monkeypatch):
    dev = gpu_device()
    B, T, N = 3, 2, 64
    k_new = torch.randn(B, T, 128, device=dev)
    kv_new = torch.randn(B, T, 576, device=dev).to(torch.bfloat16)
    k_cache = torch.zeros(B, N, 128, dtype=torch.uint8, device=dev)
    k_scale = torch.zeros(B, N, device=dev)
    kv_cache = torch.zeros(B, N, 576, dtype=torch.bfloat16, device=dev)
    monkeypatch.setenv("DSA_VALIDATE", "1")
    print("[validate] cache append", flush=True)
    dsa.cache_append(k_new, kv_new, k_cache, k_scale, kv_cache, torch.tensor([0, 10, N - T], dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    before = kv_cache.clone()
    for pos in ([0, 10, N - 1], [-1, 0, 0]):             # last row past the end / first before the start
        _expect_bad(lambda: dsa.cache_append(k_new, kv_new, k_cache, k_scale, kv_cache,
                                             torch.tensor(pos, dtype=torch.int32, device=dev)))
    torch.cuda.synchronize()
    assert torch.equal(kv_cache, before)
