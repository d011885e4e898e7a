"""GPU parity of dsa_sparse_mla_attn against the oracle (float64)."""
import numpy as np
import pytest
import torch

import long_context_02_amd as dsa
import oracle
from dsa_parity import Guarded, check_attention, check_lse, gpu_device, np64, poisoned_workspace
from long_context_02_amd.synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _random_idx(B, T, N, k, rng, n_valid=None, junk=False):
    idx = np.full((B, T, k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(T):
            n = k if n_valid is None else n_valid[t]
            n = min(n, N)
            idx[b, t, :n] = np.sort(rng.choice(N, n, replace=False))
            if junk and n > 4:
                idx[b, t, 1] = N + 5          # out of range: skipped
                idx[b, t, 3] = -7             # negative: skipped
                idx[b, t, 2] = idx[b, t, 0]   # duplicate: counts twice
    return idx


def _run(wl, idx_np, seed, where, scale=None):
    dev = gpu_device()
    scale = wl.sm_scale if scale is None else scale
    inp = make_inputs(wl, seed=seed, device="cpu")
    q, kv = inp["q"].to(dev), inp["kv"].to(dev)
    print(f"[attn] {where}", flush=True)
    B, T, H = q.shape[:3]
    k = idx_np.shape[-1]
    out_g = Guarded((B, T, H, wl.d_v), q.dtype, dev, float("nan"))
    lse_g = Guarded((B, T, H), torch.float32, dev, float("nan"))
    need = dsa.workspace_size(dsa.OP_ATTN, B, T, wl.N, 1, H, wl.d_v, k) if 1 <= k <= 2048 else 0
    ws = poisoned_workspace(need, dev)
    out, lse = dsa.sparse_mla_attn(q, kv, torch.from_numpy(idx_np).to(dev), wl.d_v, scale,
                                   out=out_g.view, lse=lse_g.view, workspace=ws.view)
    torch.cuda.synchronize()
    for name, buf in (("out", out_g), ("lse", lse_g), ("workspace", ws)):
        buf.check(f"{where} {name}")
    ref_o, ref_l = oracle.sparse_mqa_attention(np64(inp["q"]), np64(inp["kv"]), idx_np, wl.d_v, scale)
    bf16 = wl.dtype == "bf16"
    check_attention(np64(out), ref_o, bf16, where)
    check_lse(np64(lse), ref_l, bf16, where)


def test_tiny_f32():
    wl = WORKLOADS["tiny"].with_(T=40)
    rng = np.random.default_rng(0)
    _run(wl, _random_idx(1, 40, wl.N, wl.k, rng, n_valid=[min(64, t + 1) for t in range(40)]), 1,
         "tiny f32")


def test_f32_junk_indices():
    wl = WORKLOADS["tiny"].with_(T=6)
    rng = np.random.default_rng(1)
    _run(wl, _random_idx(1, 6, wl.N, wl.k, rng, junk=True), 2, "f32 junk")


@pytest.mark.parametrize("B,T,N,k", [
    (1, 3, 3000, 2048),     # split path (few rows)
    (2, 2, 2500, 2048),
    (1, 300, 4000, 256),    # one workgroup per row (>= 256 rows)
    (1, 5, 700, 100),       # k not a multiple of the tile
    (1, 80, 3000, 2048),    # 64 to 255 rows: split, several splits per CU round
    (2, 50, 2000, 300),
    (1, 64, 900, 100),
])
def test_bf16_random_sets(B, T, N, k):
    wl = WORKLOADS["prefill_8k"].with_(B=B, T=T, N=N, k=k)
    rng = np.random.default_rng(B * 100 + T)
    nv = [int(x) for x in rng.integers(1, k + 1, T)]
    nv[0] = k
    _run(wl, _random_idx(B, T, N, k, rng, n_valid=nv), 3, f"bf16 B={B} T={T} N={N} k={k}")


def test_bf16_junk_and_empty_rows():
    wl = WORKLOADS["prefill_8k"].with_(B=1, T=4, N=900, k=512)
    rng = np.random.default_rng(9)
    idx = _random_idx(1, 4, 900, 512, rng, junk=True)
    idx[0, 2] = -1                              # a row with no valid slot
    _run(wl, idx, 4, "bf16 junk/empty")
    wl = WORKLOADS["prefill_8k"].with_(B=1, T=300, N=900, k=64)
    idx = _random_idx(1, 300, 900, 64, rng, junk=True)
    idx[0, 7] = -1
    _run(wl, idx, 5, "bf16 junk/empty, unsplit")
    wl = WORKLOADS["prefill_8k"].with_(B=1, T=70, N=900, k=512)
    idx = _random_idx(1, 70, 900, 512, rng, junk=True)
    idx[0, 9] = -1
    _run(wl, idx, 6, "bf16 junk/empty, 70 rows")


@pytest.mark.parametrize("T", [3, 80, 300])
def test_bf16_negative_scale(T):
    """A negative softmax scale (the kernel copies that track max(-s)) on the
    split path (3 and 80 rows) and the one-workgroup-per-row path."""
    wl = WORKLOADS["prefill_8k"].with_(B=1, T=T, N=2500, k=2048 if T == 3 else 512)
    rng = np.random.default_rng(31 + T)
    _run(wl, _random_idx(1, T, wl.N, wl.k, rng), 7, f"bf16 negative scale T={T}", scale=-wl.sm_scale)


@pytest.mark.parametrize("T", [2, 64, 300])
def test_bf16_large_logit_gap_reruns_exactly(T):
    """A selected key in a late tile whose rope part is scaled x80 lifts some
    heads' logits far above the first tile's max (more than 2^64 in exp2
    terms); the kernel must notice and redo the pass with the exact max."""
    dev = gpu_device()
    wl = WORKLOADS["prefill_8k"].with_(B=1, T=T, N=3000, k=2048 if T <= 64 else 256)
    rng = np.random.default_rng(21)
    idx = _random_idx(1, T, wl.N, wl.k, rng)
    inp = make_inputs(wl, seed=8, device="cpu")
    hot = int(idx[0, 0, wl.k - 5])
    inp["kv"][0, hot, 512:] *= 80
    q, kv = inp["q"].to(dev), inp["kv"].to(dev)
    out, lse = dsa.sparse_mla_attn(q, kv, torch.from_numpy(idx).to(dev), wl.d_v, wl.sm_scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.sparse_mqa_attention(np64(inp["q"]), np64(inp["kv"]), idx, wl.d_v, wl.sm_scale)
    gap = (ref_l[0, 0] - ref_l[0, 0].min()).max()
    print(f"  large-gap T={T}: lse spread {gap:.1f}", flush=True)
    check_attention(np64(out), ref_o, True, f"large gap T={T}")
    check_lse(np64(lse), ref_l, True, f"large gap T={T}")


def test_bf16_largest_supported_context():
    """N just under the 2^31 / 1152 rows that the gather's 32-bit byte
    offsets cover: selections at the very end of the cache, and one row of
    mixed low and high indices.  The oracle sees only the selected rows."""
    dev = gpu_device()
    N, H, dqk, dv, k = 1_864_000, 128, 576, 512, 2048
    gen = torch.Generator(device=dev).manual_seed(31)
    kv = torch.randn(1, N, dqk, generator=gen, device=dev, dtype=torch.bfloat16)
    q = torch.randn(1, 2, H, dqk, generator=gen, device=dev, dtype=torch.bfloat16)
    rng = np.random.default_rng(31)
    idx = np.empty((1, 2, k), dtype=np.int32)
    idx[0, 0] = np.arange(N - k, N)
    idx[0, 1] = np.sort(np.concatenate([rng.choice(1000, 1000, replace=False),
                                        N - 1 - rng.choice(200_000, k - 1000, replace=False)]))
    scale = 1.0 / np.sqrt(dqk)
    print("[attn] largest context", flush=True)
    out, lse = dsa.sparse_mla_attn(q, kv, torch.from_numpy(idx).to(dev), dv, scale)
    torch.cuda.synchronize()
    for t in range(2):
        uniq, local = np.unique(idx[0, t], return_inverse=True)
        rows = np64(kv[0, torch.from_numpy(uniq.astype(np.int64)).to(dev)])
        o, l = oracle.sparse_mqa_attention_row(np64(q[0, t]), rows, local, dv, scale)
        check_attention(np64(out[0, t]), o, True, f"largest context row {t}")
        check_lse(np64(lse[0, t]), l, True, f"largest context row {t}")
    del kv
    torch.cuda.empty_cache()
