"""Seeded synthetic inputs for the DSA path.

This module only draws random tensors and lays them out the way the library
expects; it computes no part of the method.  Both the oracle-side tests and
the HIP-side tests/bench take their inputs from here, so the two sides always
see the same bytes.

The indexer operands of the bf16 workloads are FP8 e4m3fn codes with one fp32
scale per token, produced as the workload recipe says: draw N(0,1) source
values, take the token's absolute maximum a, set scale = a/448 (1 if a = 0),
and cast source/scale to e4m3fn with torch's own round-to-nearest-even cast
after clamping to +-448.  For the query this scale is per token and is
replicated over the indexer heads.

Random numbers come from ``torch.Generator`` seeded per tensor with
``seed * 16 + tensor_id``; on a GPU device the stream differs from the CPU one
but is just as deterministic.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional, Tuple

import torch

E4M3_MAX = 448.0

# tensor ids inside one seed
_QI, _KI, _W, _Q, _KV, _ROWS, _QM, _WUK, _WUV = range(9)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    N: int
    q_offset: int
    H_I: int
    d_I: int
    k: int
    H: int
    d_qk: int
    d_v: int
    dtype: str                 # "f32" (raw fp32 indexer + attention) or "bf16" (FP8 indexer + bf16 attention)
    w_scale: float = 1.0       # w ~ U(0,1) * w_scale
    idx_src_std: float = 1.0   # indexer source values ~ N(0, idx_src_std^2)
    heavy_rows: int = 0        # number of k^I rows scaled by heavy_factor before quantisation
    heavy_factor: float = 8.0
    local_bias: Optional[Tuple[int, int, float]] = None  # (start, stop, add) on k^I source rows

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)

    @property
    def query_tokens(self) -> int:
        return self.B * self.T

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the DSA path.
WORKLOADS = {
    # fp32 prefill, L = 256
    "tiny": Workload("tiny", B=1, T=256, N=256, q_offset=0, H_I=4, d_I=32, k=64,
                     H=16, d_qk=80, d_v=64, dtype="f32", idx_src_std=1.0 / math.sqrt(32)),
    # bf16 prefill, L = 8192
    "prefill_8k": Workload("prefill_8k", B=1, T=8192, N=8192, q_offset=0, H_I=8, d_I=128,
                           k=2048, H=128, d_qk=576, d_v=512, dtype="bf16", w_scale=1.0 / 8),
    # bf16 prefill, L = 32768, 1% heavy-tailed indexer keys
    "prefill_32k": Workload("prefill_32k", B=1, T=32768, N=32768, q_offset=0, H_I=8, d_I=128,
                            k=2048, H=128, d_qk=576, d_v=512, dtype="bf16", w_scale=1.0 / 8,
                            heavy_rows=328),
    # decode: 64 sequences x 1 new token against 131072 cached tokens
    "decode_128k": Workload("decode_128k", B=64, T=1, N=131072, q_offset=131071, H_I=8, d_I=128,
                            k=2048, H=128, d_qk=576, d_v=512, dtype="bf16", w_scale=1.0 / 8),
    # chunked prefill: 4096 new tokens on a 126976-token cache (total 131072)
    "chunk_128k": Workload("chunk_128k", B=1, T=4096, N=131072, q_offset=126976, H_I=8, d_I=128,
                           k=2048, H=128, d_qk=576, d_v=512, dtype="bf16", w_scale=1.0 / 8,
                           local_bias=(130560, 131072, 2.0)),
}


def _gen(device, seed: int, tid: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 16 + tid)
    return g


def quantize_rows_e4m3(src: torch.Tensor, group_dims: int):
    """Per-row FP8 e4m3fn quantisation of ``src`` (the input recipe).

    The last ``group_dims`` dimensions share one scale = amax / 448.
    Returns (codes uint8 with src's shape, scale float32 with the leading shape).
    """
    lead = src.shape[: src.dim() - group_dims]
    flat = src.reshape(*lead, -1).float()
    amax = flat.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    x = (flat / scale[..., None]).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = x.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.reshape(src.shape), scale.float()


def make_inputs(wl: Workload, seed: int = 0, device="cpu", chunk_tokens: int = 1 << 16):
    """All inputs of one DSA call for workload ``wl``.

    Returns a dict with keys q_idx, q_idx_scale, k_idx, k_idx_scale, w, q, kv
    (scales are None for the fp32 workload) laid out as
    q_idx [B,T,H_I,d_I], q_idx_scale [B,T,H_I], k_idx [B,N,d_I],
    k_idx_scale [B,N], w [B,T,H_I], q [B,T,H,d_qk], kv [B,N,d_qk].
    Large tensors are generated in chunks of ``chunk_tokens`` tokens to bound
    temporary memory.
    """
    dev = torch.device(device)
    B, T, N = wl.B, wl.T, wl.N
    out = {}
    if wl.dtype == "f32":
        g = _gen(dev, seed, _QI)
        out["q_idx"] = torch.randn(B, T, wl.H_I, wl.d_I, generator=g, device=dev) * wl.idx_src_std
        g = _gen(dev, seed, _KI)
        out["k_idx"] = torch.randn(B, N, wl.d_I, generator=g, device=dev) * wl.idx_src_std
        out["q_idx_scale"] = None
        out["k_idx_scale"] = None
        g = _gen(dev, seed, _W)
        out["w"] = torch.rand(B, T, wl.H_I, generator=g, device=dev) * wl.w_scale
        g = _gen(dev, seed, _Q)
        out["q"] = torch.randn(B, T, wl.H, wl.d_qk, generator=g, device=dev)
        g = _gen(dev, seed, _KV)
        out["kv"] = torch.randn(B, N, wl.d_qk, generator=g, device=dev)
        return out

    # FP8 indexer operands
    g = _gen(dev, seed, _QI)
    q_codes = torch.empty(B, T, wl.H_I, wl.d_I, dtype=torch.uint8, device=dev)
    q_scale = torch.empty(B, T, dtype=torch.float32, device=dev)
    for b in range(B):
        for t0 in range(0, T, chunk_tokens):
            t1 = min(T, t0 + chunk_tokens)
            src = torch.randn(t1 - t0, wl.H_I, wl.d_I, generator=g, device=dev) * wl.idx_src_std
            q_codes[b, t0:t1], q_scale[b, t0:t1] = quantize_rows_e4m3(src, 2)
    out["q_idx"] = q_codes
    out["q_idx_scale"] = q_scale[..., None].expand(B, T, wl.H_I).contiguous()

    g = _gen(dev, seed, _KI)
    gr = _gen(dev, seed, _ROWS)
    heavy = None
    if wl.heavy_rows:
        heavy = torch.randperm(N, generator=gr, device=dev)[: wl.heavy_rows]
    k_codes = torch.empty(B, N, wl.d_I, dtype=torch.uint8, device=dev)
    k_scale = torch.empty(B, N, dtype=torch.float32, device=dev)
    for b in range(B):
        for s0 in range(0, N, chunk_tokens):
            s1 = min(N, s0 + chunk_tokens)
            src = torch.randn(s1 - s0, wl.d_I, generator=g, device=dev) * wl.idx_src_std
            if heavy is not None:
                sel = heavy[(heavy >= s0) & (heavy < s1)] - s0
                src[sel] *= wl.heavy_factor
            if wl.local_bias is not None:
                a, z, add = wl.local_bias
                lo, hi = max(a, s0), min(z, s1)
                if lo < hi:
                    src[lo - s0:hi - s0] += add
            k_codes[b, s0:s1], k_scale[b, s0:s1] = quantize_rows_e4m3(src, 1)
    out["k_idx"] = k_codes
    out["k_idx_scale"] = k_scale
    out["heavy_rows"] = heavy

    g = _gen(dev, seed, _W)
    out["w"] = torch.rand(B, T, wl.H_I, generator=g, device=dev) * wl.w_scale

    g = _gen(dev, seed, _Q)
    out["q"] = torch.randn(B, T, wl.H, wl.d_qk, generator=g, device=dev, dtype=torch.bfloat16)
    g = _gen(dev, seed, _KV)
    kv = torch.empty(B, N, wl.d_qk, device=dev, dtype=torch.bfloat16)
    for b in range(B):
        for s0 in range(0, N, chunk_tokens):
            s1 = min(N, s0 + chunk_tokens)
            kv[b, s0:s1] = torch.randn(s1 - s0, wl.d_qk, generator=g, device=dev,
                                       dtype=torch.bfloat16)
    out["kv"] = kv
    return out


# MLA's MHA mode: per-head query width d_n + d_r (nope + rope), per-head
# value width d_vh, and the up-projections of the d_c-wide latent part.
MHA_D_N, MHA_D_R, MHA_D_VH = 128, 64, 128


def make_mha_inputs(wl: Workload, seed: int = 0, device="cpu"):
    """Extra inputs of sparse attention in MHA mode for a bf16 workload.

    Returns q_mha [B,T,H,d_n+d_r] ~ N(0,1), w_uk [H,d_n,d_c] and
    w_uv [H,d_vh,d_c] ~ N(0,1/d_c) (so the up-projected keys and values have
    unit variance), all bfloat16, with d_c = wl.d_v (the latent width) and
    sm_scale 1/sqrt(d_n + d_r).  The latent entries are make_inputs()' kv.
    """
    dev = torch.device(device)
    d_c = wl.d_v
    out = {}
    g = _gen(dev, seed, _QM)
    out["q_mha"] = torch.randn(wl.B, wl.T, wl.H, MHA_D_N + MHA_D_R, generator=g, device=dev,
                               dtype=torch.bfloat16)
    g = _gen(dev, seed, _WUK)
    out["w_uk"] = (torch.randn(wl.H, MHA_D_N, d_c, generator=g, device=dev) / math.sqrt(d_c)).to(torch.bfloat16)
    g = _gen(dev, seed, _WUV)
    out["w_uv"] = (torch.randn(wl.H, MHA_D_VH, d_c, generator=g, device=dev) / math.sqrt(d_c)).to(torch.bfloat16)
    out["sm_scale_mha"] = 1.0 / math.sqrt(MHA_D_N + MHA_D_R)
    return out
