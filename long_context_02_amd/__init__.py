"""DeepSeek Sparse Attention (DSA) hot path on MI355X (gfx950).

Python binding of ``libdsa.so`` (C ABI in ``include/dsa.h``).  This module only
marshals arguments: it checks tensor devices, dtypes and shapes, allocates
outputs and workspaces with torch, and passes raw device pointers plus the
current HIP stream to the library.  Every step of the path runs in the HIP
kernels; there is no other implementation behind these functions, and they
raise if the library is missing.

Tensor layouts (contiguous, device tensors):
  q_idx  [B,T,H_I,d_I]  uint8 e4m3fn codes (or float8_e4m3fn) / float32
  q_idx_scale [B,T,H_I] float32 (FP8 only)
  k_idx  [B,N,d_I]      uint8 codes / float32
  k_idx_scale [B,N]     float32 (FP8 only)
  w      [B,T,H_I]      float32
  q      [B,T,H,d_qk]   bfloat16 / float32
  kv     [B,N,d_qk]     bfloat16 / float32
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "DSAError", "lib", "lib_path", "indexer_scores", "topk_select", "sparse_mla_attn",
    "forward", "indexer_select", "cache_append", "indexer_kl", "workspace_size", "OP_TOPK", "OP_ATTN", "OP_FORWARD",
    "OP_SELECT", "OP_ATTN_BWD", "OP_ATTN_MHA", "sparse_mla_attn_bwd", "sparse_mla_attn_mha",
    "kernel_times", "probe_peaks",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdsa.so")

OP_TOPK, OP_ATTN, OP_FORWARD, OP_SELECT, OP_ATTN_BWD, OP_ATTN_MHA = 0, 1, 2, 3, 4, 5
F32, BF16, FP8_E4M3FN = 0, 1, 2

_STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED",
           3: "DSA_ERR_WORKSPACE", 4: "DSA_ERR_BAD_INDEX", 5: "DSA_ERR_HIP"}

_lib = None


class _KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int), ("total_ms", ctypes.c_double)]


class DSAError(RuntimeError):
    """A libdsa call returned a status other than DSA_OK."""

    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().dsa_status_string(status).decode()
        super().__init__(f"{fn}: {msg}")


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libdsa.so (built by ``python -m long_context_02_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m long_context_02_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    vp, fp, i32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    ci, cf, sz = ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.dsa_indexer_scores.argtypes = [vp, fp, vp, fp, fp, fp, ci, ci, ci, ci, ci, ci, ci, vp]
    L.dsa_indexer_scores.restype = ci
    L.dsa_topk_select.argtypes = [fp, i32p, ci, ci, ci, ci, ci, vp, sz, vp]
    L.dsa_topk_select.restype = ci
    L.dsa_sparse_mla_attn.argtypes = [vp, vp, i32p, vp, fp, ci, ci, ci, ci, ci, ci, ci, cf, ci, vp, sz, vp]
    L.dsa_sparse_mla_attn.restype = ci
    L.dsa_sparse_mla_attn_bwd.argtypes = [vp, vp, i32p, vp, fp, vp, fp, fp, ci, ci, ci, ci, ci, ci, ci,
                                          cf, ci, vp, sz, vp]
    L.dsa_sparse_mla_attn_bwd.restype = ci
    L.dsa_sparse_mla_attn_mha.argtypes = [vp, vp, vp, vp, i32p, vp, fp, ci, ci, ci, ci, ci, ci, ci, ci,
                                          ci, cf, ci, vp, sz, vp]
    L.dsa_sparse_mla_attn_mha.restype = ci
    L.dsa_forward.argtypes = [vp, fp, vp, fp, fp, vp, vp, vp, fp, i32p,
                              ci, ci, ci, ci, ci, ci, ci, ci, ci, ci, cf, ci, ci, vp, sz, vp]
    L.dsa_forward.restype = ci
    L.dsa_indexer_select.argtypes = [vp, fp, vp, fp, fp, i32p, ci, ci, ci, ci, ci, ci, ci, ci, vp, sz, vp]
    L.dsa_indexer_select.restype = ci
    L.dsa_cache_append.argtypes = [fp, vp, vp, fp, vp, i32p, ci, ci, ci, ci, ci, ci, ci, vp]
    L.dsa_cache_append.restype = ci
    L.dsa_indexer_kl.argtypes = [fp, fp, i32p, fp, fp, ci, ci, ci, ci, ci, vp]
    L.dsa_indexer_kl.restype = ci
    L.dsa_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci]
    L.dsa_workspace_size.restype = sz
    L.dsa_profile_start.argtypes = [ci]
    L.dsa_profile_start.restype = ci
    L.dsa_profile_stop.argtypes = [ctypes.POINTER(_KernelTime), ci, ctypes.POINTER(ci)]
    L.dsa_profile_stop.restype = ci
    L.dsa_probe_peak.argtypes = [ci, vp, sz, vp]
    L.dsa_probe_peak.restype = ctypes.c_double
    L.dsa_status_string.argtypes = [ci]
    L.dsa_status_string.restype = ctypes.c_char_p
    L.dsa_version.argtypes = []
    L.dsa_version.restype = ci
    _lib = L
    return L


# ---------------------------------------------------------------------------
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check(name, t, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _codes(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


def _idx_dtype(q_idx: torch.Tensor) -> int:
    if q_idx.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3FN
    if q_idx.dtype == torch.float32:
        return F32
    raise TypeError(f"indexer operands must be uint8/float8_e4m3fn codes or float32, got {q_idx.dtype}")


def _attn_dtype(q: torch.Tensor) -> int:
    if q.dtype == torch.bfloat16:
        return BF16
    if q.dtype == torch.float32:
        return F32
    raise TypeError(f"attention operands must be bfloat16 or float32, got {q.dtype}")


def _raise(fn, st):
    if st != 0:
        raise DSAError(fn, st)


def workspace_size(op: int, B: int, T: int, N: int, H_I: int, H: int, d_v: int, k: int) -> int:
    n = lib().dsa_workspace_size(op, B, T, N, H_I, H, d_v, k)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("dsa_workspace_size: invalid arguments")
    return n


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if nbytes == 0:
        return workspace
    if workspace is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    _check("workspace", workspace, None, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace too small: need {nbytes} bytes")
    return workspace


def _indexer_args(q_idx, k_idx, w, q_idx_scale, k_idx_scale):
    dt = _idx_dtype(q_idx)
    dev = q_idx.device
    B, T, H_I, d_I = q_idx.shape
    N = k_idx.shape[1]
    if dt == FP8_E4M3FN:
        q_idx, k_idx = _codes(q_idx), _codes(k_idx)
        _check("q_idx", q_idx, torch.uint8, (B, T, H_I, d_I), dev)
        _check("k_idx", k_idx, torch.uint8, (B, N, d_I), dev)
        if q_idx_scale is None or k_idx_scale is None:
            raise ValueError("FP8 indexer operands need q_idx_scale and k_idx_scale")
        _check("q_idx_scale", q_idx_scale, torch.float32, (B, T, H_I), dev)
        _check("k_idx_scale", k_idx_scale, torch.float32, (B, N), dev)
    else:
        _check("q_idx", q_idx, torch.float32, (B, T, H_I, d_I), dev)
        _check("k_idx", k_idx, torch.float32, (B, N, d_I), dev)
        if q_idx_scale is not None or k_idx_scale is not None:
            raise ValueError("float32 indexer operands take no scales")
    _check("w", w, torch.float32, (B, T, H_I), dev)
    return dt, q_idx, k_idx, (B, T, N, H_I, d_I)


def indexer_scores(q_idx, k_idx, w, q_offset: int, q_idx_scale=None, k_idx_scale=None,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Lightning-indexer scores [B,T,N] float32 (-inf outside the causal set)."""
    dt, q_idx, k_idx, (B, T, N, H_I, d_I) = _indexer_args(q_idx, k_idx, w, q_idx_scale, k_idx_scale)
    dev = q_idx.device
    if out is None:
        out = torch.empty(B, T, N, dtype=torch.float32, device=dev)
    _check("out", out, torch.float32, (B, T, N), dev)
    with torch.cuda.device(dev):
        st = lib().dsa_indexer_scores(_ptr(q_idx), _ptr(q_idx_scale), _ptr(k_idx), _ptr(k_idx_scale),
                                      _ptr(w), _ptr(out), B, T, N, H_I, d_I, q_offset, dt, _stream(dev))
    _raise("dsa_indexer_scores", st)
    return out


def indexer_select(q_idx, k_idx, w, k: int, q_offset: int, q_idx_scale=None, k_idx_scale=None,
                   out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Index scores and top-k selection in one call: int32 [B,T,k] ascending
    token indices, -1 padded (the scores are not returned)."""
    dt, q_idx, k_idx, (B, T, N, H_I, d_I) = _indexer_args(q_idx, k_idx, w, q_idx_scale, k_idx_scale)
    dev = q_idx.device
    if out is None:
        out = torch.empty(B, T, k, dtype=torch.int32, device=dev)
    _check("out", out, torch.int32, (B, T, k), dev)
    need = workspace_size(OP_SELECT, B, T, N, H_I, 1, 1, k) if 1 <= k <= 2048 else 0
    ws = _workspace(need, dev, workspace)
    with torch.cuda.device(dev):
        st = lib().dsa_indexer_select(_ptr(q_idx), _ptr(q_idx_scale), _ptr(k_idx), _ptr(k_idx_scale),
                                      _ptr(w), _ptr(out), B, T, N, H_I, d_I, k, q_offset, dt, _ptr(ws),
                                      0 if ws is None else ws.numel() * ws.element_size(), _stream(dev))
    _raise("dsa_indexer_select", st)
    return out


def topk_select(scores: torch.Tensor, k: int, q_offset: int, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Ascending top-k token indices per row, -1 padded: int32 [B,T,k]."""
    dev = scores.device
    _check("scores", scores, torch.float32, None, dev)
    B, T, N = scores.shape
    if out is None:
        out = torch.empty(B, T, k, dtype=torch.int32, device=dev)
    _check("out", out, torch.int32, (B, T, k), dev)
    need = workspace_size(OP_TOPK, B, T, N, 1, 1, 1, k) if 1 <= k <= 2048 else 0
    ws = _workspace(need, dev, workspace)
    with torch.cuda.device(dev):
        st = lib().dsa_topk_select(_ptr(scores), _ptr(out), B, T, N, k, q_offset, _ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(), _stream(dev))
    _raise("dsa_topk_select", st)
    return out


def sparse_mla_attn(q, kv, idx, d_v: int, sm_scale: float, out=None, lse: Optional[bool] = True,
                    workspace: Optional[torch.Tensor] = None):
    """Sparse MQA attention.  Returns (out [B,T,H,d_v], lse [B,T,H] or None)."""
    dt = _attn_dtype(q)
    dev = q.device
    B, T, H, d_qk = q.shape
    N = kv.shape[1]
    k = idx.shape[-1]
    _check("q", q, q.dtype, (B, T, H, d_qk), dev)
    _check("kv", kv, q.dtype, (B, N, d_qk), dev)
    _check("idx", idx, torch.int32, (B, T, k), dev)
    if out is None:
        out = torch.empty(B, T, H, d_v, dtype=q.dtype, device=dev)
    _check("out", out, q.dtype, (B, T, H, d_v), dev)
    lse_t = None
    if isinstance(lse, torch.Tensor):
        lse_t = lse
        _check("lse", lse_t, torch.float32, (B, T, H), dev)
    elif lse:
        lse_t = torch.empty(B, T, H, dtype=torch.float32, device=dev)
    need = workspace_size(OP_ATTN, B, T, N, 1, H, d_v, k) if 1 <= k <= 2048 else 0
    ws = _workspace(need, dev, workspace)
    with torch.cuda.device(dev):
        st = lib().dsa_sparse_mla_attn(_ptr(q), _ptr(kv), _ptr(idx), _ptr(out), _ptr(lse_t),
                                       B, T, N, H, d_qk, d_v, k, float(sm_scale), dt, _ptr(ws),
                                       0 if ws is None else ws.numel() * ws.element_size(),
                                       _stream(dev))
    _raise("dsa_sparse_mla_attn", st)
    return out, lse_t


def sparse_mla_attn_mha(q, kv, w_uk, w_uv, idx, sm_scale: float, out=None,
                        lse: Optional[bool] = True, workspace: Optional[torch.Tensor] = None):
    """Sparse MLA attention in MHA mode (bf16): every head attends over its
    own keys [W_UK[h] c[:d_c] ; c[d_c:]] and values W_UV[h] c[:d_c] of the
    selected latent rows.  q [B,T,H,d_n+d_r], kv [B,N,d_c+d_r],
    w_uk [H,d_n,d_c], w_uv [H,d_vh,d_c], idx [B,T,k] int32.
    Returns (out [B,T,H,d_vh], lse [B,T,H] or None)."""
    dev = q.device
    B, T, H, dq_ = q.shape
    N, d_lat = kv.shape[1], kv.shape[2]
    k = idx.shape[-1]
    d_n, d_c = w_uk.shape[1], w_uk.shape[2]
    d_vh = w_uv.shape[1]
    d_r = d_lat - d_c
    _check("q", q, torch.bfloat16, (B, T, H, dq_), dev)
    _check("kv", kv, torch.bfloat16, (B, N, d_lat), dev)
    _check("w_uk", w_uk, torch.bfloat16, (H, d_n, d_c), dev)
    _check("w_uv", w_uv, torch.bfloat16, (H, d_vh, d_c), dev)
    _check("idx", idx, torch.int32, (B, T, k), dev)
    if dq_ != d_n + d_r:
        raise ValueError(f"q has width {dq_}, expected d_n + d_r = {d_n + d_r}")
    if out is None:
        out = torch.empty(B, T, H, d_vh, dtype=torch.bfloat16, device=dev)
    _check("out", out, torch.bfloat16, (B, T, H, d_vh), dev)
    lse_t = lse if isinstance(lse, torch.Tensor) else (
        torch.empty(B, T, H, dtype=torch.float32, device=dev) if lse else None)
    if lse_t is not None:
        _check("lse", lse_t, torch.float32, (B, T, H), dev)
    need = workspace_size(OP_ATTN_MHA, B, T, N, 1, H, d_vh, k) if (1 <= k <= 2048 and H == 128
                                                                   and d_vh == 128) else 0
    ws = _workspace(need, dev, workspace)
    with torch.cuda.device(dev):
        st = lib().dsa_sparse_mla_attn_mha(_ptr(q), _ptr(kv), _ptr(w_uk), _ptr(w_uv), _ptr(idx),
                                           _ptr(out), _ptr(lse_t), B, T, N, H, d_c, d_r, d_n, d_vh, k,
                                           float(sm_scale), BF16, _ptr(ws),
                                           0 if ws is None else ws.numel() * ws.element_size(),
                                           _stream(dev))
    _raise("dsa_sparse_mla_attn_mha", st)
    return out, lse_t


def sparse_mla_attn_bwd(q, kv, idx, out, lse, dout, sm_scale: float, dq=None, dkv=None,
                        workspace: Optional[torch.Tensor] = None):
    """Gradients of sparse MQA attention (bf16).  Takes the forward's inputs,
    its output and log-sum-exp and the output gradient; returns
    (dq [B,T,H,d_qk] f32, dkv [B,N,d_qk] f32)."""
    dt = _attn_dtype(q)
    dev = q.device
    B, T, H, d_qk = q.shape
    N = kv.shape[1]
    k = idx.shape[-1]
    d_v = out.shape[-1]
    _check("q", q, q.dtype, (B, T, H, d_qk), dev)
    _check("kv", kv, q.dtype, (B, N, d_qk), dev)
    _check("idx", idx, torch.int32, (B, T, k), dev)
    _check("out", out, q.dtype, (B, T, H, d_v), dev)
    _check("lse", lse, torch.float32, (B, T, H), dev)
    _check("dout", dout, q.dtype, (B, T, H, d_v), dev)
    if dq is None:
        dq = torch.empty(B, T, H, d_qk, dtype=torch.float32, device=dev)
    if dkv is None:
        dkv = torch.empty(B, N, d_qk, dtype=torch.float32, device=dev)
    _check("dq", dq, torch.float32, (B, T, H, d_qk), dev)
    _check("dkv", dkv, torch.float32, (B, N, d_qk), dev)
    need = workspace_size(OP_ATTN_BWD, B, T, N, 1, H, d_v, k) if 1 <= k <= 2048 else 0
    ws = _workspace(need, dev, workspace)
    with torch.cuda.device(dev):
        st = lib().dsa_sparse_mla_attn_bwd(_ptr(q), _ptr(kv), _ptr(idx), _ptr(out), _ptr(lse),
                                           _ptr(dout), _ptr(dq), _ptr(dkv), B, T, N, H, d_qk, d_v, k,
                                           float(sm_scale), dt, _ptr(ws),
                                           0 if ws is None else ws.numel() * ws.element_size(),
                                           _stream(dev))
    _raise("dsa_sparse_mla_attn_bwd", st)
    return dq, dkv


def forward(q_idx, k_idx, w, q, kv, *, k: int, q_offset: int, d_v: int, sm_scale: float,
            q_idx_scale=None, k_idx_scale=None, out=None, lse: Optional[bool] = False,
            idx_out: Optional[bool] = False, workspace: Optional[torch.Tensor] = None):
    """The fused DSA path: index scores -> top-k -> sparse MQA attention.

    Returns (out, lse or None, idx or None).
    """
    idt, q_idx, k_idx, (B, T, N, H_I, d_I) = _indexer_args(q_idx, k_idx, w, q_idx_scale, k_idx_scale)
    adt = _attn_dtype(q)
    dev = q_idx.device
    H, d_qk = q.shape[2], q.shape[3]
    _check("q", q, q.dtype, (B, T, H, d_qk), dev)
    _check("kv", kv, q.dtype, (B, N, d_qk), dev)
    if out is None:
        out = torch.empty(B, T, H, d_v, dtype=q.dtype, device=dev)
    _check("out", out, q.dtype, (B, T, H, d_v), dev)
    lse_t = lse if isinstance(lse, torch.Tensor) else (
        torch.empty(B, T, H, dtype=torch.float32, device=dev) if lse else None)
    idx_t = idx_out if isinstance(idx_out, torch.Tensor) else (
        torch.empty(B, T, k, dtype=torch.int32, device=dev) if idx_out else None)
    if idx_t is not None:
        _check("idx_out", idx_t, torch.int32, (B, T, k), dev)
    need = workspace_size(OP_FORWARD, B, T, N, H_I, H, d_v, k)
    ws = _workspace(need, dev, workspace)
    with torch.cuda.device(dev):
        st = lib().dsa_forward(_ptr(q_idx), _ptr(q_idx_scale), _ptr(k_idx), _ptr(k_idx_scale), _ptr(w),
                               _ptr(q), _ptr(kv), _ptr(out), _ptr(lse_t), _ptr(idx_t),
                               B, T, N, H_I, d_I, H, d_qk, d_v, k, q_offset, float(sm_scale), idt, adt,
                               _ptr(ws), ws.numel() * ws.element_size(), _stream(dev))
    _raise("dsa_forward", st)
    return out, lse_t, idx_t


def cache_append(k_new: torch.Tensor, kv_new: torch.Tensor, k_cache: torch.Tensor,
                 k_cache_scale: Optional[torch.Tensor], kv_cache: torch.Tensor,
                 pos: torch.Tensor) -> None:
    """Write new tokens into the caches in place: token t of sequence b goes
    to row pos[b] + t (rows outside [0, N) are dropped).  FP8 key caches
    (uint8 codes with float32 per-token scales) get the keys quantised with
    scale = amax / 448; float32 key caches and the latent cache get copies.

    k_new [B,T,d_I] float32, kv_new [B,T,d_qk] (kv_cache's dtype),
    k_cache [B,N,d_I] uint8/float8_e4m3fn or float32, k_cache_scale [B,N]
    float32 (FP8 only, else None), kv_cache [B,N,d_qk] bfloat16/float32,
    pos [B] int32 (device)."""
    dev = k_new.device
    _check("k_new", k_new, torch.float32, None, dev)
    B, T, d_I = k_new.shape
    idt = _idx_dtype(k_cache)
    _check("k_cache", k_cache, None, None, dev)
    N = k_cache.shape[1]
    if k_cache.dim() != 3 or k_cache.shape[0] != B or k_cache.shape[2] != d_I:
        raise ValueError(f"k_cache has shape {tuple(k_cache.shape)}, expected ({B}, N, {d_I})")
    if idt == FP8_E4M3FN:
        _check("k_cache_scale", k_cache_scale, torch.float32, (B, N), dev)
    elif k_cache_scale is not None:
        raise ValueError("k_cache_scale must be None for a float32 key cache")
    adt = _attn_dtype(kv_cache)
    _check("kv_cache", kv_cache, None, None, dev)
    if kv_cache.dim() != 3 or kv_cache.shape[:2] != (B, N):
        raise ValueError(f"kv_cache has shape {tuple(kv_cache.shape)}, expected ({B}, {N}, d_qk)")
    d_qk = kv_cache.shape[2]
    _check("kv_new", kv_new, kv_cache.dtype, (B, T, d_qk), dev)
    _check("pos", pos, torch.int32, (B,), dev)
    with torch.cuda.device(dev):
        st = lib().dsa_cache_append(_ptr(k_new), _ptr(kv_new), _ptr(_codes(k_cache)), _ptr(k_cache_scale),
                                    _ptr(kv_cache), _ptr(pos), B, T, N, d_I, d_qk, idt, adt, _stream(dev))
    _raise("dsa_cache_append", st)


def indexer_kl(scores: torch.Tensor, p: torch.Tensor, q_offset: int = 0,
               idx: Optional[torch.Tensor] = None, grad: bool = True):
    """KL(p || softmax(I)) per row and its gradient with respect to the
    scores: dense over the causal candidates (idx None; p [B,T,N], gradient
    [B,T,N]) or over the selected slots (idx [B,T,k]; p [B,T,k], gradient
    [B,T,k]).  Returns (loss [B,T], grad or None)."""
    dev = scores.device
    _check("scores", scores, torch.float32, None, dev)
    B, T, N = scores.shape
    if idx is None:
        _check("p", p, torch.float32, (B, T, N), dev)
        k = 0
        gshape = (B, T, N)
    else:
        _check("idx", idx, torch.int32, None, dev)
        if idx.dim() != 3 or idx.shape[:2] != (B, T):
            raise ValueError(f"idx has shape {tuple(idx.shape)}, expected ({B}, {T}, k)")
        k = idx.shape[2]
        _check("p", p, torch.float32, (B, T, k), dev)
        gshape = (B, T, k)
    loss = torch.empty(B, T, dtype=torch.float32, device=dev)
    g = torch.empty(gshape, dtype=torch.float32, device=dev) if grad else None
    with torch.cuda.device(dev):
        st = lib().dsa_indexer_kl(_ptr(scores), _ptr(p), _ptr(idx), _ptr(loss), _ptr(g), B, T, N, k,
                                  q_offset, _stream(dev))
    _raise("dsa_indexer_kl", st)
    return loss, g


def kernel_times(fn, max_launches: int = 8192) -> dict:
    """Run fn() with the library's per-kernel timing window open (HIP events
    recorded around every kernel launch on its stream) and return
    {kernel name: (launches, total milliseconds)}."""
    L = lib()
    _raise("dsa_profile_start", L.dsa_profile_start(max_launches))
    try:
        fn()
    finally:
        entries = (_KernelTime * 64)()
        dropped = ctypes.c_int(0)
        n = L.dsa_profile_stop(entries, 64, ctypes.byref(dropped))
    if n < 0:
        raise RuntimeError("dsa_profile_stop failed")
    if dropped.value:
        raise RuntimeError(f"{dropped.value} launches beyond the timing window of {max_launches}")
    return {entries[i].name.decode(): (entries[i].launches, entries[i].total_ms) for i in range(n)}


def probe_peaks(device=None, read_mib: int = 2048) -> dict:
    """What this GPU sustains: a streaming read over read_mib MiB (GB/s) and
    back-to-back bf16 and FP8 MFMAs (TFLOP/s), from the library's probes."""
    dev = torch.device(device or "cuda")
    buf = torch.empty(read_mib << 20, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    L = lib()
    with torch.cuda.device(dev):
        s = _stream(dev)
        res = {"stream_read_gbs": L.dsa_probe_peak(0, _ptr(buf), buf.numel(), s),
               "mfma_bf16_tflops": L.dsa_probe_peak(1, _ptr(buf), buf.numel(), s),
               "mfma_fp8_tflops": L.dsa_probe_peak(2, _ptr(buf), buf.numel(), s),
               "mfma_bf16_32x32_tflops": L.dsa_probe_peak(3, _ptr(buf), buf.numel(), s)}
    del buf
    for k, v in res.items():
        if v < 0:
            raise RuntimeError(f"dsa_probe_peak failed for {k}")
    return {k: round(v, 1) for k, v in res.items()}
