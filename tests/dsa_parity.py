"""Shared helpers of the GPU parity tests: device handling, conversion of the
synthetic inputs for the oracle, and the comparison rules.

Comparison rules
* index sets (selected tokens): the GPU row must hold n = min(k, #candidates)
  distinct in-range indices in ascending order followed by -1; its symmetric
  difference with the oracle's set may only contain tokens whose oracle score
  lies within 1e-3 relative of the oracle's k-th largest score (when that
  threshold is 0 the band is the exact zeros);
* top-k on identical fp32 inputs: bit-exact;
* attention outputs: the oracle recomputes attention on the GPU's own index
  set; bf16 must be within 2e-2 max-abs and 5e-3 mean-abs, fp32 within 1e-5
  max-abs;
* index scores: |gpu - oracle| <= c * S_abs + 2^-20 |oracle|, where
  S_abs[t,s] = sum_j |w q_scale|_j k_scale_s sum_d |q8_jd k8_d| is the sum of
  the magnitudes the dot products add up.  For FP8, c = 2^-14: gfx950's
  e4m3 MFMA sums the 128 exact products with truncation relative to the
  largest of them (measured: 65536 + 1 -> 65536; worst random-dot error
  6.4e-6 = 2^-17.3 of the magnitude sum), so the bound keeps a factor 8 of
  margin.  For the fp32 path, c = 2^-18 (a 32-term fp32 dot plus the head
  sum).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 5e-3
F32_MAX_ABS = 1e-5
BAND_REL = 1e-3


def gpu_device():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def np64(t):
    """Exact float64 copy of a CPU/GPU tensor (bf16/f32 widen exactly)."""
    if t is None:
        return None
    if t.dtype == torch.uint8:
        return t.detach().cpu().numpy()
    return t.detach().cpu().double().numpy()


def oracle_inputs(inp, b_sel=None):
    """numpy views of the inputs for the oracle (optionally batch entries b_sel)."""
    def pick(x):
        if x is None:
            return None
        if b_sel is not None:
            x = x[b_sel]
        return np64(x)
    return {k: pick(inp[k]) for k in ("q_idx", "q_idx_scale", "k_idx", "k_idx_scale", "w", "q", "kv")}


def to_device(inp, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def check_index_set(gpu_row, oracle_scores_row, oracle_sel, k, n_cand, where=""):
    """Index-set rule; returns True when the set equals the oracle's exactly."""
    g = np.asarray(gpu_row, dtype=np.int64)
    n = min(k, n_cand)
    sel = g[:n]
    assert np.all(g[n:] == -1), f"{where}: padding is not -1"
    assert np.all((sel >= 0) & (sel < n_cand)), f"{where}: index out of the causal range"
    assert np.all(np.diff(sel) > 0), f"{where}: indices not strictly ascending"
    o = np.asarray(oracle_sel, dtype=np.int64)[:n]
    diff = np.setxor1d(sel, o)
    if diff.size == 0:
        return True
    v = oracle_scores_row[:n_cand]
    thr = np.partition(v, n_cand - n)[n_cand - n] if n_cand > k else -np.inf
    dv = np.abs(oracle_scores_row[diff] - thr)
    ok = dv <= BAND_REL * abs(thr) if thr != 0 else oracle_scores_row[diff] == 0
    assert np.all(ok), (f"{where}: tokens {diff[~ok][:8]} differ from the oracle's selection with "
                        f"scores {oracle_scores_row[diff[~ok][:8]]} vs threshold {thr}")
    return False


def abs_score_sum(q_idx, k_idx, w, q_scale=None, k_scale=None):
    """S_abs[b,t,s] = sum_j |w_j| * (|Q_j| . |K_s|) with dequantised operands."""
    import oracle
    Q = np.abs(oracle.dequantize(q_idx, q_scale) if q_scale is not None else np.asarray(q_idx, np.float64))
    K = np.abs(oracle.dequantize(k_idx, k_scale) if k_scale is not None else np.asarray(k_idx, np.float64))
    W = np.abs(np.asarray(w, np.float64))
    return np.einsum("btj,btjd,bsd->bts", W, Q, K, optimize=True)


def check_scores(gpu, ref, s_abs, coeff, where=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape
    ninf_g, ninf_r = np.isneginf(gpu), np.isneginf(ref)
    assert np.array_equal(ninf_g, ninf_r), f"{where}: -inf pattern differs"
    fin = ~ninf_r
    tol = coeff * s_abs + 2.0 ** -20 * np.abs(np.where(fin, ref, 0))
    err = np.zeros_like(ref)
    err[fin] = np.abs(gpu[fin] - ref[fin])
    bad = err > np.where(fin, tol, 0)
    assert not bad.any(), (f"{where}: {bad.sum()} scores off; worst err {err.max():.3e}")
    return float((err / np.maximum(np.where(fin, s_abs, 1), 1e-300)).max())


def check_attention(gpu_out, ref_out, bf16: bool, where=""):
    d = np.abs(np.asarray(gpu_out, np.float64) - np.asarray(ref_out, np.float64))
    if bf16:
        assert d.max() <= BF16_MAX_ABS, f"{where}: max abs err {d.max():.3e}"
        assert d.mean() <= BF16_MEAN_ABS, f"{where}: mean abs err {d.mean():.3e}"
    else:
        assert d.max() <= F32_MAX_ABS, f"{where}: max abs err {d.max():.3e}"
    return float(d.max()), float(d.mean())


def check_lse(gpu_lse, ref_lse, bf16: bool, where=""):
    g = np.asarray(gpu_lse, np.float64)
    r = np.asarray(ref_lse, np.float64)
    assert np.array_equal(np.isneginf(g), np.isneginf(r)), f"{where}: lse -inf pattern differs"
    fin = ~np.isneginf(r)
    tol = 2e-2 if bf16 else 1e-5
    err = np.abs(g[fin] - r[fin]).max() if fin.any() else 0.0
    assert err <= tol, f"{where}: lse err {err:.3e}"
    return float(err)


def sample_rows(T, k, rng, extra=6):
    """Rows to check at full size: first, last, around k, and random ones."""
    rows = {0, T - 1}
    for t in (k - 2, k - 1, k, k + 1):
        if 0 <= t < T:
            rows.add(t)
    rows.update(int(x) for x in rng.integers(0, T, extra))
    return sorted(rows)


# ---- poisoned outputs and guarded buffers --------------------------------
GUARD_BYTES = 4096  # canary bytes before and after every guarded buffer
_CANARY = {1: (torch.uint8, 0x5A), 2: (torch.int16, 0x5A5A), 4: (torch.int32, 0x5A5A5A5A)}


class Guarded:
    """A device buffer of `shape` with canary bytes on both sides, its own
    elements poisoned with `fill` (NaN for floats: any element the call
    fails to write stays visible).  check() asserts that no canary byte
    changed.  Alignment: the buffer starts GUARD_BYTES into a fresh
    allocation, so it keeps the allocation's 256-byte alignment."""

    def __init__(self, shape, dtype, dev, fill):
        size = torch.tensor([], dtype=dtype).element_size()
        n = int(np.prod(shape))
        g = GUARD_BYTES // size
        self.full = torch.empty(n + 2 * g, dtype=dtype, device=dev)
        bits_dtype, canary = _CANARY[size]
        self.bits = self.full.view(bits_dtype)
        self.bits.fill_(canary)
        self.canary = canary
        self.g = g
        self.n = n
        self.view = self.full[g:g + n].view(shape)
        if n:
            if isinstance(fill, int) and dtype.is_floating_point:
                self.view.view(bits_dtype).fill_(fill)
            else:
                self.view.fill_(fill)

    def check(self, where=""):
        lo = self.bits[:self.g]
        hi = self.bits[self.g + self.n:]
        ok = bool((lo == self.canary).all()) and bool((hi == self.canary).all())
        assert ok, f"{where}: a write landed outside the buffer (canary changed)"


def poisoned_workspace(nbytes, dev):
    """A workspace whose bytes all start as 0xA5 (a NaN-free but absurd
    pattern for counters and keys), guarded on both sides."""
    return Guarded((max(int(nbytes), 1),), torch.uint8, dev, 0xA5)
