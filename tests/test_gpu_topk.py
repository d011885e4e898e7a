"""GPU parity of dsa_topk_select: bit-exact against the oracle's selection
on the very same fp32 score rows.

Batches of at most 255 rows take the segmented path (several workgroups per
row), larger ones one workgroup per row; every case is run both ways by also
selecting on the rows repeated into a batch of 256 or more."""
import numpy as np
import pytest
import torch

import long_context_02_amd as dsa
import oracle
from dsa_parity import gpu_device

pytestmark = pytest.mark.gpu


ROWS_SEGMENTED = 255


def _check(scores_cpu, k, q_offset, where):
    dev = gpu_device()
    B, T, _ = scores_cpu.shape
    ref = oracle.topk_select(scores_cpu.double().numpy(), k, q_offset)
    reps = [1, -(-(ROWS_SEGMENTED + 1) // (B * T))] if B * T <= ROWS_SEGMENTED else [1]
    for r in reps:
        print(f"[topk] {where} rows={B * T * r}", flush=True)
        s = scores_cpu.repeat(r, 1, 1).to(dev)
        got = dsa.topk_select(s, k, q_offset).cpu().numpy()
        for c in range(r):
            g = got[c * B:(c + 1) * B]
            bad = np.flatnonzero((g != ref).any(axis=-1).ravel())
            assert bad.size == 0, f"{where} rows={B * T * r}: {bad.size} rows differ, first row {bad[0]}"


def _gen(seed):
    return torch.Generator().manual_seed(seed)


@pytest.mark.parametrize("B,T,N,k,q_offset", [
    (1, 64, 5000, 2048, 4936),      # chunk-like rows, many thousands of candidates
    (2, 40, 3001, 512, 2961),       # N not a multiple of 4 (scalar loads)
    (1, 300, 300, 64, 0),           # prefill: rows with fewer than k candidates
    (3, 1, 131072, 2048, 131071),   # decode-length rows
    (1, 8, 4000, 1, 3992),          # k = 1
])
def test_random_rows(B, T, N, k, q_offset):
    s = torch.randn(B, T, N, generator=_gen(N + k)).abs()
    _check(s, k, q_offset, f"random B={B} T={T} N={N} k={k}")


@pytest.mark.parametrize("N", [6000, 20000])
def test_ties_zeros_signed_zero_nan(N):
    g = _gen(5)
    T = 32
    s = torch.randint(0, 4, (1, T, N), generator=g).float() * 0.5  # heavy exact ties
    s[torch.rand(1, T, N, generator=g) < 0.3] = 0.0
    s[torch.rand(1, T, N, generator=g) < 0.1] = -0.0
    s[torch.rand(1, T, N, generator=g) < 0.02] = float("nan")
    s[0, 3] = float("nan")                     # a row of NaN only
    _check(s, 2048, N - T, "ties")


def test_one_bin_overflow_fallback():
    """Scores that share their top 12 key bits overflow the LDS candidate list
    and take the HBM fallback."""
    g = _gen(6)
    s = 1.0 + torch.rand(1, 8, 20000, generator=g) * 0.1
    s[0, 1] = 0.25                               # all equal
    s[0, 2, ::3] = 1.0                           # many exact ties at the threshold
    _check(s, 2048, 20000 - 8, "one-bin")


def test_decode_rows_ties_and_one_bin():
    """Decode-length rows: a threshold value shared by ~2000 tokens (ties
    resolved by index), and rows whose threshold bin overflows the segmented
    path's candidate list."""
    g = _gen(8)
    N = 131072
    s = torch.randint(0, 64, (1, 4, N), generator=g).float() / 8.0
    s[0, 2] = 0.5                               # one value everywhere
    s[0, 3] = 1.0 + torch.rand(N, generator=g) * 0.1  # all keys in one bin
    _check(s, 2048, N - 4, "decode ties")


@pytest.mark.parametrize("B,T,N,k,q_offset", [
    (1, 400, 8400, 2048, 7999),     # rows on both sides of 8192 candidates
    (1, 300, 33000, 2048, 32700),   # rows on both sides of 32768 candidates
    (1, 2600, 2600, 2048, 0),       # causal prefill from one candidate
    (1, 260, 32768, 700, 32508),    # up to exactly 32768 candidates, k = 700
])
def test_prefill_row_length_ranges(B, T, N, k, q_offset):
    """Rows of a prefill batch go to the selection for their candidate count
    (at most 8192, at most 32768, longer); each range and its edges."""
    s = torch.randn(B, T, N, generator=_gen(T + N)).abs()
    _check(s, k, q_offset, f"ranges B={B} T={T} N={N} k={k}")


@pytest.mark.parametrize("N", [5000, 9001])
def test_rows_with_exactly_k_numbers(N):
    """Rows whose candidates hold exactly k numbers and NaN elsewhere: the
    k-th largest key is the smallest number, its bin is kept whole, and no
    NaN may be picked."""
    g = _gen(21 + N)
    T, k = 16, 2048
    s = torch.full((1, T, N), float("nan"))
    for t in range(T):
        pos = torch.randperm(N - T + t + 1, generator=g)[:k]
        s[0, t, pos] = torch.randn(k, generator=g) if t % 2 == 0 else torch.ones(k)
    _check(s, k, N - T, f"exactly k numbers N={N}")


def test_negative_and_infinite_scores():
    g = _gen(7)
    s = torch.randn(1, 16, 4096, generator=g)
    s[0, :, ::17] = float("-inf")
    s[0, :, ::29] = float("inf")
    _check(s, 300, 4096 - 16, "signed")


def test_one_pass_rows_nan_inf_signed_zero_ties():
    """256 rows of 40000 candidates take the one-pass sampled-threshold path;
    its special values: NaN (ranks lowest), -inf, +-0 (equal), heavy exact
    ties, and rows whose sample is mostly or all NaN (threshold 0: every key
    passes, the wave regions overflow and the row falls back)."""
    g = _gen(13)
    T, N = 256, 40000
    s = torch.randn(1, T, N, generator=g)
    s[torch.rand(1, T, N, generator=g) < 0.02] = float("nan")
    s[torch.rand(1, T, N, generator=g) < 0.02] = float("-inf")
    s[torch.rand(1, T, N, generator=g) < 0.02] = 0.0
    s[torch.rand(1, T, N, generator=g) < 0.02] = -0.0
    s[0, 5][torch.rand(N, generator=g) < 0.95] = float("nan")   # mostly NaN
    s[0, 6] = float("nan")
    s[0, 6, ::400] = 1.0                                         # 100 numbers, rest NaN
    s[0, 7] = torch.randint(0, 4, (N,), generator=g).float() * 0.5  # four values
    s[0, 8] = float("-inf")
    s[0, 8, ::7] = torch.randn(len(range(0, N, 7)), generator=g)  # mostly -inf
    s[0, 9] = 0.0
    s[0, 9, ::2] = -0.0                                          # all zeros, both signs
    # NaN at every sampled position of a row that is otherwise finite (the
    # sample reads 16-key blocks starting at j * (n - 16) / 127)
    n10 = N - T + 10 + 1
    for j in range(128):
        st = (j * (n10 - 16)) // 127
        s[0, 10, st:st + 16] = float("nan")
    s[0, 11] = 2.0                                               # one value everywhere
    s[0, 11, 100:110] = float("nan")
    _check(s, 2048, N - T, "one-pass special values")
