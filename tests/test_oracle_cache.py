"""Pins for the oracle's per-token FP8 quantisation and cache append: format
facts (the largest element lands on +-448), exact power-of-two scale
invariance, zero rows, the half-step error bound of round-to-nearest, an
independent composition (torch float32 division + torch's e4m3fn cast), and
the bookkeeping of the append (positions, dropped rows, untouched rows)."""
import numpy as np
import torch

import oracle
from oracle import e4m3_decode, quantize_rows


def _rows(seed, n=64, d=128):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, (n, d)).astype(np.float32)
    x[1] *= 1e-3                                   # small magnitudes
    x[2] *= 300.0                                  # large magnitudes
    x[3, :] = 0.0
    x[3, 5] = -7.5                                 # one nonzero element
    x[4, ::3] = 0.0
    x[5] = rng.standard_t(2, d).astype(np.float32)  # heavy tails
    return x


def test_largest_element_maps_to_448():
    x = _rows(1)
    codes, scale = quantize_rows(x)
    for r in range(x.shape[0]):
        j = int(np.argmax(np.abs(x[r])))
        assert codes[r, j] == (0xFE if x[r, j] < 0 else 0x7E)
        amax = float(np.max(np.abs(x[r])))
        # float32 division correctly rounded: within half an ulp of amax / 448
        exact = amax / 448.0
        assert abs(float(scale[r]) - exact) <= np.spacing(np.float32(exact)) / 2


def test_power_of_two_scale_invariance():
    x = _rows(2)
    c0, s0 = quantize_rows(x)
    for e in (-20, -3, 1, 7, 30):
        c, s = quantize_rows(x * np.float32(2.0 ** e))
        assert np.array_equal(c, c0)
        assert np.array_equal(s, (s0 * np.float32(2.0 ** e)).astype(np.float32))


def test_zero_rows():
    c, s = quantize_rows(np.array([[0.0, -0.0, 0.0, -0.0]], np.float32))
    assert s[0] == 1.0
    assert c.tolist() == [[0x00, 0x80, 0x00, 0x80]]


def test_half_step_error_bound():
    x = _rows(3)
    c, s = quantize_rows(x)
    y = x.astype(np.float64) / s[:, None].astype(np.float64)
    deq = e4m3_decode(c)
    # grid step at |y|: 2^(floor(log2|y|) - 3) for normals, 2^-9 below 2^-6
    a = np.abs(y)
    step = np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3), 2.0 ** -9)
    slack = np.abs(y) * 2.0 ** -23                 # the float32 quotient's own rounding
    assert np.all(np.abs(deq - y) <= step / 2 + slack)


def test_matches_torch_composition():
    x = _rows(4, n=256)
    c, s = quantize_rows(x)
    xt = torch.from_numpy(x)
    amax = xt.abs().amax(dim=-1)
    st = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    ct = (xt / st[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(s, st.numpy())
    assert np.array_equal(c, ct)


def test_cache_append_bookkeeping():
    rng = np.random.default_rng(5)
    B, T, N, d, dq = 3, 2, 10, 8, 6
    k_new = rng.normal(0, 1, (B, T, d)).astype(np.float32)
    kv_new = rng.normal(0, 1, (B, T, dq)).astype(np.float32)
    kc = rng.integers(0, 255, (B, N, d), dtype=np.uint8)
    ks = rng.random((B, N)).astype(np.float32)
    kvc = rng.normal(0, 1, (B, N, dq)).astype(np.float32)
    pos = np.array([0, 9, -1])                     # b=1 keeps t=0 only; b=2 keeps t=1 only
    a, bsc, c = oracle.cache_append(k_new, kv_new, kc, ks, kvc, pos)
    written = {(0, 0, 0), (0, 1, 1), (1, 9, 0), (2, 0, 1)}
    for b in range(B):
        for p in range(N):
            hit = [t for (bb, pp, t) in written if bb == b and pp == p]
            if hit:
                codes, sc = quantize_rows(k_new[b, hit[0]])
                assert np.array_equal(a[b, p], codes) and bsc[b, p] == sc
                assert np.array_equal(c[b, p], kv_new[b, hit[0]])
            else:
                assert np.array_equal(a[b, p], kc[b, p]) and bsc[b, p] == ks[b, p]
                assert np.array_equal(c[b, p], kvc[b, p])
