"""Pins for the oracle's e4m3fn codec against torch's independent float8_e4m3fn
implementation and against format facts (max 448, min subnormal 2^-9, NaN codes)."""
import numpy as np
import torch

from oracle import e4m3_decode, e4m3_encode


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_decode_exhaustive_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = _torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_format_facts():
    d = e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert np.sum(np.isnan(d)) == 2
    assert np.nanmax(d) == 448.0 and np.nanmin(d) == -448.0
    assert d[0x01] == 2.0 ** -9 and d[0x08] == 2.0 ** -6 and d[0x38] == 1.0
    assert d[0x80] == 0.0 and np.signbit(d[0x80])
    # 254 finite values, 253 distinct numbers (+0 and -0 compare equal)
    assert np.sum(np.isfinite(d)) == 254 and np.unique(d[np.isfinite(d)]).size == 253


def test_encode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_encode_matches_torch_dense_sweep():
    rng = np.random.default_rng(7)
    pos = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[1:] + pos[:-1]) / 2  # exact ties
    vals = np.concatenate([
        pos, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
        rng.normal(0, 1, 20000), rng.normal(0, 100, 20000), rng.uniform(-448, 448, 20000),
        rng.uniform(-2 ** -6, 2 ** -6, 20000), [448.0, 447.99, 0.0, 2.0 ** -10, 3 * 2.0 ** -11],
    ])
    vals = np.concatenate([vals, -vals])
    # torch casts through float32, so compare on float32-representable inputs
    # (and step one float32 ulp around each tie as well)
    vals = np.concatenate([vals.astype(np.float32),
                           np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1000))])
    vals = np.concatenate([vals, -vals])
    ours = e4m3_encode(vals.astype(np.float64))
    ref = torch.from_numpy(np.clip(vals, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.flatnonzero(ours != ref)
    assert bad.size == 0, (vals[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_encode_clamps_and_nan():
    assert e4m3_encode(1e9) == 0x7E and e4m3_encode(-1e9) == 0xFE
    assert e4m3_encode(np.nan) == 0x7F
    assert e4m3_encode(2.0 ** -10) == 0x00  # tie between 0 and 2^-9 goes to even (0)
