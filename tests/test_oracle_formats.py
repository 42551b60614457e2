"""Pins for the oracle's number formats (CPU only).

The E4M3 decode table and encoder are checked against torch's independent
float8_e4m3fn implementation and against exhaustive search; the bf16 encoder
against torch's float32 -> bfloat16 conversion.  The OCP E4M3 facts used
(bias 7, largest finite 448, smallest normal 2^-6, smallest subnormal 2^-9,
NaN at 0x7F/0xFF, no infinities) are those of the OCP 8-bit floating point
specification, which the Netra pages name as the weight format ("E4M3 with
128x128 block scales", Netra Kernel README, supported-targets table).
"""
import math

import numpy as np
import pytest
import torch


def _torch_decode_all():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()


def test_e4m3_table_matches_torch_all_codes(oracle_mod):
    t = oracle_mod.e4m3_table()
    ref = _torch_decode_all()
    nan_t = np.isnan(t)
    assert np.array_equal(nan_t, np.isnan(ref))
    assert set(np.nonzero(nan_t)[0]) == {0x7F, 0xFF}
    assert np.array_equal(t[~nan_t], ref[~nan_t])
    # sign of zero
    assert math.copysign(1.0, t[0x80]) == -1.0 and math.copysign(1.0, t[0x00]) == 1.0


def test_e4m3_spot_values(oracle_mod):
    t = oracle_mod.e4m3_table()
    assert t[0x7E] == 448.0            # largest finite
    assert t[0x08] == 2.0 ** -6        # smallest normal
    assert t[0x01] == 2.0 ** -9        # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9    # largest subnormal
    assert t[0x38] == 1.0
    assert t[0xFE] == -448.0
    # positive finite codes strictly increasing
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)


def _all_midpoints(t):
    pos = t[:0x7F].astype(np.float64)
    mids = (pos[:-1] + pos[1:]) / 2.0
    return mids.astype(np.float32)  # all exactly representable in fp32


def _sweep_values(t, n_random=400_000, seed=0):
    rng = np.random.default_rng(seed)
    mids = _all_midpoints(t)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                           t[:0x7F], np.nextafter(t[:0x7F], np.float32(1e9))])
    logu = rng.uniform(-14, math.log2(448.0), n_random)
    rnd = (2.0 ** logu).astype(np.float32)
    tiny = rng.uniform(0, 2.0 ** -8, 20000).astype(np.float32)
    v = np.concatenate([near, rnd, tiny, np.float32([0.0, 448.0, 2.0 ** -10, 3 * 2.0 ** -10])])
    v = v[(v >= 0) & (v <= 448.0)]
    return np.concatenate([v, -v]).astype(np.float32)


def test_e4m3_encode_matches_torch_in_range(oracle_mod):
    """RNE in [-448, 448], including every midpoint and its fp32 neighbours."""
    t = oracle_mod.e4m3_table()
    v = _sweep_values(t)
    ours = oracle_mod.e4m3_encode_array(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(float(v[j]), int(ours[j]), int(ref[j])) for j in bad[:10]]


def test_e4m3_encode_bisection_equals_linear_search(oracle_mod):
    t = oracle_mod.e4m3_table()
    v = _sweep_values(t, n_random=3000, seed=1)
    v = np.concatenate([v, np.float32([500.0, -500.0, 464.0, 1e30, -1e30, np.inf, -np.inf])])
    for x in v:
        assert oracle_mod.e4m3_encode(float(x)) == oracle_mod.e4m3_encode_linear(float(x)), float(x)


def test_e4m3_encode_saturation_and_specials(oracle_mod):
    enc = oracle_mod.e4m3_encode
    for big in (448.0, 449.0, 463.99, 464.0, 480.0, 1e6, float("inf")):
        assert enc(big) == 0x7E and enc(-big) == 0xFE
    assert enc(float("nan")) == 0x7F
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    # below half the smallest subnormal -> zero with sign; exactly half -> tie to even (zero)
    assert enc(2.0 ** -11) == 0x00 and enc(-(2.0 ** -11)) == 0x80
    assert enc(2.0 ** -10) == 0x00
    assert enc(np.nextafter(np.float32(2.0 ** -10), np.float32(1)).item()) == 0x01
    assert enc(3 * 2.0 ** -10) == 0x02   # tie between codes 1 and 2 -> even


def test_e4m3_roundtrip_and_monotone(oracle_mod):
    t = oracle_mod.e4m3_table()
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle_mod.e4m3_encode(float(t[c])) == c
    xs = np.linspace(-460, 460, 20001, dtype=np.float32)
    codes = oracle_mod.e4m3_encode_array(xs)
    vals = t[codes]
    assert np.all(np.diff(vals) >= 0)


def test_bf16_encode_matches_torch(oracle_mod):
    rng = np.random.default_rng(2)
    v = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    # exact ties: fp32 values halfway between two bf16 values
    base = rng.standard_normal(2000).astype(np.float32)
    bits = base.view(np.uint32) & np.uint32(0xFFFF0000)
    ties = (bits | np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, ties, np.float32([0.0, -0.0, 1.0, 65504.0, 3.4e38, -3.4e38, 1e-40])])
    ours = oracle_mod.bf16_encode_array(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
