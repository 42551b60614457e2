"""Pins for the oracle's MXFP4 weight variant (CPU only).

MXFP4 is named on the pages as a checkpoint format (Netra Kernel README,
targets table) and as the MoE kernel moe/mxfp4_h6144_i768_e128_top4 (Inferact
amd-kernels README, naming section); the README checks its kernels against
float64 dequantised-MXFP4 references.  Pinned here against closed forms, a
brute-force nearest search, the OCP MX block rule, float64 matrix products of
the dequantised operands and a float64 brute-force layer."""
import math

import numpy as np
import pytest
import torch

from test_oracle_layer import _T64, _quant_rows_fp32, check_close


def _e2m1_closed_form(c):
    s, e, m = c >> 3, (c >> 1) & 3, c & 1
    mag = m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -mag if s else mag


def _brute_encode(v):
    """Nearest of the 8 magnitudes, ties to the even mantissa bit, sign kept."""
    mags = [_e2m1_closed_form(c) for c in range(8)]
    a = abs(v)
    best = 7 if a >= 6.0 else min(range(8), key=lambda c: (abs(a - mags[c]), c & 1))
    return best | (8 if math.copysign(1.0, v) < 0 else 0)


def test_e2m1_table_is_the_closed_form(oracle_mod):
    for c in range(16):
        got, ref = oracle_mod.e2m1_decode(c), _e2m1_closed_form(c)
        assert got == ref and math.copysign(1.0, got) == math.copysign(1.0, ref if c != 8 else -0.0)
    assert [oracle_mod.e2m1_decode(c) for c in range(8)] == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_encoder_against_brute_force(oracle_mod):
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = []
    for m in mids:
        f = np.float32(m)
        vals += [float(f), float(np.nextafter(f, np.float32(0))), float(np.nextafter(f, np.float32(10)))]
    rng = np.random.default_rng(4)
    vals += list(rng.uniform(-8, 8, 3000).astype(np.float32).astype(float))
    vals += [0.0, -0.0, 6.0, 6.5, 7.0, 1e30, -1e30, 1e-40, -1e-40]
    for v in vals + [-x for x in vals]:
        assert oracle_mod.e2m1_encode(v) == _brute_encode(v), v
    # ties go to the even code; saturation; round trip; monotone
    assert [oracle_mod.e2m1_encode(m) for m in mids] == [0, 2, 2, 4, 4, 6, 6]
    assert oracle_mod.e2m1_encode(1e9) == 7 and oracle_mod.e2m1_encode(-1e9) == 15
    for c in range(16):
        assert oracle_mod.e2m1_encode(oracle_mod.e2m1_decode(c)) == c
    xs = np.linspace(-9, 9, 5001)
    dec = [oracle_mod.e2m1_decode(oracle_mod.e2m1_encode(x)) for x in xs]
    assert all(a <= b for a, b in zip(dec, dec[1:]))


def test_e8m0_decode(oracle_mod):
    assert oracle_mod.e8m0_decode(127) == 1.0
    assert oracle_mod.e8m0_decode(128) == 2.0 and oracle_mod.e8m0_decode(126) == 0.5
    assert oracle_mod.e8m0_decode(0) == 2.0 ** -127 and oracle_mod.e8m0_decode(254) == 2.0 ** 127
    assert math.isnan(oracle_mod.e8m0_decode(255))


def test_mxfp4_quantiser_follows_the_block_rule(oracle_mod):
    rng = np.random.default_rng(7)
    rows, K = 40, 256
    w = (rng.standard_normal((rows, K)) * np.exp(rng.uniform(-20, 20, (rows, K // 32))).repeat(32, 1))
    w = w.astype(np.float32)
    w[3, 32:64] = 0.0                                     # an all-zero block
    codes, scales = oracle_mod.mxfp4_quantize(w)
    assert codes.shape == (rows, K // 2) and scales.shape == (rows, K // 32)
    for r in range(rows):
        for b in range(K // 32):
            blk = w[r, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            byte = codes[r, 16 * b:16 * b + 16]
            nib = np.stack([byte & 15, byte >> 4], -1).ravel()
            if amax == 0:
                assert scales[r, b] == 0 and np.all(nib == 0)
                continue
            e = int(np.floor(np.log2(amax))) - 2
            assert scales[r, b] == e + 127
            assert 4.0 <= amax / 2.0 ** e < 8.0
            for j in range(32):
                assert nib[j] == _brute_encode(float(np.float32(blk[j] / 2.0 ** e)))
    deq = oracle_mod.mxfp4_dequantize(codes, scales)
    step = np.where(np.abs(deq) < 2 * 2.0 ** (scales.astype(np.int64) - 127).repeat(32, 1), 0.25, 1.0)
    err = np.abs(deq - w) / 2.0 ** (scales.astype(np.int64) - 127).repeat(32, 1)
    assert np.all(err <= np.maximum(step, 2.0) + 1e-12)     # half-step, or the saturation band (6, 8)
    assert np.all(err[np.abs(w) / 2.0 ** (scales.astype(np.int64) - 127).repeat(32, 1) <= 6] <= 1.0)


def test_mxfp4_quantiser_round_trip_and_power_of_two_scaling(oracle_mod):
    rng = np.random.default_rng(8)
    rows, K = 16, 128
    vals = np.array([_e2m1_closed_form(c) for c in range(16)])
    nib = rng.integers(0, 16, (rows, K))
    nib[:, ::32] = rng.choice([6, 7, 14, 15], (rows, K // 32))  # a magnitude of 4 or 6 in each block
    sc = rng.integers(100, 150, (rows, K // 32))
    w = (vals[nib] * 2.0 ** (sc - 127 - 0).repeat(32, 1)).astype(np.float32)
    codes, scales = oracle_mod.mxfp4_quantize(w)
    assert np.array_equal(scales, sc.astype(np.uint8))
    assert np.array_equal(oracle_mod.mxfp4_dequantize(codes, scales), w.astype(np.float64))
    # element 2j in the low nibble of byte j
    assert np.array_equal(codes & 15, nib[:, 0::2]) and np.array_equal(codes >> 4, nib[:, 1::2])
    for j in (-5, 3, 11):
        c2, s2 = oracle_mod.mxfp4_quantize((w * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(c2, codes) and np.array_equal(s2.astype(int), scales.astype(int) + j)


def _mx_layer(synth_mod, oracle_mod, M, h, i, E, k, seed):
    cfg = synth_mod.LayerConfig("mx", M, h, i, E, k, "normal", "test shape")
    x = synth_mod.make_x(cfg, seed)
    logits = synth_mod.make_logits(cfg, seed)
    q13, e13 = oracle_mod.mxfp4_quantize(synth_mod.make_w13_f32(cfg, seed))
    q2, e2 = oracle_mod.mxfp4_quantize(synth_mod.make_w2_f32(cfg, seed))
    return x, logits, q13, e13, q2, e2


def test_mxfp4_gemms_are_float64_products_of_dequantised_operands(oracle_mod, synth_mod):
    """Each gate/up value and down partial is the float64 dot product of the
    dequantised weight row and the dequantised activation row, rounded once."""
    M, h, i, E, k = 3, 256, 128, 4, 2
    x, logits, q13, e13, q2, e2 = _mx_layer(synth_mod, oracle_mod, M, h, i, E, k, 3)
    out, inter = oracle_mod.moe_forward_mxfp4(x, logits, q13, e13, q2, e2, k, intermediates=True)
    T = _T64()
    W13 = oracle_mod.mxfp4_dequantize(q13, e13)
    W2 = oracle_mod.mxfp4_dequantize(q2, e2)
    for p in range(M * k):
        t, e = divmod(p, k)[0], inter["ids"].ravel()[p]
        a = T[inter["xq"][t]] * np.repeat(inter["xs"][t].astype(np.float64), 128)
        ref = W13[e] @ a
        assert np.all(np.abs(inter["g"][p] - ref) <= 2.0 ** -24 * np.abs(ref) + 1e-30)
        a2 = T[inter["a2"][p]] * np.repeat(inter["a2s"][p].astype(np.float64), 128)
        ref2 = W2[e] @ a2
        assert np.all(np.abs(inter["y"][p] - ref2) <= 2.0 ** -24 * np.abs(ref2) + 1e-30)


def _brute_mx(oracle_mod, xb, logits, q13, e13, q2, e2, k):
    """float64 brute force with dequantised MXFP4 weights; torch does the
    activation E4M3 roundings (decisions in fp32)."""
    T = _T64()
    M, h = xb.shape
    i = q2.shape[2] * 2
    W13 = oracle_mod.mxfp4_dequantize(q13, e13)
    W2 = oracle_mod.mxfp4_dequantize(q2, e2)
    x32 = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).float().numpy()
    l64 = logits.astype(np.float64)
    ids = np.argsort(-l64, axis=1, kind="stable")[:, :k]
    p = np.exp(l64 - l64.max(1, keepdims=True))
    w = np.take_along_axis(p, ids, 1)
    w /= w.sum(1, keepdims=True)
    xq, xs = _quant_rows_fp32(x32)
    xdq = T[xq] * np.repeat(xs.astype(np.float64), 128, axis=1)
    out = np.zeros((M, h))
    for t in range(M):
        for r in range(k):
            e = ids[t, r]
            gv = W13[e] @ xdq[t]
            v = gv[:i] / (1.0 + np.exp(-gv[:i])) * gv[i:]
            a2, a2s = _quant_rows_fp32(v.astype(np.float32)[None, :])
            out[t] += w[t, r] * (W2[e] @ (T[a2[0]] * np.repeat(a2s[0].astype(np.float64), 128)))
    return out


@pytest.mark.parametrize("shape", [(4, 256, 128, 8, 2), (2, 384, 256, 4, 3)])
def test_mxfp4_layer_vs_float64_bruteforce(oracle_mod, synth_mod, shape):
    M, h, i, E, k = shape
    x, logits, q13, e13, q2, e2 = _mx_layer(synth_mod, oracle_mod, M, h, i, E, k, 11)
    out = oracle_mod.moe_forward_mxfp4(x, logits, q13, e13, q2, e2, k)
    ref = _brute_mx(oracle_mod, x, logits, q13, e13, q2, e2, k)
    check_close(out, ref, rel=1e-3, cos_min=0.99999)


def test_mxfp4_layer_invariants(oracle_mod, synth_mod):
    M, h, i, E, k = 7, 256, 128, 8, 2
    x, logits, q13, e13, q2, e2 = _mx_layer(synth_mod, oracle_mod, M, h, i, E, k, 13)
    out = oracle_mod.moe_forward_mxfp4(x, logits, q13, e13, q2, e2, k)
    assert np.all(oracle_mod.moe_forward_mxfp4(np.zeros_like(x), logits, q13, e13, q2, e2, k) == 0)
    perm = np.random.default_rng(2).permutation(M)
    assert np.array_equal(oracle_mod.moe_forward_mxfp4(x[perm], logits[perm], q13, e13, q2, e2, k), out[perm])
