"""Pins for the oracle's RMSNorm + 1x128 quantisation front end (CPU only).

The front end is the normalisation-and-quantisation fusion that the Netra
Kernel README's directory map lists for gfx950, read as a standard RMSNorm
with an fp32 weight, rounded to bf16, followed by the layer's own activation
quantisation.  It is checked against closed forms, a float64 evaluation with
a rounding bound, invariants that hold exactly, and the oracle's separately
pinned activation quantiser.
"""
import numpy as np
import pytest
import torch


def _bf16_bits(a):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _bf16_val(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("j", [-20, -3, 0, 5, 30])
def test_constant_power_of_two_rows(oracle_mod, j):
    """A row of +-2^j with eps = 0 normalises to exactly +-1 (times gamma), so
    every group quantises to +-448 with scale fp32(1/448)."""
    K = 384
    x = np.full((2, K), 2.0 ** j, np.float32)
    x[1] = -x[1]
    x[1, 128:256] = 2.0 ** j              # mixed signs keep |x| constant
    y, q, s = oracle_mod.rmsnorm_act_quant(_bf16_bits(x), np.ones(K, np.float32), 0.0)
    assert np.array_equal(_bf16_val(y), np.sign(x))
    assert np.all(q[x > 0] == 0x7E) and np.all(q[x < 0] == 0xFE)
    assert np.all(s == np.float32(1.0) / np.float32(448.0))
    g = np.full(K, 0.25, np.float32)
    y2, q2, s2 = oracle_mod.rmsnorm_act_quant(_bf16_bits(x), g, 0.0)
    assert np.array_equal(_bf16_val(y2), 0.25 * np.sign(x))
    assert np.array_equal(q2, q)
    assert np.all(s2 == np.float32(0.25) / np.float32(448.0))


@pytest.mark.parametrize("eps,scale", [(1e-6, 1.0), (0.25, 0.3), (1e-5, 1e-3), (0.0, 40.0)])
def test_matches_float64_definition(oracle_mod, eps, scale):
    """y within the bf16 rounding (unit roundoff 2^-8) plus a few fp32 roundings of
    x / sqrt(mean(x^2) + eps) * gamma evaluated in float64.  eps = 0.25 on
    small rows makes eps dominate, which separates eps inside the root and
    added to the mean from the other placements."""
    rng = np.random.default_rng(11)
    M, K = 9, 640
    x = rng.standard_normal((M, K)) * scale * rng.uniform(0.2, 5.0, (M, 1))
    x[3, ::7] = 0.0
    xb = _bf16_bits(x)
    x64 = _bf16_val(xb).astype(np.float64)
    g = rng.uniform(0.5, 1.5, K).astype(np.float32)
    y, q, s = oracle_mod.rmsnorm_act_quant(xb, g, eps)
    ref = x64 / np.sqrt((x64 * x64).mean(axis=1, keepdims=True) + np.float64(np.float32(eps))) \
        * g.astype(np.float64)
    got = _bf16_val(y).astype(np.float64)
    bound = np.abs(ref) * (2.0 ** -8 + 4 * 2.0 ** -24) * (1 + 2.0 ** -20)   # bf16 unit roundoff 2^-8
    assert np.all(np.abs(got - ref) <= bound)


def test_power_of_two_scaling_invariance(oracle_mod):
    """With eps = 0, scaling a row by 2^j changes no rounding anywhere."""
    rng = np.random.default_rng(12)
    K = 512
    xb = _bf16_bits(rng.standard_normal((5, K)))
    g = rng.uniform(-2, 2, K).astype(np.float32)
    base = oracle_mod.rmsnorm_act_quant(xb, g, 0.0)
    for j in (-9, 4, 17):
        xj = _bf16_bits(_bf16_val(xb) * np.float32(2.0 ** j))
        out = oracle_mod.rmsnorm_act_quant(xj, g, 0.0)
        for a, b in zip(base, out):
            assert np.array_equal(a, b)


def test_zero_rows_and_signed_zeros(oracle_mod):
    K = 256
    x = np.zeros((3, K), np.float32)
    x[1] = -0.0
    x[2, 0] = 1.0
    x[2, 5] = -0.0
    y, q, s = oracle_mod.rmsnorm_act_quant(_bf16_bits(x), np.ones(K, np.float32), 1e-6)
    assert np.all(y[0] == 0) and np.all(y[1] == 0x8000)
    assert not q[:2].any() and not s[:2].any()
    assert y[2, 5] == 0x8000 and s[2, 1] == 0.0 and not q[2, 128:].any()


def test_quantisation_is_the_activation_quantiser(oracle_mod):
    """The codes and scales are those of the (separately pinned) 1x128
    activation quantiser applied to the bf16 output."""
    rng = np.random.default_rng(13)
    K = 1024
    xb = _bf16_bits(rng.standard_normal((7, K)) * 3.0)
    g = rng.uniform(0.1, 3.0, K).astype(np.float32)
    y, q, s = oracle_mod.rmsnorm_act_quant(xb, g, 1e-6)
    q2, s2 = oracle_mod.act_quant(y)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_thread_count_invariance(oracle_mod):
    rng = np.random.default_rng(14)
    K = 2048
    xb = _bf16_bits(rng.standard_normal((33, K)))
    g = rng.uniform(0.5, 1.5, K).astype(np.float32)
    n0 = oracle_mod.get_threads()
    try:
        oracle_mod.set_threads(1)
        a = oracle_mod.rmsnorm_act_quant(xb, g, 1e-6)
        oracle_mod.set_threads(max(2, n0))
        b = oracle_mod.rmsnorm_act_quant(xb, g, 1e-6)
    finally:
        oracle_mod.set_threads(n0)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
