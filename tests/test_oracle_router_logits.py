"""Pins for the oracle's BF16 routing logits (CPU only): exact integer
arithmetic, exact rational sums, power-of-two scaling and expert relabelling.
BF16 routing is one of the gfx950 operation families of the Netra Kernel
README capability table; the logits feed the (separately pinned) router."""
from fractions import Fraction

import numpy as np
import pytest
import torch


def _bf16_bits(a):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _bf16_val(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_integer_inputs_are_exact(oracle_mod):
    """Small-integer operands: every partial sum is an integer below 2^24, so
    the logits are the integer dot products exactly."""
    rng = np.random.default_rng(1)
    M, K, E = 6, 384, 20
    xi = rng.integers(-8, 9, (M, K))
    wi = rng.integers(-8, 9, (E, K))
    got = oracle_mod.router_logits(_bf16_bits(xi), _bf16_bits(wi))
    assert np.array_equal(got, (xi @ wi.T).astype(np.float32))


def test_matches_exact_rational_sum(oracle_mod):
    """Random bf16 operands: each logit is the exact rational dot product
    rounded once to fp32."""
    rng = np.random.default_rng(2)
    M, K, E = 2, 256, 6
    xb = _bf16_bits(rng.standard_normal((M, K)))
    wb = _bf16_bits(rng.standard_normal((E, K)) / 16)
    got = oracle_mod.router_logits(xb, wb)
    xv, wv = _bf16_val(xb), _bf16_val(wb)
    for t in range(M):
        for e in range(E):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xv[t], wv[e]))
            assert got[t, e] == np.float32(float(exact)), (t, e)


def test_scaling_and_relabelling(oracle_mod):
    rng = np.random.default_rng(3)
    M, K, E = 5, 512, 16
    xb = _bf16_bits(rng.standard_normal((M, K)))
    wb = _bf16_bits(rng.standard_normal((E, K)) / 20)
    base = oracle_mod.router_logits(xb, wb)
    x8 = _bf16_bits(_bf16_val(xb) * np.float32(8.0))
    assert np.array_equal(oracle_mod.router_logits(x8, wb), base * np.float32(8.0))
    perm = rng.permutation(E)
    assert np.array_equal(oracle_mod.router_logits(xb, wb[perm]), base[:, perm])
    # one-hot rows pick out one column of the weight
    oh = np.zeros((E, K), np.float32)
    cols = rng.integers(0, K, E)
    oh[np.arange(E), cols] = 1.0
    got = oracle_mod.router_logits(_bf16_bits(oh), wb)
    assert np.array_equal(got, _bf16_val(wb)[:, cols].T)


def test_router_weight_generator(synth_mod):
    cfg = synth_mod.CONFIGS[4]
    wb = synth_mod.make_wr(cfg, synth_mod.default_seed(4))
    assert wb.shape == (cfg.E, cfg.h) and wb.dtype == np.uint16
    v = _bf16_val(wb).astype(np.float64)
    assert abs(v.std() * np.sqrt(cfg.h) - 1.0) < 0.02
