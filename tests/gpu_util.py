"""Shared helpers of the GPU parity tests: seeded inputs (weights quantised by
the oracle, so no oracle input ever comes from the GPU), upload, and the
output acceptance check.

Acceptance bar of the layer output (the oracle's bf16 output o, over the rows
compared):
  |gpu - o| <= 1e-2 * max|o| + ulp_bf16(o)  elementwise,
  cosine(gpu_row, o_row) >= 0.9999 per token (float64; two all-zero rows pass),
and exact zeros when max|o| == 0.
"""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
import synth

REL_TOL = 1e-2
COS_MIN = 0.9999


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return oracle.bf16_to_f32(bits).astype(np.float64)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -126)))
    return 2.0 ** (np.maximum(e, -126) - 7)


# Accuracy of a GPU gate/up value.  The method fixes an fp32 accumulation per
# 128-wide K block with the block scales applied per block, but not the order
# of the sum inside a block; the matrix cores add a block's 128 exact products
# in their own order and precision.  Any fp32 summation of n terms, in any
# order, lies within gamma_{n-1} * sum|terms| of the exact sum (Higham,
# Accuracy and Stability of Numerical Algorithms, recursive summation bound),
# gamma_n = n u / (1 - n u), u = 2^-24; the promotion acc += blk * (s_act * s_w)
# over KB blocks adds the rounding of the scale product, of the scaled block
# and of the running sum.  mfma_rel(KB) is that bound relative to
# sum|x_k w_nk| * |scales|; test_mfma_block_sum_accuracy checks that the
# hardware stays inside it.
def gamma(n: int) -> float:
    u = 2.0 ** -24
    return n * u / (1.0 - n * u)


def mfma_rel(KB: int) -> float:
    return gamma(127) + gamma(KB + 3)


def _T64():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _e4m3_codes(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(np.clip(v, -448.0, 448.0), dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def gate_up_terms(layer, inter) -> np.ndarray:
    """sum over k of |x_k * w_nk| * |scales| for every gate/up value [R, 2i]
    (float64, from the same codes the kernels read).  Routes are taken expert
    by expert, one matrix product per K block."""
    T = _T64()
    ids, xq, xs = inter["ids"], inter["xq"], inter["xs"].astype(np.float64)
    M, k = ids.shape
    I2, h = layer.q13.shape[1], layer.q13.shape[2]
    KB = h // 128
    flat = ids.ravel()
    mag = np.zeros((M * k, I2))
    for e in np.unique(flat):
        P = np.nonzero(flat == e)[0]
        t = P // k
        W = np.abs(T[layer.q13[e]]).reshape(I2, KB, 128)
        srow = np.repeat(np.abs(layer.s13[e].astype(np.float64)), 128, axis=0)   # [I2, KB]
        acc = np.zeros((P.size, I2))
        for kb in range(KB):
            a = np.abs(T[xq[t, kb * 128:(kb + 1) * 128]])                        # [nP, 128]
            acc += (a @ W[:, kb, :].T) * srow[None, :, kb] * xs[t, kb][:, None]
        mag[P] = acc
    return mag


def flagged_codes(layer, inter, rel=None, terms=None):
    """(lo, hi, s) for every requantised value [R, i]: the E4M3 codes at the two
    ends of the interval the quotient v / s can reach when each gate/up value
    is off by at most rel * sum|terms| (propagated through SiLU(gate) * up and
    through the group's scale amax / 448).  lo == hi where the decision is
    clear of every rounding boundary; elsewhere either code is a correct
    result of the method."""
    g = inter["g"].astype(np.float64)
    i = g.shape[1] // 2
    if rel is None:
        rel = mfma_rel(inter["xs"].shape[1])
    dg = rel * (gate_up_terms(layer, inter) if terms is None else terms)
    a, u = g[:, :i], g[:, i:]
    da, du = dg[:, :i], dg[:, i:]
    sig = 1.0 / (1.0 + np.exp(-a))
    silu = a * sig
    dsilu = sig * (1.0 + a * (1.0 - sig))
    v = silu * u
    dv = 1.1 * (np.abs(dsilu) * da * (np.abs(u) + du) + np.abs(silu) * du)
    s = np.repeat(inter["a2s"].astype(np.float64), 128, axis=1)
    R = g.shape[0]
    ds = np.repeat(dv.reshape(R, i // 128, 128).max(-1), 128, axis=1) / 448.0
    with np.errstate(divide="ignore", invalid="ignore"):
        pos = s > 0
        q = np.where(pos, v / np.where(pos, s, 1.0), 0.0)
        dq = np.where(pos, dv / np.where(pos, s, 1.0) + np.abs(q) * ds / np.where(pos, s, 1.0), 0.0)
    return _e4m3_codes(q - dq), _e4m3_codes(q + dq), s


def flip_allowance(layer, inter, terms=None, w2_dense=None) -> np.ndarray:
    """Largest change of the output [M, h] that the flagged requantisation
    decisions can cause: the gap between the two codes times the scale, times
    |w2 column|, times the routing weight (routes taken expert by expert).
    `terms` and `w2_dense(e)` (float64 [h, i]) replace the FP8 layer's own for
    another weight format."""
    T = _T64()
    lo, hi, s = flagged_codes(layer, inter, terms=terms)
    step = np.abs(T[hi] - T[lo]) * s                # [R, i], 0 where clear
    ids, tw = inter["ids"], inter["topk_w"]
    M, k = ids.shape
    h = layer.q2.shape[1]
    allow = np.zeros((M, h))
    flat = ids.ravel()
    live = np.nonzero(step.any(axis=1))[0]
    for e in np.unique(flat[live]):
        P = live[flat[live] == e]
        if w2_dense is not None:
            W2 = w2_dense(e)
        else:
            W2 = T[layer.q2[e]] * np.repeat(np.repeat(layer.s2[e].astype(np.float64), 128, 0), 128, 1)
        contrib = (step[P] @ np.abs(W2).T) * np.abs(tw.ravel()[P])[:, None]   # [nP, h]
        np.add.at(allow, P // k, contrib)
    return allow


def check_output(got_bits: np.ndarray, ref_bits: np.ndarray, rel=REL_TOL, cos_min=COS_MIN,
                 allowance=None):
    """Returns (max_abs_err, max_ref, min_cos); raises AssertionError on failure.
    `allowance` (same shape) widens the elementwise bar by the effect of
    flagged E4M3 code flips (see flip_allowance)."""
    got = bf16_bits_to_f64(got_bits)
    ref = bf16_bits_to_f64(ref_bits)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    mx = np.abs(ref).max() if ref.size else 0.0
    if mx == 0.0:
        assert np.all(got == 0.0), "oracle output is all zero, GPU output is not"
        return 0.0, 0.0, 1.0
    err = np.abs(got - ref)
    tol = rel * mx + bf16_ulp(ref)
    if allowance is not None:
        tol = tol + allowance * (1 + 1e-6)
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{int(bad.sum())} elements outside tolerance; first {idx.tolist()}, "
                             f"got {got[bad][:5]}, ref {ref[bad][:5]}, max|ref| {mx}")
    min_cos = 1.0
    for t in range(ref.shape[0]):
        a, b = got[t], ref[t]
        na, nb = np.linalg.norm(a), np.linalg.norm(b)
        if na == 0.0 and nb == 0.0:
            continue
        c = float(a @ b / (na * nb)) if na > 0 and nb > 0 else 0.0
        bar = cos_min
        if allowance is not None and nb > 0:
            # a deviation d with ||d|| <= ||allowance_t|| lowers the cosine by
            # at most about ||d||^2 / (2 ||b||^2); allow twice that
            ratio = np.linalg.norm(allowance[t]) / nb
            bar = min(cos_min, 1.0 - ratio * ratio)
        assert c >= bar, f"token {t}: cosine {c} < {bar}"
        min_cos = min(min_cos, c)
    return float(err.max()), float(mx), min_cos


def r16_report(label, got_bits, ref_bits, allowance=None):
    """Logs how the output compares with the unwidened bar (1e-2 * max|o| +
    1 bf16 ulp elementwise, cosine >= 0.9999 per token): whether it holds,
    the largest error as a multiple of that bar and, for a widened check, the
    largest flip allowance as a multiple of it.  Returns the strict verdict."""
    got = bf16_bits_to_f64(got_bits)
    ref = bf16_bits_to_f64(ref_bits)
    mx = np.abs(ref).max() if ref.size else 0.0
    if mx == 0.0:
        strict = bool(np.all(got == 0.0))
        log(f"R16 {label}: strict={'yes' if strict else 'no'} (all-zero oracle output)")
        return strict
    bar = REL_TOL * mx + bf16_ulp(ref)
    err_ratio = float((np.abs(got - ref) / bar).max())
    cos = 1.0
    for t in range(ref.shape[0]):
        a, b = got[t], ref[t]
        na, nb = np.linalg.norm(a), np.linalg.norm(b)
        if na == 0.0 and nb == 0.0:
            continue
        cos = min(cos, float(a @ b / (na * nb)) if na > 0 and nb > 0 else 0.0)
    strict = err_ratio <= 1.0 and cos >= COS_MIN
    allow_ratio = float((allowance / bar).max()) if allowance is not None else 0.0
    log(f"R16 {label}: strict={'yes' if strict else 'no'} max_err/bar={err_ratio:.3g} "
        f"max_allowance/bar={allow_ratio:.3g} min_cos={cos:.7f}")
    return strict


def to_dev_bf16(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def to_dev_fp8(codes: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(dev)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@functools.lru_cache(maxsize=2)
def quantised_weights(cfg: synth.LayerConfig, seed: int):
    """Oracle-quantised expert weights (host numpy): q13, s13, q2, s2."""
    q13, s13 = oracle.quant_weight_block128(synth.make_w13_f32(cfg, seed))
    q2, s2 = oracle.quant_weight_block128(synth.make_w2_f32(cfg, seed))
    return q13, s13, q2, s2


class Layer:
    """Host and device copies of one layer's inputs."""

    def __init__(self, cfg: synth.LayerConfig, seed: int, dev, x=None, logits=None, weights=None):
        self.cfg = cfg
        self.seed = seed
        self.dev = dev
        self.x = synth.make_x(cfg, seed) if x is None else x
        self.logits = synth.make_logits(cfg, seed) if logits is None else logits
        self.q13, self.s13, self.q2, self.s2 = quantised_weights(cfg, seed) if weights is None else weights
        self.tx = to_dev_bf16(self.x, dev)
        self.tl = torch.from_numpy(np.ascontiguousarray(self.logits)).to(dev)
        self.t13 = to_dev_fp8(self.q13, dev)
        self.ts13 = torch.from_numpy(self.s13).to(dev)
        self.t2 = to_dev_fp8(self.q2, dev)
        self.ts2 = torch.from_numpy(self.s2).to(dev)

    @property
    def dims(self):
        c = self.cfg
        return c.M, c.h, c.i, c.E, c.k

    def oracle(self, tokens=None, intermediates=False):
        x, l = self.x, self.logits
        if tokens is not None:
            x, l = x[tokens], l[tokens]
        return oracle.moe_forward(x, l, self.q13, self.s13, self.q2, self.s2, self.cfg.k,
                                  intermediates=intermediates)


def read_ws(ws: torch.Tensor, off: int, count: int, dtype) -> np.ndarray:
    nbytes = count * np.dtype(dtype).itemsize
    return ws[off:off + nbytes].cpu().numpy().view(dtype).copy()
