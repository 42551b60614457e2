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


def check_output(got_bits: np.ndarray, ref_bits: np.ndarray, rel=REL_TOL, cos_min=COS_MIN):
    """Returns (max_abs_err, max_ref, min_cos); raises AssertionError on failure."""
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
        min_cos = min(min_cos, c)
    assert min_cos >= cos_min, f"cosine {min_cos} < {cos_min}"
    return float(err.max()), float(mx), min_cos


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
