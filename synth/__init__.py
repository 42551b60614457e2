"""Seeded synthetic inputs for the routed FP8 block-scaled MoE layer.

Holds no arithmetic of the method itself: a counter-based normal generator
(``synth.c``, SplitMix64 + Box-Muller), the five layer shapes, and how their
inputs are drawn.  Activations come out as bf16 bit patterns (the
float32 -> bfloat16 conversion is torch's), router logits as float32 and
weights as float32; quantising the weights to E4M3 is left to the caller (the
oracle in tests, the library's own block quantiser on the GPU).

Input recipe for each shape:
  x        bf16 of N(0, 1)                                     [M, h]
  logits   fp32 N(0, 1)                                        [M, E]
           shared_bias: + b[e], b ~ N(0, sd=2) drawn once per batch
           request_bias: + b[q, e] for the request q = t // request_tokens of
                        token t, one b[q] ~ N(0, sd=2) per request
           zipf:        + ln p_e, p_e = (e+1)^-1.1 / sum_j (j+1)^-1.1
  w13      fp32 N(0, sd=1/sqrt(h)) [E, 2i, h]; rows [0,i) gate, [i,2i) up
  w2       fp32 N(0, sd=1/sqrt(i)) [E, h, i]
  wr       bf16 N(0, sd=1/sqrt(h)) [E, h], the router weight of BF16 routing (tag 6)
Each tensor is its own stream (seed, tag); rotation copy c adds 256*c to the
tag, so copies are independent draws.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

TAG_X, TAG_LOGITS, TAG_BIAS, TAG_W13, TAG_W2, TAG_WR = 1, 2, 3, 4, 5, 6
COPY_TAG_STRIDE = 256


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run synth/build.py")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, ct in (("synth_normal_f32", ctypes.c_void_p), ("synth_normal_f64", ctypes.c_void_p)):
            fn = getattr(lib, name)
            fn.restype = None
            fn.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                           ctypes.c_double, ctypes.c_double, ct]
        _lib = lib
    return _lib


def normal(seed: int, tag: int, shape, std: float = 1.0, mean: float = 0.0,
           first: int = 0, dtype=np.float32) -> np.ndarray:
    """Samples first .. first+size-1 of stream (seed, tag) as mean + std*N(0,1)."""
    lib = _load()
    out = np.empty(shape, dtype=dtype)
    fn = lib.synth_normal_f32 if out.dtype == np.float32 else lib.synth_normal_f64
    if out.dtype not in (np.float32, np.float64):
        raise TypeError("dtype must be float32 or float64")
    fn(seed, tag, first, out.size, float(mean), float(std), out.ctypes.data)
    return out


@dataclass(frozen=True)
class LayerConfig:
    name: str
    M: int
    h: int
    i: int
    E: int
    k: int
    logits: str          # "normal" | "shared_bias" | "request_bias" | "zipf"
    description: str
    request_tokens: int = 0   # tokens per request ("request_bias" only)

    @property
    def routes(self) -> int:
        return self.M * self.k


CONFIGS = [
    LayerConfig("tiny_m4_h256_i128_e8_top2", 4, 256, 128, 8, 2, "normal",
                "tiny layer, M=4, logits N(0,1)"),
    LayerConfig("decode_m1_h2048_i768_e128_top8", 1, 2048, 768, 128, 8, "normal",
                "decode, one token, weight-streaming bound"),
    LayerConfig("verify_m12_h2048_i768_e128_top8", 12, 2048, 768, 128, 8, "shared_bias",
                "speculative-verify batch, shared expert bias N(0, sd=2)"),
    LayerConfig("decode_m64_h6144_i768_e128_top4", 64, 6144, 768, 128, 4, "normal",
                "wide-hidden decode batch"),
    LayerConfig("prefill_m8192_h2048_i768_e128_top8", 8192, 2048, 768, 128, 8, "zipf",
                "prefill with a Zipf(1.1) expert-popularity prior"),
    LayerConfig("verify_m768_h2048_i768_e128_top8", 768, 2048, 768, 128, 8, "request_bias",
                "verify batch of 64 requests x 12 tokens, an expert bias N(0, sd=2) per request",
                request_tokens=12),
]


def default_seed(cfg_index: int) -> int:
    return 20261202 + cfg_index


def zipf_log_prior(E: int, s: float = 1.1) -> np.ndarray:
    """ln p_e for p_e proportional to (e+1)^-s, float64."""
    ranks = np.arange(1, E + 1, dtype=np.float64)
    lw = -s * np.log(ranks)
    return lw - np.log(np.exp(lw).sum())


def make_x_f32(cfg: LayerConfig, seed: int, copy: int = 0, M: int | None = None,
               first_token: int = 0) -> np.ndarray:
    M = cfg.M if M is None else M
    return normal(seed, TAG_X + COPY_TAG_STRIDE * copy, (M, cfg.h), first=first_token * cfg.h)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def make_x(cfg: LayerConfig, seed: int, copy: int = 0, M: int | None = None,
           first_token: int = 0) -> np.ndarray:
    """bf16 bit patterns [M, h]."""
    return to_bf16_bits(make_x_f32(cfg, seed, copy, M, first_token))


def make_logits(cfg: LayerConfig, seed: int, copy: int = 0, M: int | None = None,
                first_token: int = 0) -> np.ndarray:
    """fp32 [M, E]."""
    M = cfg.M if M is None else M
    tag = TAG_LOGITS + COPY_TAG_STRIDE * copy
    if cfg.logits == "normal":
        return normal(seed, tag, (M, cfg.E), first=first_token * cfg.E)
    base = normal(seed, tag, (M, cfg.E), first=first_token * cfg.E, dtype=np.float64)
    if cfg.logits == "shared_bias":
        bias = normal(seed, TAG_BIAS + COPY_TAG_STRIDE * copy, (cfg.E,), std=2.0, dtype=np.float64)
        return (base + bias[None, :]).astype(np.float32)
    if cfg.logits == "request_bias":
        q = cfg.request_tokens
        req = np.arange(first_token, first_token + M) // q
        r0 = int(req[0]) if M else 0
        nreq = int(req[-1]) - r0 + 1 if M else 0
        bias = normal(seed, TAG_BIAS + COPY_TAG_STRIDE * copy, (nreq, cfg.E), std=2.0,
                      first=r0 * cfg.E, dtype=np.float64)
        return (base + bias[req - r0]).astype(np.float32)
    if cfg.logits == "zipf":
        return (base + zipf_log_prior(cfg.E)[None, :]).astype(np.float32)
    raise ValueError(cfg.logits)


def make_wr(cfg: LayerConfig, seed: int) -> np.ndarray:
    """bf16 bit patterns [E, h] of a router weight N(0, sd=1/sqrt(h)), so that
    x . wr has roughly unit variance, like the N(0,1) logits above."""
    return to_bf16_bits(normal(seed, TAG_WR, (cfg.E, cfg.h), std=1.0 / np.sqrt(cfg.h)))


def make_w13_f32(cfg: LayerConfig, seed: int, experts=None) -> np.ndarray:
    """fp32 [len(experts), 2i, h] (all experts by default)."""
    return _expert_weights(cfg, seed, TAG_W13, 2 * cfg.i, cfg.h, experts)


def make_w2_f32(cfg: LayerConfig, seed: int, experts=None) -> np.ndarray:
    """fp32 [len(experts), h, i] (all experts by default)."""
    return _expert_weights(cfg, seed, TAG_W2, cfg.h, cfg.i, experts)


def _expert_weights(cfg, seed, tag, N, K, experts):
    std = 1.0 / np.sqrt(K)
    per = N * K
    if experts is None:
        return normal(seed, tag, (cfg.E, N, K), std=std)
    experts = list(experts)
    out = np.empty((len(experts), N, K), dtype=np.float32)
    for j, e in enumerate(experts):
        out[j] = normal(seed, tag, (N, K), std=std, first=e * per)
    return out
