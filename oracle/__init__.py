"""CPU oracle for the routed FP8 block-scaled MoE layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check
and by the benchmark's CPU-baseline leg -- never by the GPU library or its
Python binding.  The arithmetic lives in ``moe_oracle.c`` (plain C, see its
header for the pages followed and every rounding point); this module only
marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64


class _Dbg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("ids", "topk_w", "xq", "xs", "counts", "offsets", "sorted", "g", "a2", "a2s", "y")]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run oracle/build.py")
        L = ctypes.CDLL(_LIB_PATH)
        sigs = {
            "oracle_e4m3_decode": (ctypes.c_float, [ctypes.c_uint8]),
            "oracle_e4m3_table": (ctypes.c_void_p, []),
            "oracle_e4m3_encode": (ctypes.c_uint8, [ctypes.c_float]),
            "oracle_e4m3_encode_linear": (ctypes.c_uint8, [ctypes.c_float]),
            "oracle_e4m3_encode_array": (None, [_P, _I64, _P]),
            "oracle_bf16_encode": (ctypes.c_uint16, [ctypes.c_float]),
            "oracle_bf16_decode": (ctypes.c_float, [ctypes.c_uint16]),
            "oracle_set_threads": (None, [_I]),
            "oracle_get_threads": (_I, []),
            "oracle_quant_weight_block128": (None, [_P, _I64, _I, _I, _P, _P]),
            "oracle_router": (None, [_P, _I, _I, _I, _P, _P]),
            "oracle_act_quant": (None, [_P, _I, _I, _P, _P]),
            "oracle_rmsnorm_act_quant": (None, [_P, _P, ctypes.c_float, _I, _I, _P, _P, _P]),
            "oracle_router_logits": (None, [_P, _P, _I, _I, _I, _P]),
            "oracle_group": (None, [_P, _I, _I, _P, _P, _P]),
            "oracle_block_gemm": (None, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P]),
            "oracle_silu_mul_quant": (None, [_P, _I, _I, _P, _P]),
            "oracle_combine": (None, [_P, _P, _I, _I, _I, _P]),
            "oracle_moe_forward": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                        ctypes.POINTER(_Dbg)]),
            "oracle_e2m1_decode": (ctypes.c_float, [ctypes.c_uint8]),
            "oracle_e2m1_encode": (ctypes.c_uint8, [ctypes.c_float]),
            "oracle_e8m0_decode": (ctypes.c_double, [ctypes.c_uint8]),
            "oracle_mxfp4_quantize": (None, [_P, _I64, _I, _P, _P]),
            "oracle_moe_forward_mxfp4": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                              ctypes.POINTER(_Dbg)]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(lib().oracle_get_threads())


def e4m3_table() -> np.ndarray:
    p = lib().oracle_e4m3_table()
    return np.ctypeslib.as_array(ctypes.cast(p, ctypes.POINTER(ctypes.c_float)), shape=(256,)).copy()


def e4m3_encode(v: float) -> int:
    return int(lib().oracle_e4m3_encode(float(v)))


def e4m3_encode_linear(v: float) -> int:
    return int(lib().oracle_e4m3_encode_linear(float(v)))


def e4m3_encode_array(v) -> np.ndarray:
    v, pv = _c(v, np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_array(pv, v.size, out.ctypes.data)
    return out


def bf16_encode(v: float) -> int:
    return int(lib().oracle_bf16_encode(float(v)))


def bf16_encode_array(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    f = lib().oracle_bf16_encode
    return np.array([f(float(x)) for x in v], dtype=np.uint16)


def quant_weight_block128(w: np.ndarray):
    """fp32 [B, N, K] -> (codes uint8 [B, N, K], scales fp32 [B, N/128, K/128])."""
    w, pw = _c(w, np.float32)
    B, N, K = w.shape
    q = np.empty((B, N, K), dtype=np.uint8)
    s = np.empty((B, N // 128, K // 128), dtype=np.float32)
    lib().oracle_quant_weight_block128(pw, B, N, K, q.ctypes.data, s.ctypes.data)
    return q, s


def router(logits: np.ndarray, k: int):
    logits, pl = _c(logits, np.float32)
    M, E = logits.shape
    ids = np.empty((M, k), dtype=np.int32)
    w = np.empty((M, k), dtype=np.float32)
    lib().oracle_router(pl, M, E, k, ids.ctypes.data, w.ctypes.data)
    return ids, w


def act_quant(x_bits: np.ndarray):
    x, px = _c(x_bits, np.uint16)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // 128), dtype=np.float32)
    lib().oracle_act_quant(px, M, K, q.ctypes.data, s.ctypes.data)
    return q, s


def router_logits(x_bits: np.ndarray, wr_bits: np.ndarray):
    """BF16 routing logits fp32 [M, E] of bf16 rows [M, K] and a bf16 router
    weight [E, K] (see oracle_router_logits)."""
    x, px = _c(x_bits, np.uint16)
    w, pw = _c(wr_bits, np.uint16)
    M, K = x.shape
    E = w.shape[0]
    assert w.shape == (E, K)
    out = np.empty((M, E), dtype=np.float32)
    lib().oracle_router_logits(px, pw, M, K, E, out.ctypes.data)
    return out


def rmsnorm_act_quant(x_bits: np.ndarray, gamma: np.ndarray, eps: float):
    """RMSNorm of bf16 rows to bf16, then the 1x128 quantisation (see
    oracle_rmsnorm_act_quant).  Returns (y bf16 bits, codes, scales)."""
    x, px = _c(x_bits, np.uint16)
    g, pg = _c(gamma, np.float32)
    M, K = x.shape
    assert g.shape == (K,) and K % 128 == 0
    y = np.empty((M, K), dtype=np.uint16)
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // 128), dtype=np.float32)
    lib().oracle_rmsnorm_act_quant(px, pg, float(eps), M, K, y.ctypes.data, q.ctypes.data, s.ctypes.data)
    return y, q, s


def group(ids: np.ndarray, E: int):
    ids, pi = _c(ids, np.int32)
    R = ids.size
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    srt = np.empty(R, dtype=np.int32)
    lib().oracle_group(pi, R, E, counts.ctypes.data, offsets.ctypes.data, srt.ctypes.data)
    return counts, offsets, srt


def block_gemm(A, As, arow, W, Ws, wsel):
    A, pA = _c(A, np.uint8)
    As, pAs = _c(As, np.float32)
    arow, par = _c(arow, np.int32)
    W, pW = _c(W, np.uint8)
    Ws, pWs = _c(Ws, np.float32)
    wsel, pws = _c(wsel, np.int32)
    R = arow.size
    N, K = W.shape[-2], W.shape[-1]
    out = np.empty((R, N), dtype=np.float32)
    lib().oracle_block_gemm(pA, pAs, par, pW, pWs, pws, R, N, K, out.ctypes.data)
    return out


def silu_mul_quant(g: np.ndarray):
    g, pg = _c(g, np.float32)
    R, I2 = g.shape
    I = I2 // 2
    a2 = np.empty((R, I), dtype=np.uint8)
    a2s = np.empty((R, I // 128), dtype=np.float32)
    lib().oracle_silu_mul_quant(pg, R, I, a2.ctypes.data, a2s.ctypes.data)
    return a2, a2s


def combine(y: np.ndarray, w: np.ndarray):
    w, pw = _c(w, np.float32)
    M, k = w.shape
    y, py = _c(y, np.float32)
    H = y.shape[-1]
    out = np.empty((M, H), dtype=np.uint16)
    lib().oracle_combine(py, pw, M, k, H, out.ctypes.data)
    return out


def moe_forward(x_bits, logits, w13, s13, w2, s2, k: int, intermediates: bool = False):
    """Whole layer; returns bf16 bits [M, h] (and a dict of intermediates)."""
    x, px = _c(x_bits, np.uint16)
    logits, pl = _c(logits, np.float32)
    w13, p13 = _c(w13, np.uint8)
    s13, ps13 = _c(s13, np.float32)
    w2, p2 = _c(w2, np.uint8)
    s2, ps2 = _c(s2, np.float32)
    M, h = x.shape
    E, I2, h2 = w13.shape
    i = I2 // 2
    if h2 != h or logits.shape != (M, E) or w2.shape != (E, h, i):
        raise ValueError("inconsistent shapes")
    out = np.empty((M, h), dtype=np.uint16)
    dbg = None
    arrays = {}
    if intermediates:
        R = M * k
        arrays = dict(ids=np.empty(R, np.int32), topk_w=np.empty(R, np.float32),
                      xq=np.empty((M, h), np.uint8), xs=np.empty((M, h // 128), np.float32),
                      counts=np.empty(E, np.int32), offsets=np.empty(E + 1, np.int32),
                      sorted=np.empty(R, np.int32), g=np.empty((R, 2 * i), np.float32),
                      a2=np.empty((R, i), np.uint8), a2s=np.empty((R, i // 128), np.float32),
                      y=np.empty((R, h), np.float32))
        dbg = _Dbg(**{n: a.ctypes.data for n, a in arrays.items()})
    rc = lib().oracle_moe_forward(px, pl, p13, ps13, p2, ps2, out.ctypes.data,
                                  M, h, i, E, k, ctypes.byref(dbg) if dbg is not None else None)
    if rc != 0:
        raise ValueError(f"oracle_moe_forward rejected the shape (rc={rc})")
    if intermediates:
        arrays["ids"] = arrays["ids"].reshape(M, k)
        arrays["topk_w"] = arrays["topk_w"].reshape(M, k)
        return out, arrays
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------ MXFP4 variant

def e2m1_decode(code: int) -> float:
    return float(lib().oracle_e2m1_decode(int(code)))


def e2m1_encode(v: float) -> int:
    return int(lib().oracle_e2m1_encode(float(v)))


def e8m0_decode(code: int) -> float:
    return float(lib().oracle_e8m0_decode(int(code)))


def mxfp4_quantize(w: np.ndarray):
    """fp32 [..., K] -> (codes uint8 [..., K/2], E8M0 scales uint8 [..., K/32])
    (see oracle_mxfp4_quantize)."""
    w, pw = _c(w, np.float32)
    K = w.shape[-1]
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    rows = w.size // K
    codes = np.empty(w.shape[:-1] + (K // 2,), np.uint8)
    scales = np.empty(w.shape[:-1] + (K // 32,), np.uint8)
    lib().oracle_mxfp4_quantize(pw, rows, K, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def mxfp4_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 values of MXFP4 rows: nibble decode by the oracle's table times
    2^(scale - 127)."""
    T = np.array([e2m1_decode(c) for c in range(16)], np.float64)
    lo, hi = codes & 15, codes >> 4
    vals = np.stack([T[lo], T[hi]], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
    sc = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return vals * np.repeat(sc, 32, axis=-1)


def moe_forward_mxfp4(x_bits, logits, w13, e13, w2, e2, k: int, intermediates: bool = False):
    """Whole layer with MXFP4 weights; returns bf16 bits [M, h] (and a dict of
    intermediates: ids, topk_w, xq, xs, g, a2, a2s, y)."""
    x, px = _c(x_bits, np.uint16)
    logits, pl = _c(logits, np.float32)
    w13, p13 = _c(w13, np.uint8)
    e13, pe13 = _c(e13, np.uint8)
    w2, p2 = _c(w2, np.uint8)
    e2, pe2 = _c(e2, np.uint8)
    M, h = x.shape
    E, I2, hh = w13.shape
    i = I2 // 2
    if hh * 2 != h or logits.shape != (M, E) or w2.shape != (E, h, i // 2) or e13.shape != (E, I2, h // 32) \
            or e2.shape != (E, h, i // 32):
        raise ValueError("inconsistent shapes")
    out = np.empty((M, h), dtype=np.uint16)
    dbg = None
    arrays = {}
    if intermediates:
        R = M * k
        arrays = dict(ids=np.empty(R, np.int32), topk_w=np.empty(R, np.float32),
                      xq=np.empty((M, h), np.uint8), xs=np.empty((M, h // 128), np.float32),
                      g=np.empty((R, 2 * i), np.float32), a2=np.empty((R, i), np.uint8),
                      a2s=np.empty((R, i // 128), np.float32), y=np.empty((R, h), np.float32))
        dbg = _Dbg(**{n: a.ctypes.data for n, a in arrays.items()})
    rc = lib().oracle_moe_forward_mxfp4(px, pl, p13, pe13, p2, pe2, out.ctypes.data, M, h, i, E, k,
                                        ctypes.byref(dbg) if dbg is not None else None)
    if rc != 0:
        raise ValueError(f"oracle_moe_forward_mxfp4 rejected the shape (rc={rc})")
    if intermediates:
        arrays["ids"] = arrays["ids"].reshape(M, k)
        arrays["topk_w"] = arrays["topk_w"].reshape(M, k)
        return out, arrays
    return out
