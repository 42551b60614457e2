"""Routed FP8 (E4M3, 128x128 block-scaled) MoE expert FFN for MI355X (gfx950).

Thin Python binding over the C ABI of ``include/moe_fp8.h``
(``libmoe_fp8.so``): it checks dtypes, devices, shapes and contiguity of
torch tensors and passes raw device pointers and the current HIP stream.
Every step of the layer runs in the library's HIP kernels; there is no
Python or CPU fallback -- if the library is not built, every call raises.
PyTorch only supplies device memory and streams.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_fp8.so")

MOE_OK = 0
MOE_ERR_INVALID = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4

MAX_EXPERTS = 256
MAX_TOPK = 16

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "topk_ids", "topk_w", "xq", "xs", "counts", "offsets", "sorted", "active",
        "num_active", "gate_up", "act2", "act2_scale", "partial", "sync_error", "total")] + [
        ("path", ctypes.c_int)]


PATH_STREAM = 0
PATH_PREFILL = 1
PATH_FUSED_DECODE = 2
PATH_PRODUCER = 3
PATH_NAMES = {PATH_STREAM: "stream", PATH_PREFILL: "prefill", PATH_FUSED_DECODE: "one-kernel",
              PATH_PRODUCER: "producer"}
ERR_FUSED_WAIT = 1
ERR_PRODUCER_WAIT = 2


_SIGS = {
    "moe_fp8_status_string": (ctypes.c_char_p, [_I]),
    "moe_fp8_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "moe_fp8_bind_workspace": (_I, [_P, _SZ]),
    "moe_fp8_forward": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "moe_fp8_forward_ws": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _P]),
    "moe_fp8_workspace_layout": (_I, [_I, _I, _I, _I, _I, ctypes.POINTER(WsLayout)]),
    "moe_mxfp4_workspace_layout": (_I, [_I, _I, _I, _I, _I, ctypes.POINTER(WsLayout)]),
    "moe_fp8_workspace_bytes_path": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "moe_fp8_workspace_layout_path": (_I, [_I, _I, _I, _I, _I, _I, ctypes.POINTER(WsLayout)]),
    "moe_fp8_forward_ws_path": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _I, _P]),
    "moe_mxfp4_workspace_bytes_path": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "moe_mxfp4_forward_ws_path": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _I, _P]),
    "moe_mxfp4_forward_ws_timed": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _P, _I, _P]),
    "router_topk": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_fp8_router_gemm_topk": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P]),
    "moe_mxfp4_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "moe_mxfp4_forward_ws": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _P]),
    "moe_mxfp4_forward_ws_prefix": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _I, _P]),
    "moe_fp8_act_quant": (_I, [_P, _I, _I, _P, _P, _P]),
    "moe_fp8_rmsnorm_act_quant": (_I, [_P, _P, ctypes.c_float, _I, _I, _P, _P, _P, _P]),
    "moe_fp8_group_workspace_bytes": (_SZ, [_I, _I, _I]),
    "moe_fp8_group": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_fp8_quantize_weight_block128": (_I, [_P, _I64, _I, _I, _P, _P, _P]),
    "moe_fp8_encode_e4m3": (_I, [_P, _I64, _P, _P]),
    "moe_fp8_forward_ws_timed": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _P, _I, _P]),
    "moe_fp8_forward_ws_prefix": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _I, _P]),
    "moe_fp8_forward_kernel_count": (_I, [_I, _I, _I, _I, _I]),
    "moe_fp8_forward_kernel_name": (ctypes.c_char_p, [_I, _I, _I, _I, _I, _I]),
    "moe_mxfp4_forward_kernel_count": (_I, [_I, _I, _I, _I, _I]),
    "moe_mxfp4_forward_kernel_name": (ctypes.c_char_p, [_I, _I, _I, _I, _I, _I]),
    "moe_fp8_workspace_init": (_I, [_P, _SZ, _P]),
    "moe_fp8_workspace_head_bytes": (_SZ, []),
    "moe_fp8_workspace_status": (_I, [_P, _SZ, _I, ctypes.POINTER(ctypes.c_uint32), _P]),
    "moe_fp8_probe_empty": (_I, [_I, _P]),
    "moe_fp8_forward_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "moe_fp8_probe_read": (_I, [_P, _SZ, _I, _P, _P]),
}


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run fp8_block_scaled_router_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_fp8_status_string(int(status)).decode()


def _check(rc: int, what: str) -> None:
    if rc != MOE_OK:
        raise MoeError(rc, what)


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, dtype, name, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def workspace_bytes(M: int, h: int, i: int, E: int, k: int) -> int:
    return int(lib().moe_fp8_workspace_bytes(M, h, i, E, k))


def workspace_layout(M: int, h: int, i: int, E: int, k: int) -> WsLayout:
    L = WsLayout()
    _check(lib().moe_fp8_workspace_layout(M, h, i, E, k, ctypes.byref(L)), "moe_fp8_workspace_layout")
    return L


def alloc_workspace(M: int, h: int, i: int, E: int, k: int, device=None, path: int | None = None) -> torch.Tensor:
    """A workspace for these sizes (and, when given, that path); its
    synchronisation words start at zero."""
    if path is None:
        need = workspace_bytes(M, h, i, E, k)
    else:
        need = int(lib().moe_fp8_workspace_bytes_path(M, h, i, E, k, int(path)))
        if need == 0:
            raise MoeError(MOE_ERR_UNSUPPORTED, "moe_fp8_workspace_bytes_path")
    n = max(need, int(lib().moe_fp8_workspace_head_bytes()))
    ws = torch.empty(n, dtype=torch.uint8, device=device or "cuda")
    workspace_init(ws)
    return ws


def workspace_layout_path(M: int, h: int, i: int, E: int, k: int, path: int) -> WsLayout:
    L = WsLayout()
    _check(lib().moe_fp8_workspace_layout_path(M, h, i, E, k, int(path), ctypes.byref(L)),
           "moe_fp8_workspace_layout_path")
    return L


def workspace_init(ws: torch.Tensor, stream=None) -> None:
    _dev(ws, torch.uint8, "workspace")
    _check(lib().moe_fp8_workspace_init(_ptr(ws), ws.numel(), _stream(stream)), "moe_fp8_workspace_init")


def workspace_error(ws: torch.Tensor, clear: bool = False, stream=None) -> int:
    """The workspace's sticky error word after the work queued on `stream`
    (0 = every wait between workgroups completed; otherwise a forward's wait
    timed out and its output is invalid); `clear` resets it.  Synchronises
    the stream."""
    _dev(ws, torch.uint8, "workspace")
    flags = ctypes.c_uint32(0)
    _check(lib().moe_fp8_workspace_status(_ptr(ws), ws.numel(), int(bool(clear)), ctypes.byref(flags),
                                          _stream(stream)), "moe_fp8_workspace_status")
    return int(flags.value)


def probe_empty(grid: int, stream=None) -> None:
    """Measurement: one empty kernel of `grid` 256-thread workgroups."""
    _check(lib().moe_fp8_probe_empty(int(grid), _stream(stream)), "moe_fp8_probe_empty")


def probe_read(src: torch.Tensor, grid: int, sink: torch.Tensor, stream=None) -> None:
    """Measurement: one kernel of `grid` workgroups streaming all of `src`
    (uint8, size a multiple of 16) from HBM; sink is int32 [>= 4 * grid]."""
    _dev(src, torch.uint8, "src")
    _dev(sink, torch.int32, "sink")
    if sink.numel() < 4 * grid:
        raise ValueError("sink must hold 4 * grid words")
    _check(lib().moe_fp8_probe_read(_ptr(src), src.numel(), int(grid), _ptr(sink), _stream(stream)),
           "moe_fp8_probe_read")


SYNC_EPOCH_OFFSET = 0     # forwards of the one-kernel path run on a workspace
SYNC_EXIT_OFFSET = 256    # zero between forwards


_bound = {}


def bind_workspace(ws: torch.Tensor | None) -> None:
    """Bind `ws` as the workspace moe_fp8_forward uses on ws's device (the
    tensor is kept alive here while bound); None unbinds the current device."""
    if ws is None:
        _check(lib().moe_fp8_bind_workspace(None, 0), "moe_fp8_bind_workspace")
        _bound.pop(torch.cuda.current_device(), None)
        return
    _dev(ws, torch.uint8, "workspace")
    with torch.cuda.device(ws.device):
        _check(lib().moe_fp8_bind_workspace(_ptr(ws), ws.numel()), "moe_fp8_bind_workspace")
    _bound[ws.device.index] = ws


def _layer_args(x, router_logits, w13, s13, w2, s2, k, out):
    M, h = x.shape
    E = router_logits.shape[1]
    i = w2.shape[2]
    _dev(x, torch.bfloat16, "x", (M, h))
    _dev(router_logits, torch.float32, "router_logits", (M, E))
    _dev(w13, torch.float8_e4m3fn, "w13", (E, 2 * i, h))
    _dev(s13, torch.float32, "s13", (E, 2 * i // 128, h // 128))
    _dev(w2, torch.float8_e4m3fn, "w2", (E, h, i))
    _dev(s2, torch.float32, "s2", (E, h // 128, i // 128))
    if out is None:
        out = torch.empty((M, h), dtype=torch.bfloat16, device=x.device)
    _dev(out, torch.bfloat16, "out", (M, h))
    return M, h, i, E, out


def moe_fp8_forward(x, router_logits, w13, s13, w2, s2, k: int, out=None, stream=None):
    """The layer with the workspace bound by bind_workspace()."""
    M, h, i, E, out = _layer_args(x, router_logits, w13, s13, w2, s2, k, out)
    rc = lib().moe_fp8_forward(_ptr(x), _ptr(router_logits), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2),
                               _ptr(out), M, h, i, E, int(k), _stream(stream))
    _check(rc, "moe_fp8_forward")
    return out


def moe_fp8_forward_ws(x, router_logits, w13, s13, w2, s2, k: int, workspace, out=None, stream=None):
    """The layer with an explicit workspace tensor (uint8, on the same device)."""
    M, h, i, E, out = _layer_args(x, router_logits, w13, s13, w2, s2, k, out)
    _dev(workspace, torch.uint8, "workspace")
    rc = lib().moe_fp8_forward_ws(_ptr(x), _ptr(router_logits), _ptr(w13), _ptr(s13), _ptr(w2),
                                  _ptr(s2), _ptr(out), M, h, i, E, int(k), _ptr(workspace),
                                  workspace.numel(), _stream(stream))
    _check(rc, "moe_fp8_forward_ws")
    return out


def moe_fp8_forward_ws_path(x, router_logits, w13, s13, w2, s2, k: int, workspace, path: int, out=None,
                            stream=None):
    """The layer on the given path (PATH_*), for measurement and testing; the
    workspace is sized for that path (alloc_workspace(..., path=path))."""
    M, h, i, E, out = _layer_args(x, router_logits, w13, s13, w2, s2, k, out)
    _dev(workspace, torch.uint8, "workspace")
    rc = lib().moe_fp8_forward_ws_path(_ptr(x), _ptr(router_logits), _ptr(w13), _ptr(s13), _ptr(w2),
                                       _ptr(s2), _ptr(out), M, h, i, E, int(k), _ptr(workspace),
                                       workspace.numel(), int(path), _stream(stream))
    _check(rc, "moe_fp8_forward_ws_path")
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_fp8_forward_noalloc(x, router_logits, w13, s13, w2, s2, k: int, out=None, stream=None):
    """The layer with the library's fixed per-device workspace (no allocation
    by the library; `out` is allocated here only when not given).  Sizes whose
    workspace exceeds NOALLOC_SCRATCH_BYTES raise MoeError (MOE_ERR_WORKSPACE);
    overlapping calls on one device race."""
    M, h, i, E, out = _layer_args(x, router_logits, w13, s13, w2, s2, k, out)
    rc = lib().moe_fp8_forward_noalloc(_ptr(x), _ptr(router_logits), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2),
                                       _ptr(out), M, h, i, E, int(k), _stream(stream))
    _check(rc, "moe_fp8_forward_noalloc")
    return out


def router_topk(logits, k: int, stream=None):
    M, E = logits.shape
    _dev(logits, torch.float32, "logits")
    ids = torch.empty((M, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((M, k), dtype=torch.float32, device=logits.device)
    _check(lib().router_topk(_ptr(logits), M, E, int(k), _ptr(ids), _ptr(w), _stream(stream)), "router_topk")
    return ids, w


def mxfp4_workspace_bytes(M: int, h: int, i: int, E: int, k: int) -> int:
    return int(lib().moe_mxfp4_workspace_bytes(M, h, i, E, k))


def mxfp4_workspace_layout(M: int, h: int, i: int, E: int, k: int) -> WsLayout:
    L = WsLayout()
    _check(lib().moe_mxfp4_workspace_layout(M, h, i, E, k, ctypes.byref(L)), "moe_mxfp4_workspace_layout")
    return L


def alloc_mxfp4_workspace(M: int, h: int, i: int, E: int, k: int, device=None,
                          path: int | None = None) -> torch.Tensor:
    """A workspace for moe_mxfp4_forward_ws (or, with `path`, for
    moe_mxfp4_forward_ws_path on that path) with its head cleared."""
    n = mxfp4_workspace_bytes(M, h, i, E, k) if path is None else \
        int(lib().moe_mxfp4_workspace_bytes_path(M, h, i, E, k, int(path)))
    if n == 0:
        raise MoeError(MOE_ERR_UNSUPPORTED, "moe_mxfp4_workspace_bytes")
    ws = torch.empty(n, dtype=torch.uint8, device=device or "cuda")
    workspace_init(ws)
    return ws


def moe_mxfp4_stage_names(M: int, h: int, i: int, E: int, k: int) -> list:
    """Kernels of one MXFP4 forward in launch order (the prefix stages)."""
    n = lib().moe_mxfp4_forward_kernel_count(M, h, i, E, k)
    if n < 0:
        raise MoeError(n, "moe_mxfp4_forward_kernel_count")
    return [lib().moe_mxfp4_forward_kernel_name(M, h, i, E, k, j).decode() for j in range(n)]


def moe_mxfp4_forward_ws(x, router_logits, w13, e13, w2, e2, k: int, workspace, out=None, stream=None,
                         n_stages: int | None = None):
    """The layer with MXFP4 weights: w13 uint8 codes [E, 2i, h/2] + e13 uint8
    E8M0 scales [E, 2i, h/32], w2 [E, h, i/2] + e2 [E, h, i/32].  n_stages
    cuts the forward after its first n launches (measurement)."""
    M, h = x.shape
    E = router_logits.shape[1]
    i = w2.shape[2] * 2
    _dev(x, torch.bfloat16, "x", (M, h))
    _dev(router_logits, torch.float32, "router_logits", (M, E))
    _dev(w13, torch.uint8, "w13", (E, 2 * i, h // 2))
    _dev(e13, torch.uint8, "e13", (E, 2 * i, h // 32))
    _dev(w2, torch.uint8, "w2", (E, h, i // 2))
    _dev(e2, torch.uint8, "e2", (E, h, i // 32))
    _dev(workspace, torch.uint8, "workspace")
    if out is None:
        out = torch.empty((M, h), dtype=torch.bfloat16, device=x.device)
    _dev(out, torch.bfloat16, "out", (M, h))
    if n_stages is None:
        _check(lib().moe_mxfp4_forward_ws(_ptr(x), _ptr(router_logits), _ptr(w13), _ptr(e13), _ptr(w2),
                                          _ptr(e2), _ptr(out), M, h, i, E, int(k), _ptr(workspace),
                                          workspace.numel(), _stream(stream)), "moe_mxfp4_forward_ws")
    else:
        _check(lib().moe_mxfp4_forward_ws_prefix(_ptr(x), _ptr(router_logits), _ptr(w13), _ptr(e13), _ptr(w2),
                                                 _ptr(e2), _ptr(out), M, h, i, E, int(k), _ptr(workspace),
                                                 workspace.numel(), int(n_stages), _stream(stream)),
               "moe_mxfp4_forward_ws_prefix")
    return out


def moe_mxfp4_forward_ws_path(x, router_logits, w13, e13, w2, e2, k: int, workspace, path: int, out=None,
                              stream=None):
    """The MXFP4 layer on the given path (PATH_STREAM, PATH_PREFILL or
    PATH_PRODUCER), for measurement and testing."""
    M, h = x.shape
    E = router_logits.shape[1]
    i = w2.shape[2] * 2
    _dev(x, torch.bfloat16, "x", (M, h))
    _dev(router_logits, torch.float32, "router_logits", (M, E))
    _dev(w13, torch.uint8, "w13", (E, 2 * i, h // 2))
    _dev(e13, torch.uint8, "e13", (E, 2 * i, h // 32))
    _dev(w2, torch.uint8, "w2", (E, h, i // 2))
    _dev(e2, torch.uint8, "e2", (E, h, i // 32))
    _dev(workspace, torch.uint8, "workspace")
    if out is None:
        out = torch.empty((M, h), dtype=torch.bfloat16, device=x.device)
    _dev(out, torch.bfloat16, "out", (M, h))
    _check(lib().moe_mxfp4_forward_ws_path(_ptr(x), _ptr(router_logits), _ptr(w13), _ptr(e13), _ptr(w2), _ptr(e2),
                                           _ptr(out), M, h, i, E, int(k), _ptr(workspace), workspace.numel(),
                                           int(path), _stream(stream)),
           "moe_mxfp4_forward_ws_path")
    return out


def moe_mxfp4_forward_ws_timed(x, router_logits, w13, e13, w2, e2, k: int, workspace, events, out=None,
                               stream=None):
    """moe_mxfp4_forward_ws whose stage j stamps its start and end into events
    2j and 2j + 1 (HipEvents of at least twice the stage count)."""
    M, h = x.shape
    E = router_logits.shape[1]
    i = w2.shape[2] * 2
    _dev(x, torch.bfloat16, "x", (M, h))
    _dev(router_logits, torch.float32, "router_logits", (M, E))
    _dev(w13, torch.uint8, "w13", (E, 2 * i, h // 2))
    _dev(e13, torch.uint8, "e13", (E, 2 * i, h // 32))
    _dev(w2, torch.uint8, "w2", (E, h, i // 2))
    _dev(e2, torch.uint8, "e2", (E, h, i // 32))
    _dev(workspace, torch.uint8, "workspace")
    if out is None:
        out = torch.empty((M, h), dtype=torch.bfloat16, device=x.device)
    _dev(out, torch.bfloat16, "out", (M, h))
    _check(lib().moe_mxfp4_forward_ws_timed(_ptr(x), _ptr(router_logits), _ptr(w13), _ptr(e13), _ptr(w2), _ptr(e2),
                                            _ptr(out), M, h, i, E, int(k), _ptr(workspace), workspace.numel(),
                                            events.handles, events.n, _stream(stream)),
           "moe_mxfp4_forward_ws_timed")
    return out


def router_gemm_topk(x, wr, k: int, want_logits: bool = True, out=None, stream=None):
    """BF16 routing fused with the top-k: bf16 hidden rows x [M, h] and a bf16
    router weight wr [E, h] -> (logits fp32 [M, E] or None, ids int32 [M, k],
    weights fp32 [M, k]).  `out` = (logits or None, ids, w) writes into
    existing tensors."""
    M, h = x.shape
    E = wr.shape[0]
    _dev(x, torch.bfloat16, "x")
    _dev(wr, torch.bfloat16, "wr", (E, h))
    if out is not None:
        logits, ids, w = out
        if logits is not None:
            _dev(logits, torch.float32, "logits", (M, E))
        _dev(ids, torch.int32, "ids", (M, k))
        _dev(w, torch.float32, "w", (M, k))
    else:
        logits = torch.empty((M, E), dtype=torch.float32, device=x.device) if want_logits else None
        ids = torch.empty((M, k), dtype=torch.int32, device=x.device)
        w = torch.empty((M, k), dtype=torch.float32, device=x.device)
    _check(lib().moe_fp8_router_gemm_topk(_ptr(x), _ptr(wr), M, h, E, int(k),
                                          _ptr(logits) if logits is not None else None, _ptr(ids), _ptr(w),
                                          _stream(stream)), "moe_fp8_router_gemm_topk")
    return logits, ids, w


def act_quant(x, stream=None):
    M, K = x.shape
    _dev(x, torch.bfloat16, "x")
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = torch.empty((M, K // 128), dtype=torch.float32, device=x.device)
    _check(lib().moe_fp8_act_quant(_ptr(x), M, K, _ptr(q), _ptr(s), _stream(stream)), "moe_fp8_act_quant")
    return q, s


def rmsnorm_act_quant(x, gamma, eps: float, want_y: bool = True, out=None, stream=None):
    """bf16 [M, h] rows and fp32 [h] norm weight -> (y bf16 [M, h] or None,
    E4M3 codes uint8 [M, h], fp32 scales [M, h/128]).  `out` = (y or None,
    q, s) writes into existing tensors."""
    M, h = x.shape
    _dev(x, torch.bfloat16, "x")
    _dev(gamma, torch.float32, "gamma")
    if out is not None:
        y, q, s = out
        if y is not None:
            _dev(y, torch.bfloat16, "y", (M, h))
        _dev(q, torch.uint8, "q", (M, h))
        _dev(s, torch.float32, "s", (M, h // 128))
    else:
        y = torch.empty((M, h), dtype=torch.bfloat16, device=x.device) if want_y else None
        q = torch.empty((M, h), dtype=torch.uint8, device=x.device)
        s = torch.empty((M, h // 128), dtype=torch.float32, device=x.device)
    _check(lib().moe_fp8_rmsnorm_act_quant(_ptr(x), _ptr(gamma), float(eps), M, h,
                                           _ptr(y) if y is not None else None, _ptr(q), _ptr(s),
                                           _stream(stream)), "moe_fp8_rmsnorm_act_quant")
    return y, q, s


def group(topk_ids, E: int, stream=None):
    _dev(topk_ids, torch.int32, "topk_ids")
    M, k = topk_ids.shape
    dev = topk_ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    srt = torch.empty(M * k, dtype=torch.int32, device=dev)
    nws = max(int(lib().moe_fp8_group_workspace_bytes(M, E, k)), 256)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    _check(lib().moe_fp8_group(_ptr(topk_ids), M, E, k, _ptr(counts), _ptr(offsets), _ptr(srt),
                               _ptr(ws), nws, _stream(stream)), "moe_fp8_group")
    return counts, offsets, srt


def quantize_weight_block128(w, stream=None):
    """fp32 [B, N, K] on the GPU -> (float8_e4m3fn [B, N, K], fp32 scales [B, N/128, K/128])."""
    _dev(w, torch.float32, "w")
    B, N, K = w.shape
    q = torch.empty((B, N, K), dtype=torch.float8_e4m3fn, device=w.device)
    s = torch.empty((B, N // 128, K // 128), dtype=torch.float32, device=w.device)
    _check(lib().moe_fp8_quantize_weight_block128(_ptr(w), B, N, K, _ptr(q), _ptr(s), _stream(stream)),
           "moe_fp8_quantize_weight_block128")
    return q, s


def encode_e4m3(v, stream=None):
    _dev(v, torch.float32, "v")
    out = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    _check(lib().moe_fp8_encode_e4m3(_ptr(v), v.numel(), _ptr(out), _stream(stream)), "moe_fp8_encode_e4m3")
    return out


def forward_kernel_names(M: int, h: int, i: int, E: int, k: int) -> list:
    n = lib().moe_fp8_forward_kernel_count(M, h, i, E, k)
    if n < 0:
        raise MoeError(n, "moe_fp8_forward_kernel_count")
    return [lib().moe_fp8_forward_kernel_name(M, h, i, E, k, j).decode() for j in range(n)]


class HipEvents:
    """A set of HIP timing events (hipEventCreate), for moe_fp8_forward_ws_timed."""

    def __init__(self, n: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _P, _P]
        self._hip.hipEventDestroy.argtypes = [_P]
        self.handles = (ctypes.c_void_p * n)()
        for j in range(n):
            ev = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles[j] = ev
        self.n = n

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), self.handles[a], self.handles[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def close(self):
        for j in range(self.n):
            if self.handles[j]:
                self._hip.hipEventDestroy(self.handles[j])
                self.handles[j] = None


def moe_fp8_forward_ws_prefix(x, router_logits, w13, s13, w2, s2, k: int, workspace, n_stages: int,
                              out=None, stream=None):
    """moe_fp8_forward_ws cut after its first n_stages stages (measurement)."""
    M, h, i, E, out = _layer_args(x, router_logits, w13, s13, w2, s2, k, out)
    _dev(workspace, torch.uint8, "workspace")
    rc = lib().moe_fp8_forward_ws_prefix(_ptr(x), _ptr(router_logits), _ptr(w13), _ptr(s13), _ptr(w2),
                                         _ptr(s2), _ptr(out), M, h, i, E, int(k), _ptr(workspace),
                                         workspace.numel(), int(n_stages), _stream(stream))
    _check(rc, "moe_fp8_forward_ws_prefix")
    return out


def moe_fp8_forward_ws_timed(x, router_logits, w13, s13, w2, s2, k: int, workspace, events: HipEvents,
                             out=None, stream=None):
    """moe_fp8_forward_ws whose stage j stamps its start and end into events
    2j and 2j + 1 (HipEvents of at least twice the stage count)."""
    M, h, i, E, out = _layer_args(x, router_logits, w13, s13, w2, s2, k, out)
    _dev(workspace, torch.uint8, "workspace")
    rc = lib().moe_fp8_forward_ws_timed(_ptr(x), _ptr(router_logits), _ptr(w13), _ptr(s13), _ptr(w2),
                                        _ptr(s2), _ptr(out), M, h, i, E, int(k), _ptr(workspace),
                                        workspace.numel(), events.handles, events.n, _stream(stream))
    _check(rc, "moe_fp8_forward_ws_timed")
    return out
