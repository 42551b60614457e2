"""C-ABI checks that need no GPU: every function include/*.h declares is
exported by libmoe_fp8.so, and argument checks return the documented status
before any HIP call."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(hdr).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M):
            name = m.group(1)
            if name not in ("if", "while", "for", "sizeof", "defined"):
                names.add(name)
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    import fp8_block_scaled_router_amd as moe
    if not os.path.exists(moe.LIB_PATH):
        from fp8_block_scaled_router_amd import build
        build.build()
    return moe.lib()


def test_header_declares_the_expected_entry_points():
    names = _declared_functions()
    for required in ("moe_fp8_forward", "router_topk", "moe_fp8_forward_ws", "moe_fp8_group",
                     "moe_fp8_act_quant", "moe_fp8_workspace_bytes", "moe_fp8_bind_workspace"):
        assert required in names
    assert len(names) >= 12


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings(lib):
    import fp8_block_scaled_router_amd as moe
    assert moe.status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert moe.status_string(s) not in ("ok", "unknown status")
    assert moe.status_string(12345) == "unknown status"


FAKE = ctypes.c_void_p(0x100000)   # aligned, never dereferenced: checks fail first


def _fwd_ws(lib, M, h, i, E, k, ptr=FAKE, ws=FAKE, nws=0):
    return lib.moe_fp8_forward_ws(ptr, ptr, ptr, ptr, ptr, ptr, ptr, M, h, i, E, k, ws, nws, None)


def test_timed_forward_needs_two_events_per_stage(lib):
    """The timed entry takes a start and a stop event per stage: fewer than
    twice the stage count (or none) is rejected before any HIP call."""
    import fp8_block_scaled_router_amd as moe
    for M, h, i, E, k in ((4, 256, 128, 8, 2), (40, 384, 128, 2, 1)):   # one stage; five
        n = lib.moe_fp8_forward_kernel_count(M, h, i, E, k)
        assert n > 0
        evs = (ctypes.c_void_p * (2 * n))(*([0x100000] * (2 * n)))
        for short in sorted({0, n, n + 1, 2 * n - 1} - {2 * n}):
            assert lib.moe_fp8_forward_ws_timed(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, M, h, i, E, k, FAKE, 0,
                                                evs, short, None) == moe.MOE_ERR_INVALID
        assert lib.moe_fp8_forward_ws_timed(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, M, h, i, E, k, FAKE, 0,
                                            None, 2 * n, None) == moe.MOE_ERR_INVALID
        # enough events: the checks go on to the workspace (none given)
        assert lib.moe_fp8_forward_ws_timed(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, M, h, i, E, k, FAKE, 0,
                                            evs, 2 * n, None) == moe.MOE_ERR_WORKSPACE


def test_forward_argument_checks(lib):
    import fp8_block_scaled_router_amd as moe
    assert _fwd_ws(lib, -1, 256, 128, 8, 2) == moe.MOE_ERR_INVALID
    assert _fwd_ws(lib, 4, 0, 128, 8, 2) == moe.MOE_ERR_INVALID
    assert _fwd_ws(lib, 4, 200, 128, 8, 2) == moe.MOE_ERR_UNSUPPORTED      # h % 128
    assert _fwd_ws(lib, 4, 256, 100, 8, 2) == moe.MOE_ERR_UNSUPPORTED      # i % 128
    assert _fwd_ws(lib, 4, 256, 128, 300, 2) == moe.MOE_ERR_UNSUPPORTED    # E > 256
    assert _fwd_ws(lib, 4, 256, 128, 8, 9) == moe.MOE_ERR_UNSUPPORTED      # k > E
    assert _fwd_ws(lib, 4, 256, 128, 64, 17) == moe.MOE_ERR_UNSUPPORTED    # k > 16
    assert _fwd_ws(lib, 0, 256, 128, 8, 2) == moe.MOE_OK                   # M == 0: no-op
    assert _fwd_ws(lib, 4, 256, 128, 8, 2, ptr=ctypes.c_void_p(0)) == moe.MOE_ERR_INVALID
    assert _fwd_ws(lib, 4, 256, 128, 8, 2, ptr=ctypes.c_void_p(0x100004)) == moe.MOE_ERR_INVALID
    need = moe.workspace_bytes(4, 256, 128, 8, 2)
    assert _fwd_ws(lib, 4, 256, 128, 8, 2, ws=ctypes.c_void_p(0), nws=need) == moe.MOE_ERR_WORKSPACE
    assert _fwd_ws(lib, 4, 256, 128, 8, 2, nws=need - 1) == moe.MOE_ERR_WORKSPACE
    assert _fwd_ws(lib, 4, 256, 128, 8, 2, ws=ctypes.c_void_p(0x100010), nws=need) == moe.MOE_ERR_WORKSPACE


def test_other_entry_argument_checks(lib):
    import fp8_block_scaled_router_amd as moe
    assert lib.router_topk(FAKE, -1, 8, 2, FAKE, FAKE, None) == moe.MOE_ERR_INVALID
    assert lib.router_topk(FAKE, 4, 8, 9, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.router_topk(FAKE, 4, 257, 2, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.router_topk(FAKE, 0, 8, 2, FAKE, FAKE, None) == moe.MOE_OK
    assert lib.router_topk(None, 4, 8, 2, FAKE, FAKE, None) == moe.MOE_ERR_INVALID
    assert lib.moe_fp8_act_quant(FAKE, 4, 100, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_fp8_act_quant(None, 4, 128, FAKE, FAKE, None) == moe.MOE_ERR_INVALID
    rq = lib.moe_fp8_rmsnorm_act_quant
    assert rq(FAKE, FAKE, 1e-6, 4, 200, None, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert rq(FAKE, FAKE, 1e-6, 4, 8192 + 128, None, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert rq(FAKE, FAKE, -1.0, 4, 2048, None, FAKE, FAKE, None) == moe.MOE_ERR_INVALID
    assert rq(FAKE, FAKE, float("nan"), 4, 2048, None, FAKE, FAKE, None) == moe.MOE_ERR_INVALID
    assert rq(FAKE, FAKE, 1e-6, -1, 2048, None, FAKE, FAKE, None) == moe.MOE_ERR_INVALID
    assert rq(FAKE, None, 1e-6, 4, 2048, None, FAKE, FAKE, None) == moe.MOE_ERR_INVALID
    assert rq(FAKE, FAKE, 1e-6, 4, 2048, ctypes.c_void_p(0x100008), FAKE, FAKE, None) == moe.MOE_ERR_INVALID
    assert rq(FAKE, FAKE, 1e-6, 0, 2048, None, FAKE, FAKE, None) == moe.MOE_OK
    mx = lib.moe_mxfp4_forward_ws
    need = lib.moe_mxfp4_workspace_bytes(4, 256, 128, 8, 2)
    assert need > 0 and lib.moe_mxfp4_workspace_bytes(4, 200, 128, 8, 2) == 0
    W = ctypes.c_void_p(0x100000)
    assert mx(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 200, 128, 8, 2, W, need, None) == moe.MOE_ERR_UNSUPPORTED
    assert mx(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 256, 128, 8, 9, W, need, None) == moe.MOE_ERR_UNSUPPORTED
    assert mx(FAKE, FAKE, FAKE, ctypes.c_void_p(0x100002), FAKE, FAKE, FAKE, 4, 256, 128, 8, 2, W, need,
              None) == moe.MOE_ERR_INVALID                                  # scales not 4-byte aligned
    assert mx(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 256, 128, 8, 2, W, need, None) == moe.MOE_ERR_INVALID
    assert mx(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 256, 128, 8, 2, W, need - 1, None) == moe.MOE_ERR_WORKSPACE
    assert mx(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 256, 128, 8, 2, W, 0, None) == moe.MOE_OK
    rg = lib.moe_fp8_router_gemm_topk
    assert rg(FAKE, FAKE, 4, 200, 8, 2, None, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED   # h % 128
    assert rg(FAKE, FAKE, 4, 16384 + 128, 8, 2, None, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert rg(FAKE, FAKE, 4, 256, 257, 2, None, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED  # E > 256
    assert rg(FAKE, FAKE, 4, 256, 8, 9, None, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED    # k > E
    assert rg(FAKE, FAKE, 4, 256, 64, 17, None, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED  # k > 16
    assert rg(FAKE, FAKE, -1, 256, 8, 2, None, FAKE, FAKE, None) == moe.MOE_ERR_INVALID
    assert rg(FAKE, FAKE, 4, 256, 8, 0, None, FAKE, FAKE, None) == moe.MOE_ERR_INVALID
    assert rg(FAKE, None, 4, 256, 8, 2, None, FAKE, FAKE, None) == moe.MOE_ERR_INVALID
    assert rg(FAKE, FAKE, 4, 256, 8, 2, None, None, FAKE, None) == moe.MOE_ERR_INVALID
    assert rg(ctypes.c_void_p(0x100002), FAKE, 4, 256, 8, 2, None, FAKE, FAKE, None) == moe.MOE_ERR_INVALID
    assert rg(FAKE, FAKE, 0, 256, 8, 2, None, FAKE, FAKE, None) == moe.MOE_OK
    assert lib.moe_fp8_group(FAKE, 4, 8, 2, FAKE, FAKE, FAKE, FAKE, 0, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_fp8_group(FAKE, 4, 8, 9, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_fp8_quantize_weight_block128(FAKE, 1, 100, 128, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_fp8_quantize_weight_block128(FAKE, -1, 128, 128, FAKE, FAKE, None) == moe.MOE_ERR_INVALID
    assert lib.moe_fp8_encode_e4m3(FAKE, -5, FAKE, None) == moe.MOE_ERR_INVALID
    assert lib.moe_fp8_encode_e4m3(FAKE, 0, FAKE, None) == moe.MOE_OK
    assert lib.moe_fp8_bind_workspace(ctypes.c_void_p(0x100010), 1024) == moe.MOE_ERR_INVALID
    assert lib.moe_fp8_workspace_bytes(0, 256, 128, 8, 2) == 0
    assert lib.moe_fp8_workspace_bytes(4, 200, 128, 8, 2) == 0


@pytest.mark.parametrize("M,h,i,E,k", [(4, 256, 128, 8, 2), (1, 2048, 768, 128, 8),
                                       (12, 2048, 768, 128, 8), (64, 6144, 768, 128, 4),
                                       (8192, 2048, 768, 128, 8)])
def test_workspace_layout_regions(lib, M, h, i, E, k):
    import fp8_block_scaled_router_amd as moe
    L = moe.workspace_layout(M, h, i, E, k)
    R = M * k
    sizes = {"topk_ids": 4 * R, "topk_w": 4 * R, "xq": M * h, "xs": 4 * M * h // 128,
             "counts": 4 * E, "offsets": 4 * (E + 1), "sorted": 4 * R, "active": 4 * E,
             "num_active": 4, "gate_up": 4 * R * 2 * i, "act2": R * i, "act2_scale": 4 * R * i // 128,
             "partial": (2 if L.path in (moe.PATH_PREFILL, moe.PATH_PRODUCER) else 4) * R * h}   # bf16 / fp32 partials
    spans = []
    for name, n in sizes.items():
        off = getattr(L, name)
        if off == 2 ** 64 - 1:
            continue
        assert off % 256 == 0
        assert off + n <= L.total
        spans.append((off, off + n, name))
    spans.sort()
    for a, b in zip(spans, spans[1:]):
        assert a[1] <= b[0], (a, b)
    assert L.total == moe.workspace_bytes(M, h, i, E, k)


@pytest.mark.parametrize("M,h,i,E,k", [(1, 2048, 768, 128, 8), (2, 2048, 768, 128, 8), (3, 2048, 768, 128, 8),
                                       (127, 2048, 768, 128, 8), (128, 2048, 768, 128, 8), (40, 384, 128, 2, 1),
                                       (40, 256, 128, 2, 1), (64, 6144, 768, 128, 4), (256, 6144, 768, 128, 4)])
def test_fp8_path_rule(lib, M, h, i, E, k):
    """The FP8 forward's path: the one-kernel path for the smallest batches
    whose grid fits, else the five-launch tiled kernels when M*k >= 8*E and h
    is a multiple of 256, else the streaming kernels."""
    import fp8_block_scaled_router_amd as moe
    path = moe.workspace_layout(M, h, i, E, k).path
    if path != moe.PATH_FUSED_DECODE:
        tiled = M * k >= 8 * E and h % 256 == 0
        assert path == (moe.PATH_PREFILL if tiled else moe.PATH_STREAM)
    assert (path == moe.PATH_FUSED_DECODE) == (M <= 2 and h == 2048)


@pytest.mark.parametrize("M,h,i,E,k", [(1, 128, 128, 1, 1), (64, 6144, 768, 128, 4), (300, 256, 128, 4, 2),
                                       (1200, 2048, 768, 8, 2), (8192, 2048, 768, 128, 8), (200, 640, 384, 4, 2),
                                       (191, 2048, 768, 128, 8), (192, 2048, 768, 128, 8)])
def test_mxfp4_layout_and_path(lib, M, h, i, E, k):
    """The MXFP4 forward's path: the tiled kernels when M*k >= 12*E and h is a
    multiple of 256, else the streaming kernels (no one-kernel path); its
    stage names follow, and its regions fit its workspace."""
    import fp8_block_scaled_router_amd as moe
    L = moe.mxfp4_workspace_layout(M, h, i, E, k)
    tiled = M * k >= 12 * E and h % 256 == 0
    assert L.path == (moe.PATH_PREFILL if tiled else moe.PATH_STREAM)
    assert L.total == moe.mxfp4_workspace_bytes(M, h, i, E, k)
    names = moe.moe_mxfp4_stage_names(M, h, i, E, k)
    if tiled:
        assert names == ["route_quant_kernel", "group_hist+group_scatter", "prefill_gate_up_mx_kernel",
                         "prefill_down_mx_kernel", "combine_bf16_kernel"]
        assert L.act2 + M * k * i <= L.total and L.partial + 2 * M * k * h <= L.total
        assert L.gate_up == 2 ** 64 - 1
    else:
        assert names[-3:] == ["stream_gate_up_mx_kernel", "stream_down_mx_kernel", "combine_kernel"]
        assert L.gate_up + 4 * M * k * 2 * i <= L.total and L.partial + 4 * M * k * h <= L.total
        assert L.act2 == 2 ** 64 - 1
    assert lib.moe_mxfp4_forward_kernel_count(M, h, i, E, k) == len(names)
    assert lib.moe_mxfp4_forward_kernel_name(M, h, i, E, k, len(names)) is None


@pytest.mark.parametrize("M,h,i,E,k", [(768, 2048, 768, 128, 8), (8192, 2048, 768, 128, 8), (3, 384, 256, 6, 3),
                                       (1, 2048, 768, 128, 8), (900000, 256, 128, 8, 1)])
def test_forced_path_sizes(lib, M, h, i, E, k):
    """Each path's workspace size for the forced-path entries: 0 exactly when
    the path cannot take the batch; the chosen path's size is the default."""
    import fp8_block_scaled_router_amd as moe
    R = M * k
    tiled_ok = h % 256 == 0
    prod_ok = tiled_ok and (R + 127) // 128 + E <= 7168
    for path, ok in ((moe.PATH_STREAM, True), (moe.PATH_PREFILL, tiled_ok), (moe.PATH_PRODUCER, prod_ok)):
        n = lib.moe_fp8_workspace_bytes_path(M, h, i, E, k, path)
        assert (n > 0) == ok, (path, n)
        if ok:
            L = moe.workspace_layout_path(M, h, i, E, k, path)
            assert L.path == path and L.total == n
    chosen = moe.workspace_layout(M, h, i, E, k)
    assert lib.moe_fp8_workspace_bytes_path(M, h, i, E, k, chosen.path) == moe.workspace_bytes(M, h, i, E, k)
    if M * k >= 8 * E and tiled_ok:
        assert chosen.path == moe.PATH_PREFILL


def test_status_and_probe_argument_checks(lib):
    """The status reader and the measurement probes reject bad arguments
    before any HIP call."""
    flags = ctypes.c_uint32(0)
    assert lib.moe_fp8_workspace_status(None, 1 << 24, 0, ctypes.byref(flags), None) == -1
    assert lib.moe_fp8_workspace_status(FAKE, 1 << 24, 0, None, None) == -1
    assert lib.moe_fp8_workspace_status(ctypes.c_void_p(0x100010), 1 << 24, 0, ctypes.byref(flags), None) == -1
    assert lib.moe_fp8_workspace_status(FAKE, 1024, 0, ctypes.byref(flags), None) == -3
    assert lib.moe_fp8_probe_empty(0, None) == -1
    assert lib.moe_fp8_probe_empty((1 << 20) + 1, None) == -1
    assert lib.moe_fp8_probe_read(None, 1024, 4, FAKE, None) == -1
    assert lib.moe_fp8_probe_read(FAKE, 1000, 4, FAKE, None) == -1
    assert lib.moe_fp8_probe_read(ctypes.c_void_p(0x100008), 1024, 4, FAKE, None) == -1
    assert lib.moe_fp8_probe_read(FAKE, 1024, 0, FAKE, None) == -1
    assert lib.moe_fp8_probe_read(FAKE, 0, 4, FAKE, None) == 0
