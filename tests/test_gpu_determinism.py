"""Bitwise run-to-run determinism of every path, eagerly and under HIP-graph
replay: each case runs once for its reference bits, then 20 eager runs and 20
replays of a captured graph (the outputs cleared before each replay, one eager
run between replays) must reproduce those bits exactly.  No oracle is
involved: the comparison is of the GPU result with itself, so the full batch
of every shape is cheap.

The pages ask for it twice: the Netra compiler architecture page, dense
templates paragraph (zero nondeterministic launches out of 200 and exact
20-replay HIP graphs), and the Inferact amd-kernels README, atomics rule (no
atomic sums, so a result reproduces run to run)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import log

pytestmark = pytest.mark.gpu

EAGER_RUNS = 20
GRAPH_REPLAYS = 20


@pytest.fixture(scope="module")
def moe_mod():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_block_scaled_router_amd as moe
    moe.lib()
    return moe


def _bits(t):
    return t.view(torch.uint8) if t.dtype.itemsize == 1 else t.view(torch.int16 if t.dtype.itemsize == 2 else torch.int32)


def _same(a, b):
    return torch.equal(_bits(a), _bits(b))


def _check_replays(label, run, outs):
    """run() enqueues the work that writes every tensor of `outs` on the
    current stream."""
    run()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    log(f"determinism {label}: {EAGER_RUNS} eager runs")
    for r in range(EAGER_RUNS):
        for o in outs:
            o.zero_()
        run()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert _same(o, ref), f"{label}: eager run {r} differs"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    log(f"determinism {label}: {GRAPH_REPLAYS} graph replays")
    for r in range(GRAPH_REPLAYS):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert _same(o, ref), f"{label}: graph replay {r} differs"
        run()   # eager work between replays
        torch.cuda.synchronize()
    del graph


def _device_layer(moe_mod, M, h, i, E, k, seed, cfg=None):
    """Inputs on the GPU: the shape's own x and logits when `cfg` is given
    (else N(0, 1)), weights N(0, 1/sqrt(K)) block-quantised by the library."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    if cfg is not None:
        x = torch.from_numpy(synth.make_x(cfg, seed).view(np.int16)).view(torch.bfloat16).to(dev)
        lg = torch.from_numpy(synth.make_logits(cfg, seed)).to(dev)
    else:
        x = torch.randn((M, h), generator=g, device=dev).to(torch.bfloat16)
        lg = torch.randn((M, E), generator=g, device=dev)
    q13, s13 = moe_mod.quantize_weight_block128(torch.randn((E, 2 * i, h), generator=g, device=dev) / h ** 0.5)
    q2, s2 = moe_mod.quantize_weight_block128(torch.randn((E, h, i), generator=g, device=dev) / i ** 0.5)
    return x, lg, q13, s13, q2, s2


def _layer_case(moe_mod, label, M, h, i, E, k, seed, cfg=None):
    x, lg, q13, s13, q2, s2 = _device_layer(moe_mod, M, h, i, E, k, seed, cfg)
    ws = moe_mod.alloc_workspace(M, h, i, E, k, device=x.device)
    out = torch.empty((M, h), dtype=torch.bfloat16, device=x.device)
    path = moe_mod.workspace_layout(M, h, i, E, k).path
    log(f"determinism {label}: M={M} h={h} i={i} E={E} k={k} path={path}")
    _check_replays(label, lambda: moe_mod.moe_fp8_forward_ws(x, lg, q13, s13, q2, s2, k, ws, out=out), [out])
    assert moe_mod.workspace_error(ws) == 0, "a wait between workgroups timed out"
    return path


@pytest.mark.parametrize("ci", [0, 1, 2, 3, 4, 5])
def test_layer_deterministic(moe_mod, ci):
    cfg = synth.CONFIGS[ci]
    _layer_case(moe_mod, cfg.name, cfg.M, cfg.h, cfg.i, cfg.E, cfg.k, synth.default_seed(ci), cfg)


@pytest.mark.parametrize("ci", [4, 5])
def test_producer_path_deterministic(moe_mod, ci):
    """The prefill producer and its reducer (asked for by path) on the
    prefill batch and the 768-row verify batch: grid barriers, device-scope
    hand-offs and per-M-tile counters reproduce the same bits every run, and
    leave no error."""
    cfg = synth.CONFIGS[ci]
    seed = synth.default_seed(ci)
    M, h, i, E, k = cfg.M, cfg.h, cfg.i, cfg.E, cfg.k
    x, lg, q13, s13, q2, s2 = _device_layer(moe_mod, M, h, i, E, k, seed, cfg)
    path = moe_mod.PATH_PRODUCER
    ws = moe_mod.alloc_workspace(M, h, i, E, k, device=x.device, path=path)
    out = torch.empty((M, h), dtype=torch.bfloat16, device=x.device)
    log(f"determinism producer {cfg.name}")
    _check_replays("producer_" + cfg.name,
                   lambda: moe_mod.moe_fp8_forward_ws_path(x, lg, q13, s13, q2, s2, k, ws, path, out=out), [out])
    assert moe_mod.workspace_error(ws) == 0, "a wait of the producer timed out"


def test_layer_deterministic_stream_path_many_routes(moe_mod):
    """The streaming path beyond the one-launch grouping (320 routes: routing
    and quantisation, then the chunked histogram and scatter)."""
    path = _layer_case(moe_mod, "stream_m40_h2048_i768_e128_top8", 40, 2048, 768, 128, 8, 4040)
    assert path == moe_mod.PATH_STREAM


@pytest.mark.parametrize("ci", [3, 4])
def test_mxfp4_layer_deterministic(moe_mod, ci):
    """The MXFP4-weight layer at its own shape (h 6144, i 768, E 128, top-4,
    64 tokens: the streaming kernels) and at the prefill batch's (8192 tokens,
    h 2048, i 768, E 128, top-8: the tiled kernels), random E2M1 codes and
    E8M0 scales near 2^-8."""
    cfg = synth.CONFIGS[ci]
    seed = synth.default_seed(ci)
    M, h, i, E, k = cfg.M, cfg.h, cfg.i, cfg.E, cfg.k
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    w13 = torch.randint(0, 256, (E, 2 * i, h // 2), dtype=torch.uint8, device=dev, generator=g)
    e13 = torch.randint(117, 122, (E, 2 * i, h // 32), dtype=torch.uint8, device=dev, generator=g)
    w2 = torch.randint(0, 256, (E, h, i // 2), dtype=torch.uint8, device=dev, generator=g)
    e2 = torch.randint(117, 122, (E, h, i // 32), dtype=torch.uint8, device=dev, generator=g)
    x = torch.from_numpy(synth.make_x(cfg, seed).view(np.int16)).view(torch.bfloat16).to(dev)
    lg = torch.from_numpy(synth.make_logits(cfg, seed)).to(dev)
    ws = moe_mod.alloc_mxfp4_workspace(M, h, i, E, k, device=dev)
    out = torch.empty((M, h), dtype=torch.bfloat16, device=dev)
    _check_replays("mxfp4_" + cfg.name, lambda: moe_mod.moe_mxfp4_forward_ws(x, lg, w13, e13, w2, e2, k, ws,
                                                                             out=out), [out])


@pytest.mark.parametrize("ci,want_logits", [(1, True), (2, True), (4, True), (4, False)])
def test_router_gemm_topk_deterministic(moe_mod, ci, want_logits):
    """BF16 routing fused with the top-k: the expert-split kernel plus the row
    router (few tokens, logits kept) and the fused kernel (many tokens, or no
    logits)."""
    cfg = synth.CONFIGS[ci]
    seed = synth.default_seed(ci)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(synth.make_x(cfg, seed).view(np.int16)).view(torch.bfloat16).to(dev)
    wr = torch.from_numpy(synth.make_wr(cfg, seed).view(np.int16)).view(torch.bfloat16).to(dev)
    M, E, k = cfg.M, cfg.E, cfg.k
    logits = torch.empty((M, E), dtype=torch.float32, device=dev) if want_logits else None
    ids = torch.empty((M, k), dtype=torch.int32, device=dev)
    w = torch.empty((M, k), dtype=torch.float32, device=dev)
    outs = [t for t in (logits, ids, w) if t is not None]
    _check_replays(f"router_gemm_topk_{cfg.name}_logits{int(want_logits)}",
                   lambda: moe_mod.router_gemm_topk(x, wr, k, out=(logits, ids, w)), outs)
