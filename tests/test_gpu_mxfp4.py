"""GPU parity of the MXFP4-weight layer (C entry moe_mxfp4_forward_ws) against
the oracle's oracle_moe_forward_mxfp4, through the C ABI.

Routing ids, activation codes and scales are bit-exact.  The block-scaled FP4 x
FP8 matrix cores sum each 128-wide K block with fp32 accumulation; a gate/up
value lies within mfma_rel(h/128) * sum|terms| of the oracle's float64 value (pinned by
the gate/up check in _check_layer), and that bound, propagated through SiLU * up and
the 1x128 requantisation, flags the requantisation decisions that may land on
either code (gpu_util.flagged_codes); the output bar of the FP8 layer is
widened by the largest change those flips can cause."""
import functools

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (check_output, flagged_codes, flip_allowance, log, mfma_rel, r16_report, read_ws,
                      to_dev_bf16, to_host_bits, _T64)

pytestmark = pytest.mark.gpu

# The fp32 block-accumulation bound of the FP8 layer (gpu_util.mfma_rel), the
# same reading for the FP4 x FP8 matrix cores: each 128-wide K block is an
# fp32 sum of exact products (E2M1 x E8M0 x E4M3 is exact), order unspecified.


@pytest.fixture(scope="module")
def moe_mod():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_block_scaled_router_amd as moe
    moe.lib()
    return moe


@functools.lru_cache(maxsize=2)
def _mx_weights(cfg, seed):
    q13, e13 = oracle.mxfp4_quantize(synth.make_w13_f32(cfg, seed))
    q2, e2 = oracle.mxfp4_quantize(synth.make_w2_f32(cfg, seed))
    return q13, e13, q2, e2


class _MxLayer:
    def __init__(self, cfg, seed, x=None, logits=None):
        self.cfg = cfg
        self.x = synth.make_x(cfg, seed) if x is None else x
        self.logits = synth.make_logits(cfg, seed) if logits is None else logits
        self.q13, self.e13, self.q2, self.e2 = _mx_weights(cfg, seed)

    def w13_dense(self, e):
        return oracle.mxfp4_dequantize(self.q13[e], self.e13[e])

    @functools.lru_cache(maxsize=256)
    def w2_dense(self, e):
        return oracle.mxfp4_dequantize(self.q2[e], self.e2[e])

    def terms(self, inter, routes):
        """sum over K of |weight| * |activation| for the gate/up values of the routes."""
        T = _T64()
        M, k = inter["ids"].shape
        out = np.zeros((M * k, self.q13.shape[1]))
        routes = np.asarray(routes)
        flat = inter["ids"].ravel()[routes]
        for e in np.unique(flat):
            P = routes[flat == e]
            t = P // k
            a = np.abs(T[inter["xq"][t]]) * np.repeat(inter["xs"][t].astype(np.float64), 128, axis=1)
            out[P] = a @ np.abs(self.w13_dense(e)).T
        return out


def _run(moe_mod, L):
    dev = torch.device("cuda:0")
    M, h = L.x.shape
    E = L.logits.shape[1]
    i = L.q2.shape[2] * 2
    k = L.cfg.k
    ws = moe_mod.alloc_mxfp4_workspace(M, h, i, E, k, device=dev)
    args = [to_dev_bf16(L.x, dev), torch.from_numpy(np.ascontiguousarray(L.logits)).to(dev)] + \
        [torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (L.q13, L.e13, L.q2, L.e2)]
    out = moe_mod.moe_mxfp4_forward_ws(*args, k, ws)
    torch.cuda.synchronize()
    out2 = moe_mod.moe_mxfp4_forward_ws(*args, k, ws)
    torch.cuda.synchronize()
    got = to_host_bits(out)
    assert np.array_equal(to_host_bits(out2), got), "not deterministic"
    lay = moe_mod.mxfp4_workspace_layout(M, h, i, E, k)
    R = M * k
    ws_int = dict(ids=read_ws(ws, lay.topk_ids, R, np.int32).reshape(M, k),
                  xq=read_ws(ws, lay.xq, M * h, np.uint8).reshape(M, h),
                  xs=read_ws(ws, lay.xs, M * (h // 128), np.float32).reshape(M, h // 128),
                  g=read_ws(ws, lay.gate_up, R * 2 * i, np.float32).reshape(R, 2 * i)
                  if lay.path == moe_mod.PATH_STREAM else None,
                  sorted=read_ws(ws, lay.sorted, R, np.int32),
                  a2=read_ws(ws, lay.act2, R * i, np.uint8).reshape(R, i)
                  if lay.path in (moe_mod.PATH_PREFILL, moe_mod.PATH_PRODUCER) else None,
                  path=lay.path)
    return got, ws_int


def _check_layer(moe_mod, L, tokens=None):
    cfg = L.cfg
    k = cfg.k
    log(f"mxfp4 layer {cfg.name}: M={cfg.M} h={cfg.h} i={cfg.i} E={cfg.E} k={k}")
    got, wsi = _run(moe_mod, L)
    tok = np.arange(cfg.M) if tokens is None else np.asarray(tokens)
    ref, inter = oracle.moe_forward_mxfp4(L.x[tok], L.logits[tok], L.q13, L.e13, L.q2, L.e2, k,
                                          intermediates=True)
    assert np.array_equal(wsi["ids"][tok], inter["ids"])
    assert np.array_equal(wsi["xq"][tok], inter["xq"])
    assert np.array_equal(wsi["xs"][tok].view(np.uint32), inter["xs"].view(np.uint32))
    routes = np.arange(len(tok) * k)
    terms = L.terms(inter, routes)
    if wsi["g"] is not None:
        gpu_g = wsi["g"].reshape(cfg.M, k, -1)[tok].reshape(len(tok) * k, -1)
        ratio = np.abs(gpu_g.astype(np.float64) - inter["g"]) / np.maximum(terms, 1e-300)
        bar = mfma_rel(cfg.h // 128)
        log(f"  gate/up: max |gpu - oracle| / sum|terms| = {ratio.max():.3g} (bar {bar:.3g})")
        assert ratio.max() <= bar
    if wsi["a2"] is not None and tokens is None:
        # tiled path: the requantised codes (sorted-route order) are the
        # oracle's, except where the decision sits on a rounding boundary that
        # the block sums may take either way (then a code within the bracket)
        a2 = np.empty_like(wsi["a2"])
        a2[wsi["sorted"]] = wsi["a2"]
        lo, hi, _ = flagged_codes(L, inter, terms=terms)
        clear = lo == hi
        assert np.array_equal(a2[clear], inter["a2"][clear]), "requantised codes differ"
        T = _T64()
        fl = ~clear
        assert np.all((T[a2[fl]] >= T[lo[fl]]) & (T[a2[fl]] <= T[hi[fl]])), "requantised code outside its bracket"
        log(f"  requantised codes: {int(fl.sum())} of {fl.size} on a rounding boundary")
    allow = flip_allowance(L, inter, terms=terms, w2_dense=L.w2_dense)
    r16_report(f"mxfp4_{cfg.name}_m{cfg.M}_h{cfg.h}_i{cfg.i}_e{cfg.E}_top{k}", got[tok], ref, allow)
    err, mx, cos = check_output(got[tok], ref, allowance=allow)
    log(f"  output: max err {err:.3g} of max|ref| {mx:.3g}, min cosine {cos:.6f}")


@pytest.mark.parametrize("ci", [0, 2])
def test_mxfp4_layer_matches_oracle(moe_mod, ci):
    cfg = synth.CONFIGS[ci]
    _check_layer(moe_mod, _MxLayer(cfg, synth.default_seed(ci)))


@pytest.mark.timeout(600)
def test_mxfp4_wide_decode_shape(moe_mod):
    """The MXFP4 kernel's own shape (h 6144, i 768, E 128, top-4): all 64
    tokens against the oracle."""
    cfg = synth.CONFIGS[3]
    L = _MxLayer(cfg, synth.default_seed(3))
    _check_layer(moe_mod, L)


@pytest.mark.parametrize("M,h,i,E,k", [(1, 128, 128, 1, 1), (300, 256, 128, 4, 2), (7, 640, 384, 16, 5),
                                       (5, 256, 2048, 2, 1), (9, 640, 512, 8, 2), (5, 1536, 384, 8, 3)])
def test_mxfp4_edge_shapes(moe_mod, M, h, i, E, k):
    """One expert and one K block; a batch beyond the one-launch grouping (300
    tokens, several 16-route column blocks per expert); ragged K batches and
    scale rows not 16-byte aligned (h 640); the largest intermediate size
    (i 2048: 16 K blocks in the down GEMM); whole-line weight loads in one of
    the two streaming kernels only (h 640 with i 512: down; h 1536 with i 384:
    gate/up, 12 K blocks, a last batch of 4)."""
    cfg = synth.LayerConfig("mx_edge", M, h, i, E, k, "normal", "test shape")
    _check_layer(moe_mod, _MxLayer(cfg, 91 + M))


@pytest.mark.timeout(600)
def test_mxfp4_tiled_path(moe_mod):
    """A batch on the tiled kernels: 1200 tokens over 8 experts, top-2, so each
    expert holds about 300 routes (two full 128-route tiles and a ragged
    third); h 2048 (8 row tiles of the down GEMM, 16 K blocks of gate/up),
    i 768 (6 column groups, 6 K blocks of the down GEMM)."""
    cfg = synth.LayerConfig("mx_tiled", 1200, 2048, 768, 8, 2, "normal", "test shape")
    assert moe_mod.mxfp4_workspace_layout(cfg.M, cfg.h, cfg.i, cfg.E, cfg.k).path == moe_mod.PATH_PREFILL
    _check_layer(moe_mod, _MxLayer(cfg, 1207))


@pytest.mark.parametrize("M,h,i,E,k", [(300, 256, 128, 4, 2), (1200, 2048, 768, 8, 2), (768, 2048, 768, 128, 8)])
def test_mxfp4_tiled_paths_agree(moe_mod, M, h, i, E, k):
    """The producer with its reducer and the five-launch tiled path give the
    same bits (output, ids, codes, grouping and requantised activations)."""
    cfg = synth.LayerConfig("mx_tiled_pair", M, h, i, E, k, "normal", "test shape")
    L = _MxLayer(cfg, 4321 + M)
    dev = torch.device("cuda:0")
    args = [to_dev_bf16(L.x, dev), torch.from_numpy(np.ascontiguousarray(L.logits)).to(dev)] + \
        [torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (L.q13, L.e13, L.q2, L.e2)]
    got = {}
    for path in (moe_mod.PATH_PREFILL, moe_mod.PATH_PRODUCER):
        ws = moe_mod.alloc_mxfp4_workspace(M, h, i, E, k, device=dev, path=path)
        out = moe_mod.moe_mxfp4_forward_ws_path(*args, k, ws, path)
        torch.cuda.synchronize()
        lay = moe_mod.workspace_layout_path(M, h, i, E, k, path)   # the same offsets for both weight formats
        R = M * k
        got[path] = dict(out=to_host_bits(out), ids=read_ws(ws, lay.topk_ids, R, np.int32),
                         xq=read_ws(ws, lay.xq, M * h, np.uint8), sorted=read_ws(ws, lay.sorted, R, np.int32),
                         a2=read_ws(ws, lay.act2, R * i, np.uint8), a2s=read_ws(ws, lay.act2_scale, R * i // 128,
                                                                                 np.float32).view(np.uint32))
        assert moe_mod.workspace_error(ws) == 0
    a, b = got[moe_mod.PATH_PREFILL], got[moe_mod.PATH_PRODUCER]
    for name in a:
        assert np.array_equal(a[name], b[name]), name


def test_mxfp4_zero_input(moe_mod):
    cfg = synth.CONFIGS[0]
    L = _MxLayer(cfg, synth.default_seed(0))
    L.x = np.zeros_like(L.x)
    got, _ = _run(moe_mod, L)
    assert np.all(got == 0)
