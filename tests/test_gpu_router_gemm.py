"""GPU parity of BF16 routing fused with the top-k (C entry
moe_fp8_router_gemm_topk) against the oracle's routing logits and router.

The kernel's products are exact and its sums are fp32 matrix-core
accumulations, while the oracle rounds a float64 sum once, so a GPU logit lies
within rg_rel(h) * sum_j |x_j wr_j| of the oracle's (pinned by
test_router_gemm_logit_accuracy).  The picks are then decided on fp32 logits
on both sides:
  * tokens whose oracle top-(k+1) logits are all more than twice that bound
    apart have a unique answer: ids bit-exact, weights within the bound's
    propagation (each weight's factor exp(+-4 * bound));
  * tokens with a closer pair (flagged) must get a valid answer: distinct ids,
    each pick's oracle logit within twice the bound of the oracle's k-th, and
    the ranks in non-increasing oracle order up to that slack.
With small-integer operands every partial sum is exact, so there the logits,
ids (ties included) and weights must equal the oracle's outright."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import log, to_dev_bf16

pytestmark = pytest.mark.gpu

# Bound on |gpu logit - oracle logit| relative to sum_j |x_j wr_j|.  The
# kernel adds K/32 matrix-core sums of 32 exact products into one fp32
# accumulator per logit.  Taking each matrix-core sum to be as accurate as a
# sequential fp32 sum of its 32 products (<= 32 * 2^-24 of their absolute
# sum) and each accumulation to err by at most 2^-24 of the running sum gives
# (K/32 + 32) * 2^-24 of the absolute sum (5.7e-6 at K = 2048), reached only
# by same-signed terms; random-signed ones cancel and stay far below (about
# 2^-23 measured on the layer shapes).  test_router_gemm_logit_accuracy pins
# it, same-signed rows included.
def rg_rel(K: int) -> float:
    return (K / 32 + 32) * 2.0 ** -24


@pytest.fixture(scope="module")
def moe_mod():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_block_scaled_router_amd as moe
    moe.lib()
    return moe


def _bf16_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _run(moe_mod, xb, wb, k, want_logits=True):
    dev = torch.device("cuda:0")
    lg, ids, w = moe_mod.router_gemm_topk(to_dev_bf16(xb, dev), to_dev_bf16(wb, dev), k, want_logits)
    torch.cuda.synchronize()
    return (lg.cpu().numpy() if lg is not None else None), ids.cpu().numpy(), w.cpu().numpy()


def _abs_sums(xb, wb):
    return np.abs(_bf16_f64(xb)) @ np.abs(_bf16_f64(wb)).T


def _check(moe_mod, xb, wb, k, label):
    M, h = xb.shape
    E = wb.shape[0]
    log(f"router gemm topk {label}: M={M} h={h} E={E} k={k}")
    lg, ids, w = _run(moe_mod, xb, wb, k)
    lr = oracle.router_logits(xb, wb)
    ids_r, w_r = oracle.router(lr, k)
    bound = rg_rel(h) * _abs_sums(xb, wb)
    err = np.abs(lg.astype(np.float64) - lr.astype(np.float64))
    assert np.all(err <= bound), f"logit error {err.max()} above bound at {np.unravel_index(np.argmax(err - bound), err.shape)}"
    # Flag tokens whose top-(k+1) oracle logits hold a pair closer than 2 * bound.
    kk = min(k + 1, E)
    order = np.argsort(-lr.astype(np.float64), axis=1, kind="stable")[:, :kk]
    top = np.take_along_axis(lr.astype(np.float64), order, axis=1)
    bmax = bound.max(axis=1, keepdims=True)
    flagged = np.any(np.diff(top, axis=1) > -2.0 * bmax, axis=1) if kk > 1 else np.zeros(M, bool)
    ok = ~flagged
    log(f"  max logit error {err.max():.3g} (bound {bound.max():.3g}); {int(flagged.sum())} of {M} tokens flagged")
    assert np.array_equal(ids[ok], ids_r[ok]), "ids differ on an unflagged token"
    tol = np.expm1(4.0 * bmax) * w_r + 1e-6
    assert np.all(np.abs(w[ok] - w_r[ok]) <= tol[ok]), "weights outside the propagated bound"
    for t in np.nonzero(flagged)[0]:
        sel = ids[t]
        assert len(set(sel.tolist())) == k and sel.min() >= 0 and sel.max() < E
        slack = 2.0 * bmax[t, 0]
        kth = top[t, k - 1]
        assert np.all(lr[t, sel].astype(np.float64) >= kth - slack)
        assert np.all(np.diff(lr[t, sel].astype(np.float64)) <= slack)
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) <= k * 2.0 ** -22
    # Run-to-run determinism and the logits-free variant.
    lg2, ids2, w2 = _run(moe_mod, xb, wb, k)
    _, ids3, w3 = _run(moe_mod, xb, wb, k, want_logits=False)
    assert np.array_equal(lg2.view(np.uint32), lg.view(np.uint32))
    assert np.array_equal(ids2, ids) and np.array_equal(w2.view(np.uint32), w.view(np.uint32))
    assert np.array_equal(ids3, ids) and np.array_equal(w3.view(np.uint32), w.view(np.uint32))
    return flagged


@pytest.mark.parametrize("ci", [0, 1, 2, 3, 4, 5])
def test_router_gemm_topk_layer_shapes(moe_mod, ci):
    cfg = synth.CONFIGS[ci]
    seed = synth.default_seed(ci)
    flagged = _check(moe_mod, synth.make_x(cfg, seed), synth.make_wr(cfg, seed), cfg.k, cfg.name)
    assert flagged.mean() < 0.05


def test_router_gemm_logit_accuracy(moe_mod):
    """Pin of rg_rel: GPU logits against exact (float64) dot products of the
    same bf16 operands, on rows with a wide spread of magnitudes."""
    rng = np.random.default_rng(11)
    M, h, E = 96, 4096, 64
    x = rng.standard_normal((M, h)) * np.exp(rng.uniform(-3, 3, (M, 1)))
    wr = rng.standard_normal((E, h)) / np.sqrt(h)
    x[: M // 4] = np.abs(x[: M // 4])          # same-signed terms: no cancellation
    wr[: E // 4] = np.abs(wr[: E // 4])
    xb, wb = synth.to_bf16_bits(x), synth.to_bf16_bits(wr)
    lg, _, _ = _run(moe_mod, xb, wb, 4)
    exact = _bf16_f64(xb) @ _bf16_f64(wb).T
    ratio = np.abs(lg - exact) / _abs_sums(xb, wb)
    log(f"router gemm: max |gpu - exact| / sum|x wr| = {ratio.max():.3g} (bar {rg_rel(h):.3g})")
    assert ratio.max() <= rg_rel(h)


@pytest.mark.parametrize("M,h,E,k", [
    (1, 128, 1, 1),        # one expert, one K step, one token
    (37, 384, 200, 5),     # ragged token tile (32 + 5), ragged last x chunk, E not a multiple of 16
    (33, 256, 256, 16),    # largest E and k
    (70, 16384, 128, 8),   # largest h
    (5, 1152, 8, 8),       # k = E
    (64, 2048, 24, 3),     # two full token tiles, E of 1.5 fragments
])
def test_router_gemm_topk_edge_shapes(moe_mod, M, h, E, k):
    rng = np.random.default_rng(M * 1000 + E)
    xb = synth.to_bf16_bits(rng.standard_normal((M, h)))
    wb = synth.to_bf16_bits(rng.standard_normal((E, h)) / np.sqrt(h))
    _check(moe_mod, xb, wb, k, "edge")


@pytest.mark.parametrize("M,h,E,k", [(40, 256, 128, 8), (9, 512, 256, 16), (3, 128, 8, 8)])
def test_router_gemm_topk_exact_integers_and_ties(moe_mod, M, h, E, k):
    """Small-integer operands (|x| <= 3, |wr| <= 2, h <= 512): every partial
    sum is an integer far below 2^24, so the GPU logits are exact and equal the
    oracle's bit for bit, and the many equal logits exercise the tie rule
    (lower expert first) through the fused path.  Duplicated router rows and a
    zero token add exact ties of every rank."""
    rng = np.random.default_rng(M + h + E)
    x = rng.integers(-3, 4, (M, h)).astype(np.float64)
    wr = rng.integers(-2, 3, (E, h)).astype(np.float64)
    wr[E // 2:E // 2 + 3] = wr[1]
    x[0] = 0.0
    xb, wb = synth.to_bf16_bits(x), synth.to_bf16_bits(wr)
    lg, ids, w = _run(moe_mod, xb, wb, k)
    lr = oracle.router_logits(xb, wb)
    ids_r, w_r = oracle.router(lr, k)
    assert np.array_equal(lg, lr)
    assert np.array_equal(ids, ids_r)
    assert np.allclose(w, w_r, rtol=0, atol=1e-6)


def test_router_gemm_topk_empty(moe_mod):
    dev = torch.device("cuda:0")
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
    wr = torch.zeros((8, 256), dtype=torch.bfloat16, device=dev)
    lg, ids, w = moe_mod.router_gemm_topk(x, wr, 2)
    torch.cuda.synchronize()
    assert lg.shape == (0, 8) and ids.shape == (0, 2) and w.shape == (0, 2)


def test_router_gemm_split_and_fused_paths_agree(moe_mod):
    """Few tokens with logits kept take the expert-split kernel plus the row
    router; many tokens (or no logits) take the fused kernel.  Both sum each
    logit in the same order, so the same rows give the same bits either way."""
    rng = np.random.default_rng(23)
    h, E, k = 1280, 200, 6
    xb = synth.to_bf16_bits(rng.standard_normal((4160, h)))
    wb = synth.to_bf16_bits(rng.standard_normal((E, h)) / np.sqrt(h))
    lg_big, ids_big, w_big = _run(moe_mod, xb, wb, k)                 # 130 tiles: fused
    for rows in (1, 33, 100):
        lg, ids, w = _run(moe_mod, xb[:rows], wb, k)                  # split + row router
        _, ids_f, w_f = _run(moe_mod, xb[:rows], wb, k, want_logits=False)   # fused
        assert np.array_equal(lg.view(np.uint32), lg_big[:rows].view(np.uint32))
        assert np.array_equal(ids, ids_big[:rows]) and np.array_equal(ids_f, ids)
        assert np.array_equal(w.view(np.uint32), w_big[:rows].view(np.uint32))
        assert np.array_equal(w_f.view(np.uint32), w.view(np.uint32))
