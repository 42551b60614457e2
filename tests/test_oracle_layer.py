"""Whole-layer pins for the oracle (CPU only).

An independent float64 evaluation (numpy matmuls on dequantised operands,
torch's E4M3 conversion for the two activation quantisations, quantisation
decisions taken in fp32 as the method does) must agree with the oracle ten
times tighter than the GPU acceptance bar; special cases reduce the layer to
a dense FFN or to zero; symmetries (token permutation, expert relabelling,
token subsets, thread count) must hold bit for bit.

Stage order: Netra Kernel README, MoE prefill pair (routing, gate/up, SiLU
and quantisation, down-partial, separate route reducer); fixed-order sums:
Inferact amd-kernels README, atomics rule.
"""
import numpy as np
import pytest
import torch


def _T64():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _quant_rows_fp32(v32):
    """1x128 quantisation with the decisions in fp32; torch does the E4M3 RNE."""
    R, K = v32.shape
    g = v32.reshape(R, K // 128, 128)
    amax = np.abs(g).max(-1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        quo = (g / s[..., None]).astype(np.float32)
    quo[np.broadcast_to((s == 0)[..., None], quo.shape)] = 0.0
    code = torch.from_numpy(np.ascontiguousarray(quo)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return code.reshape(R, K), s


def brute_force_f64(xb, logits, q13, s13, q2, s2, k):
    T = _T64()
    M, h = xb.shape
    E = logits.shape[1]
    i = q2.shape[2]
    x32 = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).float().numpy()
    l64 = logits.astype(np.float64)
    ids = np.argsort(-l64, axis=1, kind="stable")[:, :k]
    p = np.exp(l64 - l64.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    w = np.take_along_axis(p, ids, 1)
    w /= w.sum(1, keepdims=True)
    xq, xs = _quant_rows_fp32(x32)
    xdq = T[xq] * np.repeat(xs.astype(np.float64), 128, axis=1)
    out = np.zeros((M, h))
    for t in range(M):
        for r in range(k):
            e = ids[t, r]
            W13 = T[q13[e]] * np.repeat(np.repeat(s13[e].astype(np.float64), 128, 0), 128, 1)
            gv = W13 @ xdq[t]
            gate, up = gv[:i], gv[i:]
            v = gate / (1.0 + np.exp(-gate)) * up
            a2, a2s = _quant_rows_fp32(v.astype(np.float32)[None, :])
            adq = T[a2[0]] * np.repeat(a2s[0].astype(np.float64), 128)
            W2 = T[q2[e]] * np.repeat(np.repeat(s2[e].astype(np.float64), 128, 0), 128, 1)
            out[t] += w[t, r] * (W2 @ adq)
    return out, ids


def bf16_ulp(v):
    """ulp of bf16 at |v| (2^(floor(log2|v|) - 7)); smallest normal's ulp at 0."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -126)))
    return 2.0 ** (np.maximum(e, -126) - 7)


def check_close(got_bits, ref, rel, cos_min):
    got = torch.from_numpy(got_bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    mx = np.abs(ref).max()
    if mx == 0:
        assert np.all(got == 0)
        return
    tol = rel * mx + bf16_ulp(ref)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (np.argwhere(bad)[:5], got[bad][:5], ref[bad][:5])
    for t in range(ref.shape[0]):
        a, b = got[t], ref[t]
        na, nb = np.linalg.norm(a), np.linalg.norm(b)
        if na == 0 and nb == 0:
            continue
        assert a @ b / (na * nb) >= cos_min


def _layer(synth_mod, oracle_mod, cfg, seed, M=None):
    x = synth_mod.make_x(cfg, seed, M=M)
    logits = synth_mod.make_logits(cfg, seed, M=M)
    q13, s13 = oracle_mod.quant_weight_block128(synth_mod.make_w13_f32(cfg, seed))
    q2, s2 = oracle_mod.quant_weight_block128(synth_mod.make_w2_f32(cfg, seed))
    return x, logits, q13, s13, q2, s2


def _small_cfg(synth_mod, name, M, h, i, E, k, logits="normal"):
    return synth_mod.LayerConfig(name, M, h, i, E, k, logits, "test shape")


@pytest.mark.parametrize("shape", ["cfg0", "m2_h128_i128_e4_k2", "m3_h384_i256_e6_k3"])
def test_layer_vs_float64_bruteforce(oracle_mod, synth_mod, shape):
    if shape == "cfg0":
        cfg = synth_mod.CONFIGS[0]
    elif shape == "m2_h128_i128_e4_k2":
        cfg = _small_cfg(synth_mod, shape, 2, 128, 128, 4, 2)
    else:
        cfg = _small_cfg(synth_mod, shape, 3, 384, 256, 6, 3)
    x, logits, q13, s13, q2, s2 = _layer(synth_mod, oracle_mod, cfg, 99)
    out, inter = oracle_mod.moe_forward(x, logits, q13, s13, q2, s2, cfg.k, intermediates=True)
    ref, ids = brute_force_f64(x, logits, q13, s13, q2, s2, cfg.k)
    assert np.array_equal(inter["ids"], ids)
    check_close(out, ref, rel=1e-3, cos_min=0.99999)


def test_single_expert_k1_is_dense_ffn(oracle_mod, synth_mod):
    """E = 1, k = 1: routing weight is exactly 1 and the layer is one expert's
    dense quantised FFN, evaluated here without routing or grouping."""
    cfg = _small_cfg(synth_mod, "dense", 5, 256, 256, 1, 1)
    x, logits, q13, s13, q2, s2 = _layer(synth_mod, oracle_mod, cfg, 5)
    out, inter = oracle_mod.moe_forward(x, logits, q13, s13, q2, s2, 1, intermediates=True)
    assert np.all(inter["ids"] == 0) and np.all(inter["topk_w"] == 1.0)
    T = _T64()
    x32 = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().numpy()
    xq, xs = _quant_rows_fp32(x32)
    xdq = T[xq] * np.repeat(xs.astype(np.float64), 128, axis=1)
    W13 = T[q13[0]] * np.repeat(np.repeat(s13[0].astype(np.float64), 128, 0), 128, 1)
    W2 = T[q2[0]] * np.repeat(np.repeat(s2[0].astype(np.float64), 128, 0), 128, 1)
    G = xdq @ W13.T
    V = G[:, :256] / (1 + np.exp(-G[:, :256])) * G[:, 256:]
    a2, a2s = _quant_rows_fp32(V.astype(np.float32))
    A = T[a2] * np.repeat(a2s.astype(np.float64), 128, axis=1)
    ref = A @ W2.T
    check_close(out, ref, rel=1e-3, cos_min=0.99999)


def test_zero_input_gives_exact_zero(oracle_mod, synth_mod):
    cfg = synth_mod.CONFIGS[0]
    x, logits, q13, s13, q2, s2 = _layer(synth_mod, oracle_mod, cfg, 1)
    out = oracle_mod.moe_forward(np.zeros_like(x), logits, q13, s13, q2, s2, cfg.k)
    assert np.all(out == 0)


def test_token_permutation_and_subset(oracle_mod, synth_mod):
    cfg = _small_cfg(synth_mod, "perm", 9, 256, 128, 8, 3)
    x, logits, q13, s13, q2, s2 = _layer(synth_mod, oracle_mod, cfg, 21)
    out = oracle_mod.moe_forward(x, logits, q13, s13, q2, s2, cfg.k)
    perm = np.random.default_rng(0).permutation(cfg.M)
    outp = oracle_mod.moe_forward(x[perm], logits[perm], q13, s13, q2, s2, cfg.k)
    assert np.array_equal(outp, out[perm])
    sub = np.array([7, 2, 5])
    outs = oracle_mod.moe_forward(x[sub], logits[sub], q13, s13, q2, s2, cfg.k)
    assert np.array_equal(outs, out[sub])


def test_expert_relabelling(oracle_mod, synth_mod):
    cfg = _small_cfg(synth_mod, "relabel", 6, 256, 128, 8, 2)
    x, logits, q13, s13, q2, s2 = _layer(synth_mod, oracle_mod, cfg, 33)
    out = oracle_mod.moe_forward(x, logits, q13, s13, q2, s2, cfg.k)
    pi = np.random.default_rng(1).permutation(cfg.E)    # new expert j = old expert pi[j]
    out2 = oracle_mod.moe_forward(x, logits[:, pi], q13[pi], s13[pi], q2[pi], s2[pi], cfg.k)
    assert np.array_equal(out, out2)


def test_thread_count_invariance(oracle_mod, synth_mod):
    cfg = _small_cfg(synth_mod, "threads", 6, 512, 256, 8, 4)
    x, logits, q13, s13, q2, s2 = _layer(synth_mod, oracle_mod, cfg, 44)
    n0 = oracle_mod.get_threads()
    try:
        oracle_mod.set_threads(1)
        a, ia = oracle_mod.moe_forward(x, logits, q13, s13, q2, s2, cfg.k, intermediates=True)
        oracle_mod.set_threads(7)
        b, ib = oracle_mod.moe_forward(x, logits, q13, s13, q2, s2, cfg.k, intermediates=True)
    finally:
        oracle_mod.set_threads(n0)
    assert np.array_equal(a, b)
    for key in ia:
        assert np.array_equal(ia[key], ib[key]), key


def test_routing_weights_sum_to_one(oracle_mod, synth_mod):
    for idx in (1, 2, 4):
        cfg = synth_mod.CONFIGS[idx]
        logits = synth_mod.make_logits(cfg, synth_mod.default_seed(idx), M=min(cfg.M, 256))
        ids, w = oracle_mod.router(logits, cfg.k)
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= cfg.k * 2.0 ** -23)
        assert np.all(w > 0) and np.all(np.diff(w, axis=1) <= 0)   # rank order = descending weight


def test_request_bias_logits_are_per_request(synth_mod):
    """The M=768 verify batch: tokens of one request share their expert bias,
    so within a request the logit differences are those of the N(0,1) base;
    and any token window reproduces the same rows."""
    cfg = synth_mod.CONFIGS[5]
    assert cfg.M == 64 * cfg.request_tokens
    seed = synth_mod.default_seed(5)
    full = synth_mod.make_logits(cfg, seed).astype(np.float64)
    win = synth_mod.make_logits(cfg, seed, M=30, first_token=101)
    assert np.array_equal(win, full[101:131].astype(np.float32))
    base = synth_mod.normal(seed, synth_mod.TAG_LOGITS, (cfg.M, cfg.E), dtype=np.float64)
    bias = full - base
    q = cfg.request_tokens
    per_req = bias.reshape(64, q, cfg.E)
    assert np.allclose(per_req, per_req[:, :1, :], atol=1e-5)       # one bias per request
    assert abs(per_req[:, 0, :].std() - 2.0) < 0.1                   # sd 2
    assert not np.allclose(per_req[0, 0], per_req[1, 0], atol=0.5)  # requests differ
