"""Pins for the oracle's individual steps (CPU only).

Each step is checked against something that is not the oracle itself:
brute force (full sorts, recounts), float64 evaluation with a rounding-error
bound, torch's E4M3/bf16 conversions, and closed-form special cases.
Steps follow the routed-MoE stage order of the Netra Kernel README (MoE
prefill pair: routing, gate/up, SiLU and quantisation, down-partial, route
reducer) and the FP32 gate/up / FP8 activation / fp32 activation-scale
intermediates of the Netra compiler architecture page.
"""
import numpy as np
import pytest
import torch

U32 = 2.0 ** -24  # unit roundoff of fp32


def _gamma(n):
    return n * U32 / (1 - n * U32)


def _e4m3_decode64():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _torch_e4m3(v32):
    return torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


# ---------------------------------------------------------------- router

def _router_bruteforce(logits, k):
    """ids by a full stable sort on (-logit, index); weights in float64."""
    M, E = logits.shape
    ids = np.empty((M, k), np.int32)
    w = np.empty((M, k), np.float64)
    for t in range(M):
        l = logits[t].astype(np.float64)
        order = sorted(range(E), key=lambda e: (-l[e], e))
        ids[t] = order[:k]
        p = np.exp(l - l.max())
        p = p / p.sum()
        sel = p[ids[t]]
        w[t] = sel / sel.sum()
    return ids, w


@pytest.mark.parametrize("M,E,k", [(7, 8, 2), (5, 128, 8), (3, 256, 16), (4, 16, 16), (9, 1, 1)])
def test_router_vs_bruteforce(oracle_mod, M, E, k):
    rng = np.random.default_rng(M * 1000 + E)
    logits = rng.standard_normal((M, E)).astype(np.float32)
    ids, w = oracle_mod.router(logits, k)
    ids_ref, w_ref = _router_bruteforce(logits, k)
    assert np.array_equal(ids, ids_ref)
    np.testing.assert_allclose(w, w_ref, rtol=2e-6, atol=1e-7)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -23 + 1e-7)


def test_router_ties_go_to_lower_index(oracle_mod):
    E, k = 16, 4
    logits = np.zeros((3, E), np.float32)
    logits[1, [3, 9, 12]] = 1.0          # three-way tie at the top
    logits[2, :] = -0.0                  # -0 and +0 compare equal
    logits[2, 5] = 0.0
    ids, w = oracle_mod.router(logits, k)
    assert list(ids[0]) == [0, 1, 2, 3]
    assert np.all(w[0] == np.float32(0.25))
    assert list(ids[1]) == [3, 9, 12, 0]
    assert list(ids[2]) == [0, 1, 2, 3]


def test_router_k_equals_E_is_a_full_descending_sort(oracle_mod):
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((6, 12)).astype(np.float32)
    ids, w = oracle_mod.router(logits, 12)
    for t in range(6):
        assert list(ids[t]) == list(np.argsort(-logits[t], kind="stable"))
        # renormalising over all E experts gives back the softmax
        p = np.exp(logits[t].astype(np.float64) - logits[t].max())
        p /= p.sum()
        np.testing.assert_allclose(w[t], p[ids[t]], rtol=3e-6)


# -------------------------------------------------------- activation quant

def test_act_quant_scale_and_codes(oracle_mod, synth_mod):
    rng = np.random.default_rng(7)
    x32 = rng.standard_normal((5, 384)).astype(np.float32)
    x32[1, 128:256] = 0.0                         # an all-zero group
    x32[2, 0:128] *= 1e-3                         # small values, subnormal codes
    x32[3, 5] = -0.0
    xb = synth_mod.to_bf16_bits(x32)
    q, s = oracle_mod.act_quant(xb)
    xf = oracle_mod.bf16_to_f32(xb)
    g = xf.reshape(5, 3, 128)
    amax = np.abs(g).max(-1)
    s_ref = (amax / np.float32(448.0)).astype(np.float32)     # IEEE fp32 division
    assert np.array_equal(s, s_ref)
    # codes: torch's RNE E4M3 of the fp32 quotient (IEEE division)
    with np.errstate(invalid="ignore", divide="ignore"):
        quo = (g / s_ref[..., None]).astype(np.float32)
    ref = _torch_e4m3(quo).reshape(5, 384)
    zero_groups = np.repeat(s_ref == 0, 128, axis=-1).reshape(5, 384)
    ref[zero_groups] = 0
    assert np.array_equal(q, ref)
    assert np.all(q[1, 128:256] == 0) and s[1, 1] == 0.0
    # every group with a nonzero value has a code of magnitude 448 (0x7E / 0xFE)
    qa = (q.reshape(5, 3, 128) & 0x7F)
    for t in range(5):
        for b in range(3):
            if s[t, b] > 0:
                assert qa[t, b].max() == 0x7E


# ---------------------------------------------------------------- grouping

@pytest.mark.parametrize("R,E", [(8, 8), (1, 128), (96, 128), (256, 128), (5000, 16), (0, 4)])
def test_group_vs_recount(oracle_mod, R, E):
    rng = np.random.default_rng(R + E)
    ids = rng.integers(0, E, R).astype(np.int32)
    counts, offsets, srt = oracle_mod.group(ids, E)
    assert np.array_equal(counts, np.bincount(ids, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == R
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(srt, np.argsort(ids, kind="stable"))
    assert np.array_equal(np.sort(srt), np.arange(R))
    for e in range(E):
        seg = srt[offsets[e]:offsets[e + 1]]
        assert np.all(ids[seg] == e) and np.all(np.diff(seg) > 0)


# --------------------------------------------------------- weight quant

def test_weight_block_quant(oracle_mod, synth_mod):
    cfg = synth_mod.CONFIGS[0]
    w = synth_mod.make_w13_f32(cfg, 11, experts=[0, 3])
    w[1, 0:128, 128:256] = 0.0            # an all-zero block
    q, s = oracle_mod.quant_weight_block128(w)
    B, N, K = w.shape
    blocks = w.reshape(B, N // 128, 128, K // 128, 128).transpose(0, 1, 3, 2, 4)
    amax = np.abs(blocks).max(axis=(-1, -2))
    s_ref = (amax / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(s, s_ref)
    with np.errstate(invalid="ignore", divide="ignore"):
        quo = (blocks / s_ref[..., None, None]).astype(np.float32)
    ref = _torch_e4m3(quo)
    ref[np.broadcast_to((s_ref == 0)[..., None, None], ref.shape)] = 0
    ref = ref.transpose(0, 1, 3, 2, 4).reshape(B, N, K)
    assert np.array_equal(q, ref)
    # dequantisation error is at most half a step of the E4M3 grid
    T = _e4m3_decode64()
    deq = T[q].reshape(B, N // 128, 128, K // 128, 128) * s.astype(np.float64)[:, :, None, :, None]
    err = np.abs(deq - w.reshape(deq.shape).astype(np.float64))
    assert np.all(err <= np.abs(w.reshape(deq.shape)) * 2.0 ** -4 + 2.0 ** -10 * s.max() + 1e-12)


# --------------------------------------------------------- block GEMM

@pytest.mark.parametrize("R,N,K", [(3, 128, 128), (5, 256, 384), (2, 128, 1024)])
def test_block_gemm_within_higham_bound(oracle_mod, R, N, K):
    rng = np.random.default_rng(R * N + K)
    A = rng.integers(0, 256, (4, K), dtype=np.uint8)
    A[(A & 0x7F) == 0x7F] = 0x10                     # no NaN codes
    W = rng.integers(0, 256, (3, N, K), dtype=np.uint8)
    W[(W & 0x7F) == 0x7F] = 0x22
    As = rng.uniform(1e-3, 2.0, (4, K // 128)).astype(np.float32)
    Ws = rng.uniform(1e-3, 2.0, (3, N // 128, K // 128)).astype(np.float32)
    arow = rng.integers(0, 4, R).astype(np.int32)
    wsel = rng.integers(0, 3, R).astype(np.int32)
    out = oracle_mod.block_gemm(A, As, arow, W, Ws, wsel)
    T = _e4m3_decode64()
    KB = K // 128
    n_terms = 128 + KB + 2
    for r in range(R):
        a = T[A[arow[r]]].reshape(KB, 128)
        w = T[W[wsel[r]]].reshape(N, KB, 128)
        blk = np.einsum("bk,nbk->nb", a, w)                       # exact in float64
        sc = As[arow[r]].astype(np.float64)[None, :] * \
            np.repeat(Ws[wsel[r]].astype(np.float64), 128, axis=0)  # [N, KB]
        exact = (blk * sc).sum(-1)
        mag = (np.einsum("bk,nbk->nb", np.abs(a), np.abs(w)) * np.abs(sc)).sum(-1)
        assert np.all(np.abs(out[r] - exact) <= _gamma(n_terms) * mag + 1e-30)


def test_block_gemm_single_block_is_exact_dot(oracle_mod):
    """K = 128 with unit scales and small integer codes: the fp32 result must
    equal the integer dot product exactly."""
    K, N = 128, 128
    T = _e4m3_decode64()
    small = [c for c in range(0x38, 0x50) if T[c] == int(T[c])]   # 1.0 .. 15.0 integers
    rng = np.random.default_rng(3)
    A = rng.choice(small, (1, K)).astype(np.uint8)
    W = rng.choice(small, (1, N, K)).astype(np.uint8)
    out = oracle_mod.block_gemm(A, np.ones((1, 1), np.float32), np.zeros(1, np.int32),
                                W, np.ones((1, 1, 1), np.float32), np.zeros(1, np.int32))
    ref = (T[W[0]] * T[A[0]][None, :]).sum(-1)
    assert np.array_equal(out[0].astype(np.float64), ref)


# ---------------------------------------------------------- SiLU-mul-quant

def test_silu_mul_quant(oracle_mod):
    rng = np.random.default_rng(4)
    R, I = 6, 256
    g = (rng.standard_normal((R, 2 * I)) * 3).astype(np.float32)
    g[2, :I] = -200.0      # silu underflows to -0
    g[3] = 0.0             # whole route zero -> zero scale and codes
    a2, a2s = oracle_mod.silu_mul_quant(g)
    gate = g[:, :I].astype(np.float64)
    up = g[:, I:].astype(np.float64)
    v = gate / (1 + np.exp(-gate)) * up
    vb = v.reshape(R, I // 128, 128)
    amax = np.abs(vb).max(-1)
    # scale within 1 ulp of the float64 amax/448 (fp32 silu differs by ulps)
    np.testing.assert_allclose(a2s, amax / 448.0, rtol=1e-6, atol=1e-38)
    assert np.all(a2s[3] == 0) and np.all(a2[3] == 0)
    # dequantised values are within half an E4M3 step (plus fp32 slack)
    T = _e4m3_decode64()
    deq = T[a2].reshape(R, I // 128, 128) * a2s.astype(np.float64)[..., None]
    step = np.maximum(np.abs(vb) * 2.0 ** -3, 2.0 ** -9 * a2s[..., None])
    # (1e-30: fp32 underflow of silu at very negative gate, where float64 is not 0)
    assert np.all(np.abs(deq - vb) <= 0.5 * step * (1 + 1e-4) + 1e-6 * amax[..., None] + 1e-30)


# ------------------------------------------------------------------ combine

def test_combine_vs_float64(oracle_mod):
    rng = np.random.default_rng(6)
    M, k, H = 5, 8, 256
    y = rng.standard_normal((M * k, H)).astype(np.float32)
    w = rng.uniform(0, 1, (M, k)).astype(np.float32)
    w /= w.sum(1, keepdims=True)
    out = oracle_mod.combine(y, w)
    ref = (w.astype(np.float64)[:, :, None] * y.reshape(M, k, H).astype(np.float64)).sum(1)
    got = oracle_mod.bf16_to_f32(out).astype(np.float64)
    # bf16 rounding (half an ulp, 2^-8 relative) plus the fp32 sum's error
    mag = (np.abs(w)[:, :, None] * np.abs(y.reshape(M, k, H))).sum(1)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 * 1.0001 + _gamma(2 * k) * mag)
    # k = 1 with weight 1: combine is the bf16 rounding of y itself
    out1 = oracle_mod.combine(y[:M], np.ones((M, 1), np.float32))
    ref1 = torch.from_numpy(y[:M]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out1, ref1)
