"""GPU parity of the RMSNorm + 1x128 quantisation front end, through the C
ABI, against the oracle: normalised bf16 rows, codes and scales bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import log, to_dev_bf16, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_block_scaled_router_amd as moe
    moe.lib()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def moe_mod(dev):
    import fp8_block_scaled_router_amd as moe
    return moe


def _gamma(h, seed):
    return np.random.default_rng(seed).uniform(0.5, 1.5, h).astype(np.float32)


def _check(moe_mod, dev, xb, gamma, eps, label):
    M, h = xb.shape
    log(f"rmsnorm quant {label}: M={M} h={h} eps={eps}")
    y, q, s = moe_mod.rmsnorm_act_quant(to_dev_bf16(xb, dev), torch.from_numpy(gamma).to(dev), eps)
    _, q2, s2 = moe_mod.rmsnorm_act_quant(to_dev_bf16(xb, dev), torch.from_numpy(gamma).to(dev), eps,
                                          want_y=False)
    torch.cuda.synchronize()
    yr, qr, sr = oracle.rmsnorm_act_quant(xb, gamma, eps)
    yg = to_host_bits(y)
    bad = np.nonzero(yg != yr)
    assert bad[0].size == 0, f"y differs at {list(zip(*bad))[:5]}"
    assert np.array_equal(s.cpu().numpy(), sr)
    assert np.array_equal(q.cpu().numpy(), qr)
    assert torch.equal(q2, q) and torch.equal(s2, s)


@pytest.mark.parametrize("ci", [1, 2, 3, 4, 5])
def test_rmsnorm_quant_layer_shapes(dev, moe_mod, ci):
    cfg = synth.CONFIGS[ci]
    xb = synth.make_x(cfg, synth.default_seed(ci))
    _check(moe_mod, dev, xb, _gamma(cfg.h, ci), 1e-6, cfg.name)


@pytest.mark.parametrize("M,h,eps", [
    (1, 128, 1e-6),        # one group
    (5, 640, 1e-5),        # ragged last 512-column step (one group in it)
    (7, 8192, 1e-6),       # largest h (16 steps)
    (9, 2176, 0.25),       # eps that dominates small rows; ragged step
    (3, 1152, 0.0),        # eps = 0
])
def test_rmsnorm_quant_ragged_and_max(dev, moe_mod, M, h, eps):
    rng = np.random.default_rng(M * 7 + h)
    x = rng.standard_normal((M, h)) * rng.uniform(0.01, 20.0, (M, 1))
    _check(moe_mod, dev, synth.to_bf16_bits(x), _gamma(h, h), eps, "ragged")


def test_rmsnorm_quant_degenerate_rows(dev, moe_mod):
    h = 1024
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, h)).astype(np.float32)
    x[0] = 0.0                          # zero row (eps > 0): y = 0, codes 0, scales 0
    x[1] = -0.0                         # negative zeros
    x[2] = 3.0                          # constant row
    x[3, ::2] *= 1e30                   # huge values: squares only fit in float64
    x[4] *= 1e-35                       # tiny values, some bf16 subnormal
    x[5, 128:256] = 0.0                 # one all-zero group in a live row
    x[6, 7] = 3.0e38                    # one huge element dominates the row
    gamma = _gamma(h, 6)
    gamma[100:140] = 0.0                # zero weights
    gamma[300] = -2.0                   # negative weight
    _check(moe_mod, dev, synth.to_bf16_bits(x), gamma, 1e-6, "degenerate")
