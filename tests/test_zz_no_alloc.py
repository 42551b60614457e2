"""The allocation-free entry point moe_fp8_forward_noalloc (workspace in the
library's fixed per-device array) against moe_fp8_forward_ws on the same
inputs: bitwise equal outputs (the same kernels, deterministic), on two calls
in a row -- the verify batch (12 tokens, the weight-streaming path), then a
smaller one (one token, the one-kernel path) -- a third on the first shape
again, and a size beyond the array rejected with MOE_ERR_WORKSPACE."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import Layer, check_output, log, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe_mod():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_block_scaled_router_amd as moe
    moe.lib()
    return moe


def _pair(moe_mod, L):
    M, h, i, E, k = L.dims
    ws = moe_mod.alloc_workspace(M, h, i, E, k, device=L.dev)
    ref = moe_mod.moe_fp8_forward_ws(L.tx, L.tl, L.t13, L.ts13, L.t2, L.ts2, k, ws)
    out = torch.full_like(ref, float("nan"))
    moe_mod.moe_fp8_forward_noalloc(L.tx, L.tl, L.t13, L.ts13, L.t2, L.ts2, k, out=out)
    torch.cuda.synchronize()
    return to_host_bits(out), to_host_bits(ref)


def test_noalloc_matches_workspace_entry(moe_mod):
    dev = torch.device("cuda:0")
    big = Layer(synth.CONFIGS[2], synth.default_seed(2), dev)          # M = 12, streaming path
    small_cfg = synth.LayerConfig("m1_of_verify", 1, 2048, 768, 128, 8, "normal", "noalloc")
    small = Layer(small_cfg, synth.default_seed(2), dev, x=big.x[3:4], logits=big.logits[3:4],
                  weights=(big.q13, big.s13, big.q2, big.s2))            # M = 1, one-kernel path
    assert moe_mod.workspace_layout(12, 2048, 768, 128, 8).path == moe_mod.PATH_STREAM
    assert moe_mod.workspace_layout(1, 2048, 768, 128, 8).path == moe_mod.PATH_FUSED_DECODE
    for label, L in (("verify M=12", big), ("decode M=1", small), ("verify M=12 again", big)):
        log(f"noalloc {label}")
        got, ref = _pair(moe_mod, L)
        assert np.array_equal(got, ref), f"{label}: allocation-free output differs from the workspace entry's"
        check_output(got, L.oracle())


def test_noalloc_rejects_sizes_beyond_the_array(moe_mod):
    dev = torch.device("cuda:0")
    M, h, i, E, k = 8192, 2048, 768, 128, 8
    assert moe_mod.workspace_bytes(M, h, i, E, k) > moe_mod.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, h), dtype=torch.bfloat16, device=dev)
    lg = torch.zeros((M, E), dtype=torch.float32, device=dev)
    w13 = torch.zeros((E, 2 * i, h), dtype=torch.float8_e4m3fn, device=dev)
    s13 = torch.zeros((E, 2 * i // 128, h // 128), dtype=torch.float32, device=dev)
    w2 = torch.zeros((E, h, i), dtype=torch.float8_e4m3fn, device=dev)
    s2 = torch.zeros((E, h // 128, i // 128), dtype=torch.float32, device=dev)
    with pytest.raises(moe_mod.MoeError) as ex:
        moe_mod.moe_fp8_forward_noalloc(x, lg, w13, s13, w2, s2, k)
    assert ex.value.status == moe_mod.MOE_ERR_WORKSPACE
