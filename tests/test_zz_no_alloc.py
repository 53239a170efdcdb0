"""moe_forward_noalloc (no workspace argument: the library's fixed device
scratch) against moe_forward with a caller workspace, through the C ABI.

Two calls in a row on each layer, the second with fewer tokens, so the second
runs on scratch that still holds the first call's contents; outputs and the
optional routing outputs must equal moe_forward's bit for bit (same kernels,
same plan). A prefill-sized batch whose workspace exceeds the scratch is
refused with MOE_ERR_SCRATCH_LIMIT.
"""
import pytest
import torch

import mixture_experts_layer_count_amd as moe
from mixture_experts_layer_count_amd._lib import MOE_ERR_SCRATCH_LIMIT
from synth import CONFIGS, MINI_CONFIGS
from _gpu import say, screened_layer

pytestmark = pytest.mark.gpu

CASES = ["mini_bf16_decode", "mini_fp8_decode", "mini_fp8_prefill", "mini_bf16_prefill", "mini_mxfp4_shared",
         "mini_fp8_bf16s_decode", "mini_f32", "qwen3_decode", "mixtral_decode"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    moe.lib()


@pytest.mark.parametrize("name", CASES)
def test_noalloc_matches_forward(name):
    cfg = MINI_CONFIGS.get(name) or CONFIGS[name]
    say(f"[noalloc] {name} T={cfg.T}")
    d = screened_layer(cfg)
    layer = moe.MoELayer(d, cfg.k)
    T2 = max(1, cfg.T // 2 - 1)
    inputs = (d["X"], d["X"][:T2].contiguous())
    # two no-alloc calls in a row (the second, smaller, on the first's leftovers)
    got = [layer.forward_noalloc(X, aux=True) for X in inputs]
    ref = [layer.forward(X.clone(), aux=True) for X in inputs]
    torch.cuda.synchronize()
    for X, g1, r1 in zip(inputs, got, ref):
        for g, r, what in zip(g1, r1, ("Y", "logits", "topk_idx", "topk_w", "counts")):
            assert torch.equal(g, r), f"{name} T={X.shape[0]}: {what} differs"
        say(f"    T={X.shape[0]}: equal")


def test_noalloc_refuses_prefill_batch():
    cfg = MINI_CONFIGS["mini_fp8_prefill"]
    d = screened_layer(cfg)
    layer = moe.MoELayer(d, cfg.k)
    assert layer.workspace_bytes(cfg.T) <= moe.lib().moe_forward_noalloc_max_bytes()
    big = cfg.with_(name="noalloc_big", H=7168, F=2048, E=16, T=8192)
    # a descriptor of a large layer (weights never read: refused on the host)
    import ctypes
    from mixture_experts_layer_count_amd import _lib
    desc = _lib.LayerDesc()
    desc.H, desc.F, desc.E, desc.k, desc.Fs = big.H, big.F, big.E, 2, 0
    desc.act_dt, desc.w_dt = _lib.MOE_BF16, _lib.MOE_BF16
    for key in ("Wg", "W1", "W3", "W2"):
        setattr(desc, key, d["X"].data_ptr())
    X = torch.empty((big.T, big.H), dtype=torch.bfloat16, device="cuda")
    st = moe.lib().moe_forward_noalloc(ctypes.byref(desc), X.data_ptr(), big.T, X.data_ptr(), None,
                                       None, None, None, None, None)
    assert st == MOE_ERR_SCRATCH_LIMIT
