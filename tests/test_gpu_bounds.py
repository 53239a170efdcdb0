"""GPU: the bounds-checked debug build, libmoe_debug.so (every source built
with -DMOE_BOUNDS_CHECK; include/moe.h, moe_debug_bounds).

On valid inputs no kernel check may fail, on every FFN path of the mini
layers, a full-size prefill layer (256-row tiles, the tail split of the down
projection) and the expert-parallel loopback; and the debug build's results
must equal the release build's bit for bit (the checks add no arithmetic).
A Yp row planted one past the end of combine's input is caught: the check
sets its bit and clamps the row, so the kernel still reads in bounds.
"""
import pytest
import torch

import mixture_experts_layer_count_amd as moe
from mixture_experts_layer_count_amd import _lib
from synth import CONFIGS, MINI_CONFIGS
from _gpu import say, screened_layer

pytestmark = pytest.mark.gpu

FFN_CASES = [(n, p) for n in MINI_CONFIGS for p in ("gemv", "tiled", "tiled_a8")
             if not (p == "tiled" and MINI_CONFIGS[n].w == "f32")
             and not (p == "tiled_a8" and MINI_CONFIGS[n].w != "fp8")]
FULL_CASES = ["qwen3_prefill"]
EP_CASES = [("mini_bf16_prefill", 4), ("mini_fp8_prefill", 8)]


@pytest.fixture(scope="module")
def debug_lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    moe.lib()
    h = _lib.load(_lib.DEBUG_LIB_PATH)
    assert h.moe_debug_bounds() in (0,), "flags left over before any debug launch"
    return h


def _forward(d, k, path):
    Y, logits, idx, w, counts = moe.MoELayer(d, k, path=path).forward(d["X"], aux=True)
    torch.cuda.synchronize()
    return [t.clone() for t in (Y, logits, idx, w, counts)]


def _same(rel, dbg):
    for a, b in zip(rel, dbg):
        assert a.dtype == b.dtype and a.shape == b.shape
        assert torch.equal(a, b)


@pytest.mark.parametrize("name,path", FFN_CASES + [(n, "auto") for n in FULL_CASES])
def test_debug_build_forward(debug_lib, name, path):
    cfg = MINI_CONFIGS.get(name) or CONFIGS[name]
    say(f"[bounds] forward {name} path={path}")
    d = screened_layer(cfg)
    rel = _forward(d, cfg.k, path)
    with _lib.use_library(debug_lib):
        dbg = _forward(d, cfg.k, path)
        flags = debug_lib.moe_debug_bounds()
    assert flags == 0, f"failed bounds checks: {flags:#x}"
    _same(rel, dbg)


@pytest.mark.parametrize("name,G", EP_CASES)
def test_debug_build_ep(debug_lib, name, G):
    cfg = MINI_CONFIGS[name]
    say(f"[bounds] ep {name} G={G}")
    d = screened_layer(cfg)
    Y = moe.EPLoopback(d, cfg.k, G).forward(d["X"]).clone()
    torch.cuda.synchronize()
    with _lib.use_library(debug_lib):
        Yd = moe.EPLoopback(d, cfg.k, G).forward(d["X"]).clone()
        torch.cuda.synchronize()
        flags = debug_lib.moe_debug_bounds()
    assert flags == 0, f"failed bounds checks: {flags:#x}"
    assert torch.equal(Y, Yd)


def test_debug_build_catches_combine_row(debug_lib):
    # combine's Yp holds T*k rows; one assignment names row T*k
    T, k, H = 64, 2, 256
    g = torch.Generator(device="cpu").manual_seed(7)
    Yp = torch.randn(T * k, H, generator=g).to(torch.bfloat16).cuda()
    w = torch.rand(T, k, generator=g).cuda()
    assign_row = torch.randperm(T * k, generator=g).to(torch.int32).cuda()
    assign_row[5] = T * k
    say("[bounds] planted combine row T*k")
    with _lib.use_library(debug_lib):
        debug_lib.moe_debug_bounds()
        Y = moe.combine(Yp, assign_row, w)
        flags = debug_lib.moe_debug_bounds()
    assert flags == _lib.MOE_BOUNDS_COMBINE_ROW
    # the clamped assignment read row 0; every other token is exact
    ar = assign_row.clone()
    ar[5] = 0
    ref = moe.combine(Yp, ar, w)
    torch.cuda.synchronize()
    assert torch.equal(Y, ref)
