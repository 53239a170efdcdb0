"""The fp8 parity inputs can expose block-scale indexing mistakes (CPU only).

The synthetic 128x128 block scales are amax/448 of N(0, 0.02) blocks, so they
all lie within about 1.5x of each other, and a kernel that read a neighbouring
block's scale would stay inside the fp8 bar of 6e-2. The GPU tests therefore
also run on layers whose block scales are spread by seeded powers of two in
2^-4 .. 2^4 (synth.spread_block_scales). Here, on the CPU, mistakes of that
kind are planted in the oracle's inputs (a scale array shifted by one block,
which is what a mis-indexed read returns) and each must move the layer output
by at least three times the fp8 bar. Block scales are part of the format the
page "MoE-推理部署" (expert-quantisation section) gives for FP8 experts.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import MINI_CONFIGS, make_layer, spread_block_scales

FP8_BAR = 6e-2


def _rel(a, b):
    return float(np.abs(a - b).max() / np.abs(b).max())


@pytest.fixture(scope="module")
def spread_layer():
    cfg = MINI_CONFIGS["mini_fp8_prefill"]
    d = spread_block_scales(make_layer(cfg), seed=2025)
    return cfg, d, oracle.forward(oracle.Layer(d, cfg.k))["Y"]


def _planted(d, **mod):
    d2 = dict(d)
    d2.update(mod)
    return d2


# (name, mutation of the layer's scales): each is what a kernel would see if it
# indexed the scale array wrongly
MISTAKES = {
    "S1 K-block index + 1": lambda d: {"S1": torch.roll(d["S1"], -1, dims=1)},
    "S3 K-block index + 1": lambda d: {"S3": torch.roll(d["S3"], -1, dims=1)},
    "S1 N-block index + 1": lambda d: {"S1": torch.roll(d["S1"], -1, dims=2)},
    "S2 K-block index + 1": lambda d: {"S2": torch.roll(d["S2"], -1, dims=1)},
    "S2 last K-block reads the first": lambda d: {"S2": torch.cat([d["S2"][:, :-1], d["S2"][:, :1]], dim=1)},
    "S2 expert index + 1": lambda d: {"S2": torch.roll(d["S2"], -1, dims=0)},
    "Ss2 K-block index + 1": lambda d: {"Ss2": torch.roll(d["Ss2"], -1, dims=0)},
    "Ss1 read as S1 of expert 0": lambda d: {"Ss1": d["S1"][0].clone()},
}


@pytest.mark.parametrize("name", list(MISTAKES))
def test_scale_mistake_exceeds_bar(spread_layer, name):
    cfg, d, ref = spread_layer
    Y = oracle.forward(oracle.Layer(_planted(d, **MISTAKES[name](d)), cfg.k))["Y"]
    err = _rel(Y, ref)
    assert err >= 3 * FP8_BAR, f"{name}: moves Y by only {err:.3f}"


def test_spread_keeps_codes_and_powers_of_two():
    cfg = MINI_CONFIGS["mini_fp8_decode"]
    d = make_layer(cfg)
    s = spread_block_scales(d, seed=7)
    for key in ("W1", "W3", "W2", "Ws1", "Ws3", "Ws2"):
        assert torch.equal(s[key], d[key])
    spread = []
    for key in ("S1", "S3", "S2", "Ss1", "Ss3", "Ss2"):
        r = (s[key] / d[key]).numpy()
        e = np.log2(r)
        assert np.array_equal(e, np.round(e)) and e.min() >= -4 and e.max() <= 4
        spread.append(e)
    e = np.concatenate([x.ravel() for x in spread])
    assert e.min() == -4 and e.max() == 4  # the whole range is drawn
    # deterministic per seed
    assert torch.equal(spread_block_scales(d, seed=7)["S2"], s["S2"])
