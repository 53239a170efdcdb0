"""The synthetic input generator: seeding, storage formats, shapes."""
import numpy as np
import pytest
import torch

import oracle

from synth import CONFIGS, MINI_CONFIGS, make_layer, quantize_e4m3_blocks, redraw_rows
from synth.gen import gate_bias


def _e4m3_grid():
    """All finite non-negative E4M3 values, from the format definition."""
    vals = [m * 2.0 ** -9 for m in range(8)]
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append((1 + m / 8) * 2.0 ** (e - 7))
    return np.array(sorted(set(vals)))


def _rne_brute(x, grid):
    """Nearest grid value, ties to the one with even mantissa (even code)."""
    out = []
    for v in x:
        a = abs(v)
        if a >= 448.0:
            r = 448.0
        else:
            i = np.searchsorted(grid, a)
            lo, hi = grid[max(i - 1, 0)], grid[min(i, len(grid) - 1)]
            if a - lo < hi - a:
                r = lo
            elif hi - a < a - lo:
                r = hi
            else:  # tie: the even code (index parity within the grid)
                r = lo if (np.searchsorted(grid, lo) % 2 == 0) else hi
        out.append(np.copysign(r, v))
    return np.array(out)


def test_e4m3_quantisation_is_rne_with_saturation():
    grid = _e4m3_grid()
    mids = (grid[:-1] + grid[1:]) / 2  # exact ties
    rng = np.random.default_rng(0)
    x = np.concatenate([mids, -mids, rng.normal(size=4000) * 50, [500.0, -1e4, 0.0]])
    x = x[: (x.size // 128) * 128]
    x = np.resize(x, (128, 128 * ((x.size + 16383) // 16384)))
    # with the block amax at exactly 448 the scale is 1 and codes are plain RNE
    x[0, :] = 448.0
    codes, scales = quantize_e4m3_blocks(torch.tensor(x, dtype=torch.float32))
    assert np.all(scales.numpy() == 1.0)
    dec = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = _rne_brute(np.float32(x).astype(np.float64).ravel(), grid).reshape(x.shape)
    np.testing.assert_array_equal(dec, ref)


def test_e4m3_block_scale_is_amax_over_448():
    rng = np.random.default_rng(1)
    w = torch.tensor(rng.normal(size=(256, 384)) * 0.02, dtype=torch.float32)
    codes, scales = quantize_e4m3_blocks(w)
    for bi in range(2):
        for bj in range(3):
            blk = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            assert scales[bi, bj].item() == (blk.abs().max() / 448.0).item()
    dec = codes.view(torch.float8_e4m3fn).to(torch.float32) * scales.repeat_interleave(128, 0).repeat_interleave(128, 1)
    rel = ((dec - w).abs() / w.abs().clamp_min(1e-30)).numpy()
    big = w.abs().numpy() > 2.0 ** -6 * scales.repeat_interleave(128, 0).repeat_interleave(128, 1).numpy()
    assert rel[big].max() <= 2.0 ** -4 + 1e-7  # half an ulp of a 3-bit mantissa


def test_zero_block_gets_unit_scale():
    codes, scales = quantize_e4m3_blocks(torch.zeros(128, 128))
    assert scales.item() == 1.0 and int(codes.sum()) == 0


def test_layer_shapes_and_dtypes():
    for cfg in MINI_CONFIGS.values():
        d = make_layer(cfg)
        assert d["X"].shape == (cfg.T, cfg.H)
        assert d["Wg"].shape == (cfg.H, cfg.E)
        if cfg.w != "mxfp4":
            assert d["W1"].shape == (cfg.E, cfg.H, cfg.F) and d["W2"].shape == (cfg.E, cfg.F, cfg.H)
        if cfg.w == "fp8":
            assert d["W1"].dtype == torch.uint8
            assert d["S1"].shape == (cfg.E, cfg.H // 128, cfg.F // 128)
            assert d["S2"].shape == (cfg.E, cfg.F // 128, cfg.H // 128)
        elif cfg.w == "mxfp4":
            assert d["W1"].dtype == torch.uint8 and d["S1"].dtype == torch.uint8
            assert d["W1"].shape == (cfg.E, cfg.H // 2, cfg.F) and d["W2"].shape == (cfg.E, cfg.F // 2, cfg.H)
            assert d["S1"].shape == (cfg.E, cfg.H // 32, cfg.F) and d["S2"].shape == (cfg.E, cfg.F // 32, cfg.H)
        else:
            assert d["S1"] is None
        assert (d["Ws1"] is not None) == (cfg.Fs > 0)
        if cfg.Fs > 0:
            packed = cfg.shared_w == "mxfp4"
            assert d["Ws1"].shape == (cfg.H // (2 if packed else 1), cfg.Fs)
            assert d["Ws2"].shape == (cfg.Fs // (2 if packed else 1), cfg.H)
            assert (d["Ss1"] is not None) == (cfg.shared_w in ("fp8", "mxfp4"))
            assert d["Ws1"].dtype == (torch.uint8 if cfg.shared_w in ("fp8", "mxfp4") else torch.bfloat16)


def test_bf16_shared_expert_holds_the_same_draws():
    # the bf16 shared expert of a layer is the same draw as its E4M3 form:
    # decoding the codes with their block scales lands within E4M3 rounding
    base = MINI_CONFIGS["mini_fp8_bf16s_decode"]
    d16 = make_layer(base)
    d8 = make_layer(base.with_(ws=""))
    assert torch.equal(d16["W1"], d8["W1"]) and torch.equal(d16["X"], d8["X"])
    codes, scales = d8["Ws1"], d8["Ss1"]
    deq = torch.from_numpy(oracle.dequant_blocks(codes.numpy(), scales.numpy()))
    w16 = d16["Ws1"].double()
    # E4M3 rounding of the fp32 draw (2^-4 relative) plus the bf16 rounding of it
    assert (deq - w16).abs().max() <= (2.0 ** -4 + 2.0 ** -8) * w16.abs().max()


def test_generation_is_deterministic_and_per_expert():
    cfg = MINI_CONFIGS["mini_bf16_wide"]
    a, b = make_layer(cfg), make_layer(cfg)
    for key in ("X", "Wg", "W1", "W2"):
        assert torch.equal(a[key], b[key])
    assert not torch.equal(a["W1"][0], a["W1"][1])
    c = make_layer(cfg.with_(seed=99))
    assert not torch.equal(a["X"], c["X"])


def test_weight_statistics():
    cfg = MINI_CONFIGS["mini_bf16_prefill"]
    d = make_layer(cfg)
    w = d["W1"].float()
    assert abs(w.std().item() - 0.02) < 5e-4 and abs(w.mean().item()) < 5e-4
    x = d["X"].float()
    assert abs(x.std().item() - 1.0) < 0.02


def test_zipf_bias_and_redraw():
    b = gate_bias(CONFIGS["mixtral_prefill"])
    np.testing.assert_allclose(b.numpy(), -1.1 * np.log(np.arange(1, 9)), rtol=1e-6)
    assert gate_bias(CONFIGS["mixtral_decode"]) is None
    cfg = MINI_CONFIGS["mini_bf16_decode"]
    d = make_layer(cfg, experts=False)
    X0 = d["X"].clone()
    redraw_rows(cfg, d["X"], [3, 7], attempt=0)
    changed = (d["X"] != X0).any(dim=1)
    assert changed[3] and changed[7] and changed.sum() == 2


@pytest.mark.parametrize("name", list(CONFIGS))
def test_full_configs_are_well_formed(name):
    cfg = CONFIGS[name]
    assert 1 <= cfg.k <= cfg.E
    if cfg.w == "fp8":
        assert cfg.H % 128 == 0 and cfg.F % 128 == 0 and cfg.Fs % 128 == 0
