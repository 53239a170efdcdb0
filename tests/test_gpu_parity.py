"""GPU parity: libmoe (through its C ABI) against the fp64 oracle.

Bars: routing (top-k indices), counts, offsets, permutation and inverse map
bit-exact given the same fp32 logits; layer outputs within the max relative
error max|Y - Y_ref| / max|Y_ref| of 2e-2 (bf16), 6e-2 (fp8 weights) and 1e-4
(f32). Inputs are seeded, with top-k logit gaps of at least 1e-3.
"""
import os

import numpy as np
import pytest
import torch

import mixture_experts_layer_count_amd as moe
import oracle
from synth import CONFIGS, MINI_CONFIGS, LayerConfig
from synth.worked import load_fixture, worked_example_layer
from _gpu import TOL, cover_tokens, rel_err, say, screened_layer, tol_for

TOL_BF16 = TOL["bf16"]

# host threads for the oracle's per-expert work (model-sized layers)
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    moe.lib()  # the HIP library must load: no fallback exists


def _to_dev_i32(a):
    return torch.as_tensor(np.asarray(a), dtype=torch.int32).cuda()


def _check_routing(cfg, d, logits, idx, w):
    L64 = oracle.router_logits(d["X"], d["Wg"], d.get("gate_bias"))
    lg = logits.cpu().numpy()
    assert rel_err(lg, L64) < 1e-5
    idx_np = idx.cpu().numpy()
    np.testing.assert_array_equal(idx_np, oracle.select_topk(lg, cfg.k))   # same fp32 decision
    np.testing.assert_array_equal(idx_np, oracle.select_topk(L64, cfg.k))  # = exact decision
    np.testing.assert_allclose(w.cpu().numpy(), oracle.routing_weights(lg.astype(np.float64), idx_np),
                               rtol=0, atol=2e-6)
    return idx_np


# ----------------------------------------------------------------------------
# route
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(MINI_CONFIGS))
def test_route(name):
    cfg = MINI_CONFIGS[name]
    say(f"[route] {name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k}")
    d = screened_layer(cfg, experts=False)
    logits, idx, w = moe.route(d["X"], d["Wg"], cfg.k, d["gate_bias"])
    torch.cuda.synchronize()
    _check_routing(cfg, d, logits, idx, w)


def test_route_worked_example():
    fx = load_fixture()
    say("[route] worked example (H padded to 32)")
    d = worked_example_layer(F=32, H=32, device="cuda")
    logits, idx, w = moe.route(d["X"], d["Wg"], fx["k"])
    torch.cuda.synchronize()
    exp_idx = [[e - 1 for e, _ in sorted(p, key=lambda q: (-q[1], q[0]))] for p in fx["choices"]]
    exp_w = [[v for _, v in sorted(p, key=lambda q: (-q[1], q[0]))] for p in fx["choices"]]
    np.testing.assert_array_equal(idx.cpu().numpy(), exp_idx)
    np.testing.assert_allclose(w.cpu().numpy(), exp_w, atol=1e-6)


@pytest.mark.parametrize("T,E,k,H", [
    (1, 4, 1, 256), (33, 8, 8, 256), (70, 256, 8, 256), (5, 1024, 64, 256), (129, 64, 1, 256),
    # 512 tokens and more: the tiled router GEMM (128-row tiles, split over H),
    # with ragged rows, fewer experts than one 256-column tile, and K splits
    (600, 64, 4, 1024), (777, 40, 2, 512), (1100, 256, 8, 2048), (4096, 16, 2, 256),
    # and fewer than 16 experts, where the row-streaming router runs at any
    # token count (wide and narrow gates, ragged token counts)
    (514, 8, 2, 4096), (1030, 12, 3, 800), (701, 4, 1, 224),
])
def test_route_shapes(T, E, k, H):
    cfg = LayerConfig(f"route_{T}_{E}_{k}_{H}", T=T, H=H, F=32, E=E, k=k, w_std=0.2, seed=T + E)
    say(f"[route] T={T} E={E} k={k} H={H}")
    d = screened_layer(cfg, experts=False)
    logits, idx, w = moe.route(d["X"], d["Wg"], k)
    torch.cuda.synchronize()
    _check_routing(cfg, d, logits, idx, w)
    np.testing.assert_allclose(w.sum(dim=1).cpu().numpy(), 1.0, atol=1e-6)


def test_route_exact_ties():
    """Equal scores go to the lower expert index. Zero token rows (padding
    tokens) give all-equal logits: the k lowest experts, each with weight
    1/k. Duplicated gate columns give pairs of equal logits: the lower index
    of a pair comes first wherever both are chosen. The row-streaming router
    (few tokens, or fewer than 16 experts) and the tiled one (512 tokens and
    more) run."""
    for T, E in ((200, 64), (600, 64), (600, 8)):
        cfg = LayerConfig(f"ties_{T}_{E}", T=T, H=256, F=32, E=E, k=6, seed=90 + T + E)
        say(f"[route] exact ties T={T} E={E}")
        d = screened_layer(cfg, experts=False)
        X = d["X"].clone()
        X[::3] = 0.0                                  # every third token is padding
        Wg = d["Wg"].clone()
        # same slice, next column, other slices (few experts: adjacent and apart)
        pairs = [(3, 40), (10, 11), (17, 63), (0, 32)] if E == 64 else [(1, 2), (0, 6)]
        for a, b in pairs:
            Wg[:, b] = Wg[:, a]
        logits, idx, w = moe.route(X, Wg, cfg.k)
        torch.cuda.synchronize()
        lg, ix, wt = logits.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
        for a, b in pairs:
            assert np.array_equal(lg[:, a], lg[:, b])  # the tie is exact in the GPU's fp32 logits
        np.testing.assert_array_equal(ix, oracle.select_topk(lg, cfg.k))
        zero = np.arange(0, T, 3)
        assert (lg[zero] == 0.0).all()
        np.testing.assert_array_equal(ix[zero], np.tile(np.arange(cfg.k), (zero.size, 1)))
        np.testing.assert_allclose(wt[zero], 1.0 / cfg.k, rtol=0, atol=1e-7)
        both = 0
        for a, b in pairs:
            for t in range(T):
                row = list(ix[t])
                if a in row and b in row:
                    assert row.index(a) == row.index(b) - 1  # adjacent, lower index first
                    both += 1
        assert both > 0
        np.testing.assert_allclose(wt, oracle.routing_weights(lg.astype(np.float64), ix), rtol=0, atol=2e-6)


# ----------------------------------------------------------------------------
# permute
# ----------------------------------------------------------------------------

def _idx(T, k, E, mode, seed):
    rng = np.random.default_rng(seed)
    if mode == "one":  # every token picks the same k experts
        return np.tile(np.arange(k)[::-1] + 1, (T, 1)) % E
    if mode == "zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        return np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)])
    return np.argsort(rng.random((T, E)), axis=1)[:, :k]


@pytest.mark.parametrize("T,k,E,mode", [
    (1, 1, 4, "rand"), (13, 2, 8, "rand"), (5, 4, 4, "rand"), (600, 2, 8, "zipf"), (1000, 8, 128, "rand"),
    (8192, 8, 128, "rand"), (4096, 8, 256, "rand"), (3000, 2, 8, "zipf"), (777, 4, 16, "one"),
    (1025, 3, 1024, "rand"), (64, 8, 256, "rand"),
])
def test_permute(T, k, E, mode):
    say(f"[permute] T={T} k={k} E={E} {mode}")
    idx = _idx(T, k, E, mode, T * 31 + E)
    X = torch.randn((T, 64), device="cuda").to(torch.bfloat16)
    counts, offsets, row_src, assign_row, Xp = moe.permute(_to_dev_i32(idx), E, X)
    torch.cuda.synchronize()
    rc, ro, rr, ra = oracle.permute(idx, E)
    np.testing.assert_array_equal(counts.cpu().numpy(), rc)
    np.testing.assert_array_equal(offsets.cpu().numpy(), ro)
    np.testing.assert_array_equal(row_src.cpu().numpy(), rr)
    np.testing.assert_array_equal(assign_row.cpu().numpy(), ra)
    assert torch.equal(Xp, X[torch.as_tensor(rr // k, device="cuda")])
    again = moe.permute(_to_dev_i32(idx), E)
    torch.cuda.synchronize()
    for a, b in zip((counts, offsets, row_src, assign_row), again[:4]):
        assert torch.equal(a, b)


# ----------------------------------------------------------------------------
# grouped FFN and combine
# ----------------------------------------------------------------------------

FFN_CASES = [(n, p) for n in MINI_CONFIGS for p in ("gemv", "tiled", "tiled_a8")
             if not (p == "tiled" and MINI_CONFIGS[n].w == "f32")
             and not (p == "tiled_a8" and MINI_CONFIGS[n].w != "fp8")]
# W8A8 against the oracle's mirror of the activation quantisation. The two
# agree except where an h value lands on the other side of an E4M3 rounding
# boundary (fp32 accumulation here, fp64 there): such a flip moves one h
# element by a whole E4M3 step, so single outputs can move by ~1e-2 of the
# output scale while the mean stays near the accumulation noise. The mean
# absolute difference over max |ref| is checked; the max is checked against
# the exact layer (tol_for).
MIRROR_TOL = 1e-3


def mean_rel(got, ref) -> float:
    got = got.detach().float().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(got.astype(np.float64) - ref).mean() / max(np.abs(ref).max(), 1e-300))


@pytest.mark.parametrize("name,path", FFN_CASES)
def test_grouped_ffn(name, path):
    cfg = MINI_CONFIGS[name]
    say(f"[ffn] {name} path={path}")
    d = screened_layer(cfg)
    L = oracle.Layer(d, cfg.k)
    _, idx, _ = oracle.route(L.X(), L.Wg(), L.gate_bias(), cfg.k)
    counts, offsets, row_src, assign_row = oracle.permute(idx, cfg.E)
    Xp = L.X()[row_src // cfg.k]
    ref = oracle.grouped_ffn(Xp, offsets, L.expert)
    off_d, rs_d = _to_dev_i32(offsets), _to_dev_i32(row_src)
    # gather fused into the loads
    Yp = moe.grouped_ffn(d["X"], off_d, d["W1"], d["W3"], d["W2"], d["S1"], d["S3"], d["S2"],
                         row_src=rs_d, k=cfg.k, path=path)
    # pre-permuted rows
    Xp_d = d["X"][torch.as_tensor(row_src // cfg.k, device="cuda")].contiguous()
    Yp2 = moe.grouped_ffn(Xp_d, off_d, d["W1"], d["W3"], d["W2"], d["S1"], d["S3"], d["S2"], path=path)
    torch.cuda.synchronize()
    tol = tol_for(cfg)
    err = rel_err(Yp, ref)
    say(f"    max rel err {err:.3e} (tol {tol})")
    assert err <= tol
    assert torch.equal(Yp, Yp2)
    if path == "tiled_a8":
        mirror = oracle.grouped_ffn(Xp, offsets, L.expert, act_quant=True)
        err_m = mean_rel(Yp, mirror)
        say(f"    against the quantisation mirror: mean {err_m:.3e} (tol {MIRROR_TOL})")
        assert err_m <= MIRROR_TOL



@pytest.mark.parametrize("name", ["mini_mxfp4_decode", "mini_mxfp4_shared"])
def test_mxfp4_every_code(name):
    """Every E2M1 code in both nibbles (uniform random bytes: +-0, subnormal
    +-0.5, up to +-6) and E8M0 scales spread over 2^-9 .. 2^7, so a wrong
    nibble order, sign or scale exponent in the kernel's decode shows."""
    cfg = MINI_CONFIGS[name]
    say(f"[mxfp4 codes] {name}")
    d = screened_layer(cfg)
    rng = np.random.default_rng(2024)
    for key in ("W1", "W3", "W2", "Ws1", "Ws3", "Ws2"):
        if d.get(key) is None:
            continue
        w = d[key]
        d[key] = torch.as_tensor(rng.integers(0, 256, size=tuple(w.shape), dtype=np.uint8), device="cuda")
        skey = "S" + key[1:]
        sc = d[skey]
        d[skey] = torch.as_tensor(rng.integers(118, 135, size=tuple(sc.shape), dtype=np.uint8), device="cuda")
    codes = d["W1"].cpu().numpy()
    assert len(np.unique(codes & 15)) == 16 and len(np.unique(codes >> 4)) == 16
    L = oracle.Layer(d, cfg.k)
    _, idx, _ = oracle.route(L.X(), L.Wg(), L.gate_bias(), cfg.k)
    counts, offsets, row_src, _ = oracle.permute(idx, cfg.E)
    ref = oracle.grouped_ffn(L.X()[row_src // cfg.k], offsets, L.expert)
    # row-streaming decode in registers, and the bf16 decode pass feeding the tiled kernels
    for path in ("gemv", "tiled"):
        Yp = moe.grouped_ffn(d["X"], _to_dev_i32(offsets), d["W1"], d["W3"], d["W2"], d["S1"], d["S3"], d["S2"],
                             row_src=_to_dev_i32(row_src), k=cfg.k, path=path)
        torch.cuda.synchronize()
        err = rel_err(Yp, ref)
        say(f"    grouped FFN ({path}) max rel err {err:.3e} (tol {tol_for(cfg)})")
        assert err <= tol_for(cfg)
        _check_forward(cfg, d, moe.MoELayer(d, cfg.k, path=path))

# fp8 block scales spread by seeded powers of two (2^-4 .. 2^4): with the
# synthetic scales alone (all within about 1.5x of each other) a kernel that
# read a neighbouring block's scale would stay inside the fp8 bar; with the
# spread it moves the output far beyond it (shown on the CPU in
# test_scale_spread.py). Routed experts through moe_grouped_ffn, then the whole
# layer with its shared expert, on every path.
SPREAD_CASES = [(n, p) for n in ("mini_fp8_decode", "mini_fp8_prefill", "mini_fp8_wide", "mini_fp8_bf16s_prefill")
                for p in ("gemv", "tiled", "tiled_a8")]


@pytest.mark.parametrize("name,path", SPREAD_CASES)
def test_fp8_block_scales_spread(name, path):
    from synth import spread_block_scales
    cfg = MINI_CONFIGS[name]
    say(f"[fp8 spread scales] {name} path={path}")
    d = spread_block_scales(screened_layer(cfg), seed=cfg.seed + 2025)
    L = oracle.Layer(d, cfg.k)
    _, idx, _ = oracle.route(L.X(), L.Wg(), L.gate_bias(), cfg.k)
    counts, offsets, row_src, _ = oracle.permute(idx, cfg.E)
    ref = oracle.grouped_ffn(L.X()[row_src // cfg.k], offsets, L.expert)
    Yp = moe.grouped_ffn(d["X"], _to_dev_i32(offsets), d["W1"], d["W3"], d["W2"], d["S1"], d["S3"], d["S2"],
                         row_src=_to_dev_i32(row_src), k=cfg.k, path=path)
    torch.cuda.synchronize()
    err = rel_err(Yp, ref)
    say(f"    grouped FFN max rel err {err:.3e} (tol {tol_for(cfg)})")
    assert err <= tol_for(cfg)
    _check_forward(cfg, d, moe.MoELayer(d, cfg.k, path=path), mirror=path == "tiled_a8")


def _mx_layer_extremes(cfg, d):
    """E8M0 extremes in one layer: a K block of W1 and W3 with scale code 254
    (2^127; its E2M1 codes limited to magnitudes <= 1.5 so the decoded bf16
    weights stay finite) facing token values scaled by 2^-124, and a K block
    with scale code 0 (2^-127) facing token values scaled by 2^126 (so that
    block's products are of order 1, and decoding 2^-127 as zero would show);
    W2 has a block of code 0 too."""
    g = torch.Generator(device="cpu").manual_seed(cfg.seed + 4242)
    hi, lo = 3, 5  # K blocks (32 rows each) of H
    X = d["X"].float().cpu()
    mag = X.abs().clamp(0.25, 1.9) * torch.where(X < 0, -1.0, 1.0)
    X[:, 32 * hi:32 * hi + 32] = mag[:, 32 * hi:32 * hi + 32] * 2.0 ** -124
    X[:, 32 * lo:32 * lo + 32] = mag[:, 32 * lo:32 * lo + 32] * 2.0 ** 126
    d = dict(d)
    d["X"] = X.to(torch.bfloat16).cuda()
    for key in ("W1", "W3"):
        W = d[key].clone()
        S = d["S" + key[1:]].clone()
        rows = slice(16 * hi, 16 * hi + 16)  # byte rows of K block hi
        codes = torch.randint(0, 256, tuple(W[:, rows].shape), generator=g, dtype=torch.uint8).cuda()
        W[:, rows] = codes & 0xBB  # both nibbles: sign kept, magnitude index <= 3 (0, 0.5, 1, 1.5)
        S[:, hi] = 254
        S[:, lo] = 0
        d[key], d["S" + key[1:]] = W, S
    S2 = d["S2"].clone()
    S2[:, 2] = 0
    d["S2"] = S2
    return d


@pytest.mark.parametrize("path", ["gemv", "tiled"])
def test_mxfp4_scale_extremes(path):
    cfg = MINI_CONFIGS["mini_mxfp4_decode"]
    say(f"[mxfp4 E8M0 extremes] path={path}")
    d = _mx_layer_extremes(cfg, screened_layer(cfg))
    L = oracle.Layer(d, cfg.k)
    _, idx, _ = oracle.route(L.X(), L.Wg(), L.gate_bias(), cfg.k)
    counts, offsets, row_src, _ = oracle.permute(idx, cfg.E)
    Xp = L.X()[row_src // cfg.k]
    ref = oracle.grouped_ffn(Xp, offsets, L.expert)
    # the code-0 block alone moves the output well beyond the bar
    d0 = dict(d)
    d0["X"] = d["X"].clone()
    d0["X"][:, 160:192] = 0
    ref0 = oracle.grouped_ffn(oracle.Layer(d0, cfg.k).X()[row_src // cfg.k], offsets, L.expert)
    assert rel_err(ref0, ref) > 5 * TOL_BF16
    Yp = moe.grouped_ffn(d["X"], _to_dev_i32(offsets), d["W1"], d["W3"], d["W2"], d["S1"], d["S3"], d["S2"],
                         row_src=_to_dev_i32(row_src), k=cfg.k, path=path)
    torch.cuda.synchronize()
    err = rel_err(Yp, ref)
    say(f"    max rel err {err:.3e} (tol {TOL_BF16})")
    assert torch.isfinite(Yp.float()).all()
    assert err <= TOL_BF16


@pytest.mark.parametrize("path", ["gemv", "tiled"])
def test_mxfp4_nan_scale(path):
    """E8M0 code 255 is NaN: the outputs that depend on it are not finite,
    and every other output is unchanged."""
    cfg = MINI_CONFIGS["mini_mxfp4_decode"]
    say(f"[mxfp4 E8M0 NaN] path={path}")
    d = dict(screened_layer(cfg))
    S1 = d["S1"].clone()
    S1[2, 4, 7] = 255  # expert 2, K block 4, column 7 of W1
    d["S1"] = S1
    L = oracle.Layer(d, cfg.k)
    _, idx, _ = oracle.route(L.X(), L.Wg(), L.gate_bias(), cfg.k)
    counts, offsets, row_src, _ = oracle.permute(idx, cfg.E)
    ref = oracle.grouped_ffn(L.X()[row_src // cfg.k], offsets, L.expert)
    assert counts[2] > 0
    Yp = moe.grouped_ffn(d["X"], _to_dev_i32(offsets), d["W1"], d["W3"], d["W2"], d["S1"], d["S3"], d["S2"],
                         row_src=_to_dev_i32(row_src), k=cfg.k, path=path)
    torch.cuda.synchronize()
    got = Yp.float().cpu().numpy()
    bad = ~np.isfinite(ref)
    assert bad[offsets[2]:offsets[3]].all() and not bad[:offsets[2]].any() and not bad[offsets[3]:].any()
    np.testing.assert_array_equal(~np.isfinite(got), bad)
    assert rel_err(got[~bad.any(axis=1)], ref[~bad.any(axis=1)]) <= TOL_BF16


# Group sizes on both sides of every tile height (128, 160, 256 rows), with
# empty groups; the rows are pre-permuted token rows drawn by the generator.
EDGE_SIZES = {
    "mini_fp8_prefill": [0, 1, 159, 160, 161, 0, 320, 7, 128, 129, 255, 256, 257, 0, 33, 2],
    "mini_bf16_prefill": [1, 255, 256, 257, 0, 513, 129, 127],  # 1538 rows: 256-row tiles
    "mini_fp8_wide": [0, 1, 159, 160, 161, 0, 320, 7, 128, 129, 255, 256, 257, 0, 33, 2],
    "mini_mxfp4_prefill": [1, 255, 256, 257, 0, 513, 129, 127],  # 1538 rows: 256-row tiles
    "mini_mxfp4_shared": [0, 1, 127, 128, 129, 0, 40, 7, 3, 64, 2, 0, 33, 2, 5, 1],  # 128-row tiles
}
EDGE_CASES = [("mini_fp8_prefill", "tiled_a8"), ("mini_fp8_wide", "tiled_a8"), ("mini_fp8_prefill", "tiled"),
              ("mini_fp8_prefill", "gemv"),
              ("mini_bf16_prefill", "tiled"), ("mini_bf16_prefill", "gemv"),
              ("mini_mxfp4_prefill", "tiled"), ("mini_mxfp4_shared", "tiled"), ("mini_mxfp4_prefill", "gemv")]


@pytest.mark.parametrize("name,path", EDGE_CASES)
def test_grouped_ffn_tile_edges(name, path):
    import dataclasses
    from synth import make_layer
    cfg = MINI_CONFIGS[name]
    sizes = EDGE_SIZES[name]
    assert len(sizes) == cfg.E
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(offsets[-1])
    say(f"[ffn edges] {name} path={path} sizes={sizes}")
    d = screened_layer(cfg)
    if cfg.w == "fp8":  # block scales spread, so scale indexing at the tile edges shows
        from synth import spread_block_scales
        d = spread_block_scales(d, seed=cfg.seed + 77)
    L = oracle.Layer(d, cfg.k)
    Xp = make_layer(dataclasses.replace(cfg, name=cfg.name + "_edges", T=M), device="cuda", experts=False)["X"]
    Yp = moe.grouped_ffn(Xp, _to_dev_i32(offsets), d["W1"], d["W3"], d["W2"], d["S1"], d["S3"], d["S2"], path=path)
    torch.cuda.synchronize()
    Xp64 = oracle.to_f64(Xp)
    ref = oracle.grouped_ffn(Xp64, offsets, L.expert)
    tol = tol_for(cfg)
    err = rel_err(Yp, ref)
    say(f"    max rel err {err:.3e} (tol {tol})")
    assert err <= tol
    if path == "tiled_a8":
        err_m = mean_rel(Yp, oracle.grouped_ffn(Xp64, offsets, L.expert, act_quant=True))
        say(f"    against the quantisation mirror: mean {err_m:.3e} (tol {MIRROR_TOL})")
        assert err_m <= MIRROR_TOL


@pytest.mark.parametrize("R,C,gather", [(1, 128, False), (37, 384, False), (300, 7168, False),
                                         (520, 512, True)])
def test_quantize_rows(R, C, gather):
    say(f"[quant] R={R} C={C} gather={gather}")
    g = torch.Generator(device="cpu").manual_seed(R * 7 + C)
    T = R // 4 if gather else R
    X = torch.randn((max(T, 1), C), generator=g).to(torch.bfloat16)
    if C >= 256:
        X[0, 128:256] = 0.0                      # an all-zero group: scale 1, codes 0
        X[-1, :128] *= 1000.0                    # large values: scale follows amax
    Xd = X.cuda()
    row_src = None
    if gather:
        rs = torch.randperm(R, generator=g).to(torch.int32) % (4 * T)
        row_src = rs.cuda()
        Q, S = moe.quantize_e4m3_rows(Xd, row_src, k=4)
        rows = X[(rs // 4).long()]
    else:
        Q, S = moe.quantize_e4m3_rows(Xd)
        rows = X
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows_e4m3(rows)
    np.testing.assert_array_equal(S.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(Q.cpu().numpy(), q_ref)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("k,H", [(4, 1024), (10, 100), (1, 8)])
def test_combine(dtype, shared, k, H):
    # (10, 100): more than 8 contributions a token (two batches, the second
    # partial) and a row width that is not a multiple of 8 (4 columns a thread)
    T = 300
    say(f"[combine] {dtype} shared={shared} k={k} H={H}")
    rng = np.random.default_rng(7)
    idx = np.argsort(rng.random((T, 16)), axis=1)[:, :k]
    _, _, _, assign_row = oracle.permute(idx, 16)
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    Yp = torch.randn((T * k, H), device="cuda").to(dtype)
    S = torch.randn((T, H), device="cuda").to(dtype) if shared else None
    Y = moe.combine(Yp, _to_dev_i32(assign_row), torch.as_tensor(w).cuda(), S)
    torch.cuda.synchronize()
    ref = oracle.combine(oracle.to_f64(Yp), assign_row, w.astype(np.float64), T, k,
                         None if S is None else oracle.to_f64(S))
    assert rel_err(Y, ref) <= (1e-6 if dtype == torch.float32 else 4e-3)


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------

def _check_forward(cfg, d, layer, tokens=None, mirror=False):
    Y, logits, idx, w, counts = layer.forward(d["X"], aux=True)
    torch.cuda.synchronize()
    idx_np = _check_routing(cfg, d, logits, idx, w)
    np.testing.assert_array_equal(counts.cpu().numpy(), oracle.permute(idx_np, cfg.E)[0])
    L = oracle.Layer(d, cfg.k)
    if tokens is None:
        tokens = np.arange(cfg.T)
    elif isinstance(tokens, str) and tokens == "cover":
        # every touched expert, the first and last row of every expert block
        # (and of the shared expert's block), and a few tokens drawn at random
        rng = np.random.default_rng(cfg.T)
        tokens = cover_tokens(idx_np, [0, cfg.T - 1, *rng.choice(cfg.T, size=4, replace=False)])
        say(f"    comparing {tokens.size} of {cfg.T} tokens (covering {np.unique(idx_np[tokens]).size} of "
            f"{np.unique(idx_np).size} touched experts)")
    ref = oracle.forward_tokens(L, tokens, idx=idx_np[tokens], workers=ORACLE_THREADS)
    err = rel_err(Y[torch.as_tensor(tokens, device="cuda")], ref["Y"])
    say(f"    max rel err {err:.3e} (tol {tol_for(cfg)})")
    assert err <= tol_for(cfg)
    assert torch.isfinite(Y.float()).all()
    if mirror:
        ref_m = oracle.forward_tokens(L, tokens, idx=idx_np[tokens], act_quant=True, workers=ORACLE_THREADS)
        err_m = mean_rel(Y[torch.as_tensor(tokens, device="cuda")], ref_m["Y"])
        say(f"    against the quantisation mirror: mean {err_m:.3e} (tol {MIRROR_TOL})")
        assert err_m <= MIRROR_TOL
    return Y


@pytest.mark.parametrize("name,path", FFN_CASES)
def test_forward_mini(name, path):
    cfg = MINI_CONFIGS[name]
    say(f"[forward] {name} path={path}")
    d = screened_layer(cfg)
    Y = _check_forward(cfg, d, moe.MoELayer(d, cfg.k, path=path), mirror=path == "tiled_a8")
    Y2 = moe.MoELayer(d, cfg.k, path=path).forward(d["X"])
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)  # deterministic


def test_forward_worked_example():
    say("[forward] worked example (H, F padded to 32)")
    d = worked_example_layer(F=32, H=32, device="cuda")
    cfg = d["cfg"].with_(H=32, F=32)
    _check_forward(cfg, d, moe.MoELayer(d, cfg.k))


@pytest.mark.parametrize("variant", ["k1", "kE", "one_hot_expert", "T1"])
def test_forward_edge_cases(variant):
    base = MINI_CONFIGS["mini_bf16_decode"]
    cfg = {"k1": base.with_(k=1), "kE": base.with_(k=8), "T1": base.with_(T=1),
           "one_hot_expert": base.with_(T=200)}[variant]
    say(f"[forward] edge case {variant}")
    d = screened_layer(cfg)
    if variant == "one_hot_expert":
        # a large gate bias sends every token to expert 3 first and expert 5 second
        b = torch.zeros(cfg.E, dtype=torch.float32, device="cuda")
        b[3], b[5] = 60.0, 40.0
        d["gate_bias"] = b
    _check_forward(cfg, d, moe.MoELayer(d, cfg.k))


@pytest.mark.parametrize("variant", ["k16_shared", "k20", "k20_shared"])
def test_forward_w8a8_many_picks(variant):
    # the W8A8 forward quantises each token row once and writes its scales at
    # the rows of all its picks (and the shared expert's row); 16 lanes share
    # a row's picks, so 16 or more picks take a second pass over the lanes
    kw = {"k16_shared": dict(E=32, k=16), "k20": dict(E=32, k=20, Fs=0), "k20_shared": dict(E=32, k=20)}[variant]
    cfg = MINI_CONFIGS["mini_fp8_prefill"].with_(**kw)
    say(f"[forward] W8A8 with {cfg.k} picks of {cfg.E}, shared expert width {cfg.Fs}")
    d = screened_layer(cfg)
    _check_forward(cfg, d, moe.MoELayer(d, cfg.k, path="tiled_a8"), mirror=True)


def test_forward_empty_batch():
    cfg = MINI_CONFIGS["mini_bf16_decode"]
    d = screened_layer(cfg)
    layer = moe.MoELayer(d, cfg.k)
    X = d["X"][:0]
    Y = layer.forward(X)
    torch.cuda.synchronize()
    assert Y.shape == (0, cfg.H)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_forward_full_size(name):
    """Routing on every token; outputs on every token of the decode batches,
    and at prefill sizes on a set of tokens that covers every touched expert
    and the first and last row of every expert block."""
    cfg = CONFIGS[name]
    say(f"[forward] full size {name} T={cfg.T} H={cfg.H} F={cfg.F} E={cfg.E} k={cfg.k} Fs={cfg.Fs} w={cfg.w}")
    d = screened_layer(cfg)
    _check_forward(cfg, d, moe.MoELayer(d, cfg.k), None if cfg.T <= 64 else "cover")


# The method's size limits: 1024 experts (the most the router and permutation
# take) with and without the shared expert's extra group (1025 groups do not
# fit the one-block tile list, so that case builds it separately), and the
# largest batch (65535 tokens) on a small layer, checked on sampled tokens.
LIMIT_CASES = {
    "E1024": LayerConfig("limit_E1024", T=40, H=128, F=64, E=1024, k=2, seed=21),
    "E1024_shared": LayerConfig("limit_E1024_shared", T=40, H=128, F=64, E=1024, k=2, Fs=64, seed=22),
    "T65535": LayerConfig("limit_T65535", T=65535, H=64, F=64, E=8, k=2, seed=23),
    # more than one 1024-assignment chunk: the scan block writes the tile list
    # for 1024 groups, and leaves 1025 groups to the separate tile kernel
    "E1024_chunks": LayerConfig("limit_E1024_chunks", T=600, H=128, F=64, E=1024, k=2, seed=24),
    "E1024_chunks_shared": LayerConfig("limit_E1024_chunks_shared", T=600, H=128, F=64, E=1024, k=2, Fs=64,
                                       seed=25),
}


@pytest.mark.parametrize("name", list(LIMIT_CASES))
def test_forward_size_limits(name):
    cfg = LIMIT_CASES[name]
    say(f"[forward] size limit {name}: T={cfg.T} H={cfg.H} F={cfg.F} E={cfg.E} k={cfg.k} Fs={cfg.Fs}")
    d = screened_layer(cfg)
    tokens = None
    if cfg.T > 4096:
        rng = np.random.default_rng(cfg.seed)
        tokens = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, size=30, replace=False)]))
    _check_forward(cfg, d, moe.MoELayer(d, cfg.k), tokens)


# moe_forward enqueues kernels only (no host synchronisation, no memsets), so a
# whole layer can be captured in a HIP graph. Each replay runs after eager work
# of the program (the output zeroed, new token values copied into the captured
# input) and must equal an eager forward of the same input bit for bit.
GRAPH_CASES = [("mini_bf16_decode", "auto"), ("mini_fp8_decode", "auto"), ("mini_bf16_prefill", "auto"),
               ("mini_fp8_prefill", "auto"), ("mini_fp8_bf16s_decode", "auto")]


@pytest.mark.parametrize("name,path", GRAPH_CASES)
def test_forward_graph_replay(name, path):
    from synth import make_layer
    cfg = MINI_CONFIGS[name]
    say(f"[graph] {name} path={path}")
    d = screened_layer(cfg)
    layer = moe.MoELayer(d, cfg.k, path=path)
    X = d["X"].clone()
    Yg = torch.empty_like(X)
    # warm up on a side stream (sizes the workspace), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            layer.forward(X, Yg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward(X, Yg)
    torch.cuda.synchronize()
    inputs = [d["X"]] + [make_layer(cfg.with_(seed=cfg.seed + 100 + i), device="cuda", experts=False)["X"]
                         for i in range(3)]
    for rep, Xn in enumerate(inputs):
        X.copy_(Xn)
        Yg.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        Ye = layer.forward(Xn.clone())
        torch.cuda.synchronize()
        say(f"    replay {rep}: equal={torch.equal(Yg, Ye)}")
        assert torch.equal(Yg, Ye)
    del graph
