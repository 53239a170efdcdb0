"""Pins of the fp64 oracle against facts that do not come from the oracle.

Sources of truth used here: the worked example printed on the page
"MOE推理流程解析" (section 二), closed forms, library routines (scipy softmax,
numpy stable argsort, torch's float8_e4m3fn decoding, torch's silu), special
cases that reduce the layer to a dense SwiGLU FFN, invariants stated on the
pages, and a brute-force per-token loop written element by element.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import brute_force_forward
from synth import make_layer, LayerConfig
from synth.worked import load_fixture, worked_example_layer

FX = load_fixture()


# --------------------------------------------------------------------------
# Worked example (page "MOE推理流程解析", section 二)
# --------------------------------------------------------------------------

def _expected_route():
    idx, w = [], []
    for pairs in FX["choices"]:
        pairs = sorted(pairs, key=lambda p: (-p[1], p[0]))  # best first
        idx.append([e - 1 for e, _ in pairs])
        w.append([v for _, v in pairs])
    return np.array(idx), np.array(w)


def test_worked_example_route():
    L = oracle.Layer(worked_example_layer(), FX["k"])
    logits, idx, w = oracle.route(L.X(), L.Wg(), None, L.k)
    exp_idx, exp_w = _expected_route()
    np.testing.assert_array_equal(idx, exp_idx)
    # the inputs are fp32 logs of the printed weights; fp32 rounding of ln(w)
    # moves the weights by ~1e-7 relative
    np.testing.assert_allclose(w, exp_w, rtol=0, atol=1e-6)


def test_worked_example_permute():
    exp_idx, _ = _expected_route()
    counts, offsets, row_src, assign_row = oracle.permute(exp_idx, FX["E"])
    assert int(counts.sum()) == FX["assignments"] == FX["T"] * FX["k"]
    np.testing.assert_array_equal(counts, FX["row_counts"])
    np.testing.assert_array_equal(offsets, [0, 3, 5, 7, 8])
    for e1, toks in FX["groups"].items():
        e = int(e1) - 1
        rows = range(offsets[e], offsets[e + 1])
        assert [int(row_src[r]) // FX["k"] + 1 for r in rows] == toks
    # with slots best-first, the page's assignments land in these rows
    np.testing.assert_array_equal(row_src, [0, 3, 4, 5, 6, 1, 2, 7])
    np.testing.assert_array_equal(assign_row, [0, 5, 6, 1, 2, 3, 4, 7])


def test_worked_example_combine_constant_rows():
    """Expert e returns the constant row c_e; token 1 gets 0.7*c_E1 + 0.3*c_E3."""
    T, k, E, H = FX["T"], FX["k"], FX["E"], 3
    exp_idx, exp_w = _expected_route()
    counts, offsets, row_src, assign_row = oracle.permute(exp_idx, E)
    c = np.array([[1.0, 10.0, 100.0], [2.0, 20.0, 200.0], [3.0, 30.0, 300.0], [4.0, 40.0, 400.0]])
    Yp = np.zeros((T * k, H))
    for e in range(E):
        Yp[offsets[e]:offsets[e + 1]] = c[e]
    Y = oracle.combine(Yp, assign_row, exp_w, T, k)
    (e_a, w_a), (e_b, w_b) = FX["combine_token_1"]
    np.testing.assert_allclose(Y[0], w_a * c[e_a - 1] + w_b * c[e_b - 1], rtol=1e-15)
    for t, pairs in enumerate(FX["choices"]):
        np.testing.assert_allclose(Y[t], sum(v * c[e - 1] for e, v in pairs), rtol=1e-15)


def test_worked_example_full_layer_matches_brute_force():
    d = worked_example_layer()
    L = oracle.Layer(d, FX["k"])
    ref = oracle.forward(L)
    experts = [tuple(m.tolist() for m in L.expert(e)) for e in range(L.E)]
    chosen, weights, Y = brute_force_forward(L.X().tolist(), L.Wg().tolist(), None, L.k, experts)
    np.testing.assert_array_equal(ref["idx"], chosen)
    np.testing.assert_allclose(ref["w"], weights, atol=1e-14)
    np.testing.assert_allclose(ref["Y"], Y, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Router closed forms and special cases
# --------------------------------------------------------------------------

def _rand_logits(T, E, seed):
    return np.random.default_rng(seed).normal(size=(T, E)) * 2.0


@pytest.mark.parametrize("T,E,k", [(50, 8, 2), (40, 128, 8), (20, 256, 8), (10, 5, 3)])
def test_renormalised_topk_is_softmax_over_selected(T, E, k):
    L = _rand_logits(T, E, T + E + k)
    idx = oracle.select_topk(L, k)
    w = oracle.routing_weights(L, idx)
    sel = np.take_along_axis(L, idx, axis=1)
    np.testing.assert_allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-13, atol=0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(sel, axis=1) <= 0)  # best first


def test_select_topk_matches_stable_argsort():
    L = _rand_logits(200, 64, 7)
    L[:, 10] = L[:, 3]  # exact ties: lower index must come first
    for k in (1, 2, 8, 64):
        ref = np.argsort(-L, axis=1, kind="stable")[:, :k]
        np.testing.assert_array_equal(oracle.select_topk(L, k), ref)


def test_select_topk_in_float32_decides_in_float32():
    L = np.array([[1.0, 1.0 + 1e-12, 0.5]])
    assert oracle.select_topk(L, 1)[0, 0] == 1
    assert oracle.select_topk(L.astype(np.float32), 1)[0, 0] == 0  # equal in fp32: lower index


def test_k1_weight_is_one_and_kE_is_full_softmax():
    L = _rand_logits(30, 16, 3)
    idx1 = oracle.select_topk(L, 1)
    np.testing.assert_array_equal(oracle.routing_weights(L, idx1), 1.0)
    np.testing.assert_array_equal(idx1[:, 0], np.argmax(L, axis=1))
    idxE = oracle.select_topk(L, 16)
    wE = oracle.routing_weights(L, idxE)
    full = scipy.special.softmax(L, axis=1)
    np.testing.assert_allclose(wE, np.take_along_axis(full, idxE, axis=1), rtol=1e-13)


def test_softmax_matches_scipy_and_survives_large_logits():
    L = _rand_logits(10, 32, 1) * 200.0
    np.testing.assert_allclose(oracle.softmax(L), scipy.special.softmax(L, axis=1), rtol=1e-12, atol=1e-300)


def test_router_logits_bias_shift():
    rng = np.random.default_rng(0)
    X, Wg, b = rng.normal(size=(6, 9)), rng.normal(size=(9, 4)), rng.normal(size=4)
    ref = np.array([[sum(X[t, h] * Wg[h, e] for h in range(9)) + b[e] for e in range(4)] for t in range(6)])
    np.testing.assert_allclose(oracle.router_logits(X, Wg, b), ref, rtol=1e-13)


# --------------------------------------------------------------------------
# Permutation invariants (pages: T*k assignments, inverse map, stable rows)
# --------------------------------------------------------------------------

def _counting_sort_by_hand(flat, E):
    buckets = [[] for _ in range(E)]
    for a, e in enumerate(flat):
        buckets[e].append(a)
    return [a for b in buckets for a in b]


@pytest.mark.parametrize("T,E,k,seed", [(1, 4, 1, 0), (37, 5, 2, 1), (300, 64, 8, 2), (64, 256, 8, 3), (9, 3, 3, 4)])
def test_permute_invariants(T, E, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    counts, offsets, row_src, assign_row = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    assert counts.sum() == T * k
    assert offsets[0] == 0 and offsets[-1] == T * k
    np.testing.assert_array_equal(np.sort(assign_row), np.arange(T * k))
    np.testing.assert_array_equal(row_src[assign_row], np.arange(T * k))
    np.testing.assert_array_equal(list(row_src), _counting_sort_by_hand(flat.tolist(), E))
    for e in range(E):
        rows = row_src[offsets[e]:offsets[e + 1]]
        assert np.all(flat[rows] == e)
        assert np.all(np.diff(rows) > 0)
        # a token never picks an expert twice, so rows also ascend by token
        assert np.all(np.diff(rows // k) > 0)
    # unpermute(permute(X)) gives each token row back k times
    X = rng.normal(size=(T, 3))
    Xp = X[row_src // k]
    np.testing.assert_array_equal(Xp[assign_row].reshape(T, k, 3), np.repeat(X[:, None], k, axis=1))


def test_permute_empty_experts():
    idx = np.array([[2, 0], [2, 0], [0, 2]])
    counts, offsets, row_src, assign_row = oracle.permute(idx, 5)
    np.testing.assert_array_equal(counts, [3, 0, 3, 0, 0])
    np.testing.assert_array_equal(offsets, [0, 3, 3, 6, 6, 6])
    np.testing.assert_array_equal(row_src, [1, 3, 4, 0, 2, 5])


# --------------------------------------------------------------------------
# Expert FFN and whole-layer special cases
# --------------------------------------------------------------------------

def test_silu_matches_torch():
    z = np.linspace(-30, 30, 1001)
    ref = torch.nn.functional.silu(torch.tensor(z, dtype=torch.float64)).numpy()
    np.testing.assert_allclose(oracle.silu(z), ref, rtol=1e-15, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0


def _tiny(T=7, H=6, F=5, E=4, k=2, Fs=0, zipf=0.0, seed=0):
    cfg = LayerConfig("tiny", T=T, H=H, F=F, E=E, k=k, Fs=Fs, act="f32", w="f32",
                      w_std=0.4, zipf_s=zipf, seed=seed)
    return cfg, make_layer(cfg)


def test_swiglu_ffn_matches_elementwise_loop():
    rng = np.random.default_rng(5)
    x = rng.normal(size=(3, 6))
    W1, W3, W2 = rng.normal(size=(6, 4)), rng.normal(size=(6, 4)), rng.normal(size=(4, 6))
    ref = []
    for r in range(3):
        h = []
        for f in range(4):
            g = sum(x[r, i] * W1[i, f] for i in range(6))
            u = sum(x[r, i] * W3[i, f] for i in range(6))
            h.append(g * u / (1 + math.exp(-g)))
        ref.append([sum(h[f] * W2[f, o] for f in range(4)) for o in range(6)])
    np.testing.assert_allclose(oracle.swiglu_ffn(x, W1, W3, W2), ref, rtol=1e-13)


def test_single_expert_top1_is_dense_swiglu_ffn():
    cfg, d = _tiny(E=1, k=1)
    L = oracle.Layer(d, 1)
    out = oracle.forward(L)
    x = torch.tensor(L.X())
    W1, W3, W2 = (torch.tensor(m) for m in L.expert(0))
    dense = (torch.nn.functional.silu(x @ W1) * (x @ W3)) @ W2
    np.testing.assert_allclose(out["Y"], dense.numpy(), rtol=1e-13)
    np.testing.assert_array_equal(out["w"], 1.0)


def test_identical_experts_ignore_routing():
    cfg, d = _tiny(E=5, k=3, seed=1)
    for key in ("W1", "W3", "W2"):
        d[key] = d[key][0:1].repeat(5, 1, 1)
    L = oracle.Layer(d, 3)
    out = oracle.forward(L)
    np.testing.assert_allclose(out["Y"], oracle.swiglu_ffn(L.X(), *L.expert(0)), rtol=1e-12)


def test_zero_up_projection_gives_zero():
    cfg, d = _tiny(seed=2)
    d["W3"] = torch.zeros_like(d["W3"])
    assert np.all(oracle.forward(oracle.Layer(d, 2))["Y"] == 0.0)


def test_linear_in_down_projection():
    cfg, d = _tiny(seed=3)
    y1 = oracle.forward(oracle.Layer(d, 2))["Y"]
    d2 = dict(d)
    d2["W2"] = d["W2"] * 4.0  # power of two: exact in fp32
    y3 = oracle.forward(oracle.Layer(d2, 2))["Y"]
    np.testing.assert_allclose(y3, 4.0 * y1, rtol=1e-13, atol=1e-15)


def test_padding_rows_do_not_change_real_rows():
    """Page "MOE推理流程解析" §二: padding rows carry no tokens; padded groups
    computed with the same experts give the same real rows."""
    cfg, d = _tiny(T=9, seed=4)
    L = oracle.Layer(d, 2)
    out = oracle.forward(L)
    pad = 3
    rows, offs = [], [0]
    for e in range(L.E):
        lo, hi = out["offsets"][e], out["offsets"][e + 1]
        rows.append(out["Xp"][lo:hi])
        rows.append(np.zeros((pad, L.H)))
        offs.append(offs[-1] + (hi - lo) + pad)
    Yp_pad = oracle.grouped_ffn(np.concatenate(rows), np.array(offs), L.expert)
    for e in range(L.E):
        lo, hi = out["offsets"][e], out["offsets"][e + 1]
        np.testing.assert_array_equal(Yp_pad[offs[e]:offs[e] + (hi - lo)], out["Yp"][lo:hi])


def test_grouped_equals_per_expert_loop():
    """§三: grouping reduces launches but does not change the content."""
    cfg, d = _tiny(T=11, E=6, k=3, seed=8)
    L = oracle.Layer(d, 3)
    out = oracle.forward(L)
    for a in range(11 * 3):
        t, j = divmod(a, 3)
        e = out["idx"][t, j]
        np.testing.assert_allclose(out["Yp"][out["assign_row"][a]],
                                   oracle.swiglu_ffn(L.X()[t:t + 1], *L.expert(e))[0], rtol=1e-14)


@pytest.mark.parametrize("seed,E,k,Fs,zipf", [(0, 4, 2, 0, 0.0), (1, 6, 3, 0, 1.1), (2, 8, 8, 0, 0.0),
                                              (3, 5, 1, 4, 0.0), (4, 7, 2, 5, 1.1)])
def test_oracle_matches_brute_force(seed, E, k, Fs, zipf):
    cfg, d = _tiny(T=8, H=6, F=5, E=E, k=k, Fs=Fs, zipf=zipf, seed=seed)
    L = oracle.Layer(d, k)
    out = oracle.forward(L)
    experts = [tuple(m.tolist() for m in L.expert(e)) for e in range(E)]
    shared = tuple(m.tolist() for m in L.shared()) if L.has_shared() else None
    b = L.gate_bias()
    chosen, weights, Y = brute_force_forward(L.X().tolist(), L.Wg().tolist(),
                                             None if b is None else b.tolist(), k, experts, shared)
    np.testing.assert_array_equal(out["idx"], chosen)
    np.testing.assert_allclose(out["w"], weights, rtol=1e-13)
    np.testing.assert_allclose(out["Y"], Y, rtol=1e-12, atol=1e-13)
    sub = oracle.forward_tokens(L, [5, 0, 3])
    np.testing.assert_allclose(sub["Y"], out["Y"][[5, 0, 3]], rtol=1e-13, atol=1e-14)
    # experts evaluated on a thread pool: the same values, bit for bit
    par = oracle.forward_tokens(L, [5, 0, 3], workers=4)
    assert np.array_equal(par["Y"], sub["Y"]) and np.array_equal(par["y"], sub["y"])


def test_shared_expert_special_cases():
    cfg, d = _tiny(Fs=4, seed=6)
    L = oracle.Layer(d, 2)
    d0 = dict(d)
    d0["W2"] = torch.zeros_like(d["W2"])
    only_shared = oracle.forward(oracle.Layer(d0, 2))["Y"]
    np.testing.assert_allclose(only_shared, oracle.swiglu_ffn(L.X(), *L.shared()), rtol=1e-13)
    d1 = dict(d)
    d1["Ws2"] = torch.zeros_like(d["Ws2"])
    routed = oracle.forward(oracle.Layer(d1, 2))["Y"]
    dn = dict(d)
    for kk in ("Ws1", "Ws3", "Ws2"):
        dn[kk] = None
    np.testing.assert_array_equal(routed, oracle.forward(oracle.Layer(dn, 2))["Y"])


# --------------------------------------------------------------------------
# fp8 (OCP E4M3) decoding
# --------------------------------------------------------------------------

def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]


def test_e4m3_decode_closed_forms():
    d = oracle.e4m3_decode
    assert d([0x7E])[0] == 448.0
    assert d([0xFE])[0] == -448.0
    assert d([0x38])[0] == 1.0
    assert d([0x01])[0] == 2.0 ** -9
    assert d([0x07])[0] == 7 * 2.0 ** -9
    assert d([0x08])[0] == 2.0 ** -6
    assert d([0x00])[0] == 0.0 and np.signbit(d([0x80])[0])


def test_dequant_blocks_applies_block_scales():
    codes = np.full((256, 384), 0x38, dtype=np.uint8)  # all 1.0
    scales = np.arange(6, dtype=np.float32).reshape(2, 3) + 0.5
    W = oracle.dequant_blocks(codes, scales)
    for bi in range(2):
        for bj in range(3):
            assert np.all(W[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128] == scales[bi, bj])
