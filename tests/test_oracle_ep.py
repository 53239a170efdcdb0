"""Pins of the expert-parallel dispatch/combine oracle (oracle/ep.py), CPU only.

Page "MOE推理流程解析" §五: experts placed on GPUs, each assignment whose
expert lives elsewhere travels as a record (token vector + token id, target
expert, source GPU, routing weight), every GPU groups what it holds by expert
and runs one matrix per active local expert, and the source GPU restores token
order, applies the weights and sums. The page's own example (GPU A holds E1
and E2, GPU B holds E3 and E4; a token on A choosing E1 and E3 keeps E1 on A
and sends E3 to B) is checked on the §二 routing, with buckets derived by
hand in tests/golden/ep_example.json.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import ep
from synth import LayerConfig, make_layer
from synth.worked import worked_example_layer

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "ep_example.json")
RANK = {"A": 0, "B": 1}


@pytest.fixture(scope="module")
def fx():
    with open(GOLDEN, encoding="utf-8") as fh:
        return json.load(fh)


@pytest.fixture(scope="module")
def page_example(fx):
    d = worked_example_layer(F=8)
    L = oracle.Layer(d, 2)
    _, idx, w = oracle.route(L.X(), L.Wg(), None, 2)
    sends = []
    for name in ("A", "B"):
        tk = np.asarray(fx["rank_tokens"][name]) - 1
        sends.append(ep.dispatch(idx[tk], w[tk], L.X()[tk], tk, 4, fx["G"], RANK[name]))
    return L, idx, w, sends, ep.exchange(sends)


def test_owner_placement(fx):
    for e1, gpu in fx["owner"].items():
        assert ep.owner(int(e1) - 1, 4, 2) == RANK[gpu]
    # contiguous blocks of E/G experts
    np.testing.assert_array_equal(ep.owner(np.arange(16), 16, 4), np.repeat(np.arange(4), 4))
    with pytest.raises(ValueError):
        ep.owner(0, 6, 4)


def test_page_example_token_stays_and_travels(fx, page_example):
    _, idx, _, sends, _ = page_example
    pe = fx["page_example"]
    t = pe["token"] - 1
    src = RANK[pe["start"]]
    s = sends[src]
    a_stay = t * 2 + list(idx[t]).index(pe["stays"][0] - 1)
    a_go = t * 2 + list(idx[t]).index(pe["travels"][0] - 1)
    # the send row of each assignment lies in the segment of the named GPU
    for a, gpu in ((a_stay, pe["stays"][1]), (a_go, pe["travels"][1])):
        row = s["send_slot"][a]
        d = RANK[gpu]
        assert s["send_offsets"][d] <= row < s["send_offsets"][d + 1]


def test_page_example_buckets(fx, page_example):
    _, _, _, sends, _ = page_example
    for name, exp in fx["send"].items():
        s = sends[RANK[name]]
        np.testing.assert_array_equal(s["send_offsets"], exp["send_offsets"])
        np.testing.assert_array_equal(s["send_slot"], exp["send_slot"])
        for i, (tok, e, src, wt) in enumerate(exp["records"]):
            assert s["meta"]["token"][i] == tok - 1 and s["meta"]["expert"][i] == e - 1
            assert s["meta"]["src"][i] == RANK[src]
            assert s["meta"]["weight"][i] == pytest.approx(wt, abs=1e-6)  # fp32 ln(w) gate entries
            # the token vector travels with its record (X = identity here)
            np.testing.assert_array_equal(s["rows"][i], np.eye(4)[tok - 1])


def test_page_example_exchange_and_local_matrices(fx, page_example):
    L, _, _, _, recvs = page_example
    for name, exp in fx["receive"].items():
        r = recvs[RANK[name]]
        np.testing.assert_array_equal(r["recv_offsets"], exp["recv_offsets"])
        got = list(zip(r["meta"]["token"], r["meta"]["expert"], r["meta"]["src"]))
        assert got == [(t - 1, e - 1, RANK[g]) for t, e, g in exp["records"]]
    counts = []
    for name, exp in fx["local_expert_rows"].items():
        d = RANK[name]
        out = ep.expert_compute(recvs[d], 4, 2, d, L.expert)
        tokens = recvs[d]["meta"]["token"][out["row_src"]]
        for e1, toks in exp.items():
            l = int(e1) - 1 - 2 * d
            lo, hi = out["local_offsets"][l], out["local_offsets"][l + 1]
            assert list(tokens[lo:hi]) == [t - 1 for t in toks]
        counts += list(out["local_counts"])
    # the per-GPU expert matrices are the section 二 matrices
    assert counts == fx["row_counts_section_2"]


def test_page_example_combine_at_source(fx, page_example):
    """Constant expert outputs c_e: the source sums w * c_e over the token's
    experts (section 二: T1 = 0.7 E1 + 0.3 E3)."""
    _, idx, w, sends, recvs = page_example
    c = np.array([[1.0, 10.0], [100.0, 1000.0], [3.0, 5.0], [7.0, 11.0]])
    results = [c[recvs[d]["meta"]["expert"]] for d in range(2)]
    rets = ep.give_back(results, recvs, sends)
    for name, toks in fx["rank_tokens"].items():
        r = RANK[name]
        tk = np.asarray(toks) - 1
        Y = ep.combine_at_source(rets[r], sends[r]["send_slot"], w[tk], 2)
        for i, t in enumerate(tk):
            np.testing.assert_allclose(Y[i], w[t, 0] * c[idx[t, 0]] + w[t, 1] * c[idx[t, 1]], rtol=1e-15)
    (e_a, w_a), (e_b, w_b) = fx["combine_token_1"]
    Y1 = ep.combine_at_source(rets[0], sends[0]["send_slot"], w[[0, 1]], 2)[0]
    # the printed weights (the computed ones match them to the fp32 gate's 1e-6)
    np.testing.assert_allclose(Y1, w_a * c[e_a - 1] + w_b * c[e_b - 1], rtol=1e-6)
    np.testing.assert_allclose(Y1, 0.7 * c[0] + 0.3 * c[2], rtol=1e-6)


def _tiny(T, E, k, Fs=0, seed=0):
    cfg = LayerConfig(f"ep_tiny_{T}_{E}_{k}_{Fs}_{seed}", T=T, H=12, F=10, E=E, k=k, Fs=Fs, act="f32",
                      w="f32", w_std=0.3, seed=seed)
    return oracle.Layer(make_layer(cfg), k)


@pytest.mark.parametrize("T,E,k,Fs,G", [(10, 8, 2, 0, 1), (10, 8, 2, 0, 2), (11, 8, 3, 0, 4), (9, 8, 2, 6, 8),
                                        (3, 8, 2, 0, 4), (17, 12, 4, 5, 3), (16, 16, 16, 0, 4)])
def test_ep_forward_equals_single_gpu_layer(T, E, k, Fs, G):
    """Spreading the experts over G ranks changes where rows are computed,
    not what: Y equals the single-GPU layer (ranks may hold no tokens, and a
    rank may receive nothing)."""
    L = _tiny(T, E, k, Fs, seed=T + G)
    out = ep.forward(L, G)
    ref = oracle.forward(L)["Y"]
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("G", [1, 2, 4])
def test_ep_invariants(G):
    L = _tiny(13, 8, 3, seed=40 + G)
    out = ep.forward(L, G)
    sends, recvs = out["sends"], out["recvs"]
    T, k, E = 13, 3, 8
    total = 0
    for d, r in enumerate(recvs):
        # every received record names an expert of this rank, from the named source
        assert (ep.owner(r["meta"]["expert"], E, G) == d).all()
        for s in range(G):
            lo, hi = r["recv_offsets"][s], r["recv_offsets"][s + 1]
            assert (r["meta"]["src"][lo:hi] == s).all()
        total += r["recv_offsets"][-1]
    assert total == T * k
    X = L.X()
    for s in range(G):
        tk = ep.rank_tokens(T, G, s)
        n = tk.size * k
        assert sorted(sends[s]["send_slot"]) == list(range(n))
        # rows are ascending in assignment within each destination's segment
        order = np.argsort(sends[s]["send_slot"])
        for d in range(G):
            seg = order[sends[s]["send_offsets"][d]:sends[s]["send_offsets"][d + 1]]
            assert (np.diff(seg) > 0).all()
        # round trip: the result at send row send_slot[a] is expert e's FFN of token a // k
        for a in range(n):
            t = tk[a // k]
            e = int(out["idx"][t, a % k])
            expect = oracle.swiglu_ffn(X[t:t + 1], *L.expert(e))[0]
            np.testing.assert_allclose(out["returns"][s][sends[s]["send_slot"][a]], expect, rtol=1e-12, atol=1e-14)
