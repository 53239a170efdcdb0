"""Expert-parallel dispatch and combine between G ranks on one GPU, against
the oracle (oracle/ep.py; page "MOE推理流程解析" §五).

Bit for bit: the owner bucketing (send offsets, send slots, records, token
rows), the all-to-all (receive offsets, records and rows), each rank's local
permutation of what it received, and the order in which results return to
their sources. Within the layer tolerance: the output Y against the exact
single-GPU oracle (which the G-rank oracle equals, pinned on the CPU).
"""
import os

import numpy as np
import pytest
import torch

import mixture_experts_layer_count_amd as moe
import oracle
from oracle import ep as oep
from synth import CONFIGS, MINI_CONFIGS
from _gpu import rel_err, say, screened_layer, tol_for

pytestmark = pytest.mark.gpu
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))

CASES = [("mini_bf16_decode", 2), ("mini_bf16_decode", 8), ("mini_bf16_prefill", 4), ("mini_bf16_wide", 8),
         ("mini_fp8_decode", 4), ("mini_fp8_prefill", 8), ("mini_mxfp4_shared", 2), ("mini_f32", 3),
         ("qwen3_decode", 8), ("dsv3_decode", 8)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    moe.lib()


def _np(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("name,G", CASES)
def test_ep_loopback(name, G):
    cfg = MINI_CONFIGS.get(name) or CONFIGS[name]
    say(f"[ep] {name} G={G} T={cfg.T} E={cfg.E} k={cfg.k}")
    d = screened_layer(cfg)
    epl = moe.EPLoopback(d, cfg.k, G)
    Y = epl.forward(d["X"], keep=True)
    torch.cuda.synchronize()
    st = epl.last
    L = oracle.Layer(d, cfg.k)
    X64 = L.X()
    T, k, E = cfg.T, cfg.k, cfg.E
    sends = []
    idx_all = np.zeros((T, k), dtype=np.int64)
    for r in range(G):
        tk = oep.rank_tokens(T, G, r)
        if tk.size == 0:
            sends.append(oep.dispatch(np.zeros((0, k), np.int64), np.zeros((0, k)), X64[:0], tk, E, G, r))
            continue
        logits, idx, w = (_np(x) for x in st["routes"][r])
        np.testing.assert_array_equal(idx, oracle.select_topk(logits, k))  # the rank's own routing
        idx_all[tk] = idx
        # dispatch: the oracle's buckets from the same routing
        s = oep.dispatch(idx, w.astype(np.float64), X64[tk], tk, E, G, r)
        sends.append(s)
        n = tk.size * k
        np.testing.assert_array_equal(_np(st["send_off"][r]), s["send_offsets"])
        np.testing.assert_array_equal(_np(st["send_slot"][r, :n]), s["send_slot"])
        meta = _np(st["send_meta"][r, :n])
        np.testing.assert_array_equal(meta[:, 0], s["meta"]["token"])
        np.testing.assert_array_equal(meta[:, 1], s["meta"]["expert"])
        np.testing.assert_array_equal(meta[:, 2], s["meta"]["src"])
        np.testing.assert_array_equal(meta[:, 3].view(np.float32), w.reshape(-1)[np.argsort(s["send_slot"])])
        assert torch.equal(st["send_rows"][r, :n], d["X"][torch.as_tensor(s["meta"]["token"], device="cuda")])
    # exchange
    recvs = oep.exchange(sends)
    for dd in range(G):
        r = recvs[dd]
        np.testing.assert_array_equal(_np(st["recv_off"][dd]), r["recv_offsets"])
        n = st["n_recv"][dd]
        assert n == r["recv_offsets"][-1]
        meta = _np(st["recv_meta"][dd, :n])
        np.testing.assert_array_equal(meta[:, 0], r["meta"]["token"])
        np.testing.assert_array_equal(meta[:, 1], r["meta"]["expert"])
        np.testing.assert_array_equal(meta[:, 2], r["meta"]["src"])
        assert torch.equal(st["recv_rows"][dd, :n], d["X"][torch.as_tensor(r["meta"]["token"], device="cuda")])
        if n == 0:
            continue
        # the receiver's local permutation
        local = (r["meta"]["expert"] - dd * (E // G)).reshape(-1, 1)
        counts, offsets, row_src, assign_row = oracle.permute(local, E // G)
        lidx, c_g, o_g, rs_g = st["local"][dd]
        np.testing.assert_array_equal(_np(lidx), local[:, 0])
        np.testing.assert_array_equal(_np(c_g), counts)
        np.testing.assert_array_equal(_np(o_g), offsets)
        np.testing.assert_array_equal(_np(rs_g), row_src)
        np.testing.assert_array_equal(_np(st["assign"][dd, :n]), assign_row)
    # returned rows: each result lands at its source's send row, bit for bit
    ret, Yp, assign = st["ret"], st["Yp"], st["assign"]
    for s_ in range(G):
        so = sends[s_]["send_offsets"]
        for dd in range(G):
            ro = recvs[dd]["recv_offsets"]
            cnt = so[dd + 1] - so[dd]
            if cnt == 0:
                continue
            src_rows = assign[dd, ro[s_]:ro[s_] + cnt].long()
            assert torch.equal(ret[s_, so[dd]:so[dd] + cnt], Yp[dd][src_rows])
    # the layer output
    np.testing.assert_array_equal(idx_all, oracle.select_topk(oracle.router_logits(X64, L.Wg(), L.gate_bias()), k))
    ref = oracle.forward_tokens(L, np.arange(T), idx=idx_all, workers=ORACLE_THREADS)["Y"]
    err = rel_err(Y, ref)
    say(f"    max rel err {err:.3e} (tol {tol_for(cfg)})")
    assert err <= tol_for(cfg)
    assert torch.isfinite(Y.float()).all()
