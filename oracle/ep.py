"""fp64 reference for expert-parallel dispatch and combine (test infrastructure
only).

Page "MOE推理流程解析" §五 (dispatch and combine under expert parallelism):
experts are placed on GPUs; an assignment whose expert lives on another GPU
travels there as a record holding the token vector and its routing metadata
(token id, target expert, source GPU, routing weight); every GPU groups the
assignments it holds by expert and runs one matrix per active local expert;
results go back to the source GPU, which restores token order with the saved
identifiers, applies the routing weights and sums each token's
contributions. With more GPUs the traffic becomes all-to-all; the expert
weights stay where they are.

Here G ranks stand for the GPUs. Expert e is owned by rank e // (E / G)
(contiguous blocks of E/G experts, E divisible by G). Rank r's tokens are the
contiguous slice `rank_tokens(T, G, r)`. Each step is written plainly, in the
page's order, on numpy arrays; nothing is shared with the HIP path.
"""
from __future__ import annotations

import numpy as np

from . import ref


def owner(e, E: int, G: int):
    """Rank holding expert e: experts are placed in contiguous blocks of E/G."""
    if E % G:
        raise ValueError("E must be divisible by G")
    return np.asarray(e, dtype=np.int64) // (E // G)


def rank_tokens(T: int, G: int, r: int) -> np.ndarray:
    """Token ids held by rank r: the r-th of G contiguous slices of ceil(T/G)
    tokens (the last ones may be shorter or empty)."""
    n = -(-T // G)
    return np.arange(min(r * n, T), min((r + 1) * n, T), dtype=np.int64)


def dispatch(idx, w, X, tokens, E: int, G: int, rank: int) -> dict:
    """Bucket one rank's assignments by destination rank and pack the records.

    idx, w: [n, k] routing of the rank's n tokens (global token ids `tokens`),
    X: [n, H] their rows. Assignment a = i*k + j (local token i, slot j).
    Send order: by destination rank, ascending a within each destination (a
    stable sort on the owner of the chosen expert).
      send_offsets[d] = first send row for rank d ([G+1], send_offsets[G] = n*k)
      send_slot[a]    = send row of assignment a
      rows[s]         = X[a // k] for a = the assignment at send row s
      meta[s]         = (token id, expert, source rank, weight) of that assignment
    """
    idx = np.asarray(idx, dtype=np.int64)
    n, k = idx.shape
    flat = idx.reshape(-1)
    dest = owner(flat, E, G)
    order = np.argsort(dest, kind="stable")  # send row -> assignment
    counts = np.bincount(dest, minlength=G)
    send_offsets = np.zeros(G + 1, dtype=np.int64)
    send_offsets[1:] = np.cumsum(counts)
    send_slot = np.empty(n * k, dtype=np.int64)
    send_slot[order] = np.arange(n * k)
    X = np.asarray(X)
    rows = X[order // k] if n * k else X[:0]
    wf = np.asarray(w, dtype=np.float64).reshape(-1)
    meta = {"token": np.asarray(tokens, dtype=np.int64)[order // k], "expert": flat[order],
            "src": np.full(n * k, rank, dtype=np.int64), "weight": wf[order]}
    return dict(send_offsets=send_offsets, send_slot=send_slot, rows=rows, meta=meta)


def exchange(sends) -> list:
    """All-to-all: rank d receives, for each source rank s in ascending order,
    s's send rows for d in their send order. `sends[s]` has send_offsets, rows
    and meta (as from `dispatch`). Returns per destination: rows, meta and
    recv_offsets ([G+1]: where each source's segment starts)."""
    G = len(sends)
    out = []
    for d in range(G):
        seg_rows, seg_meta, starts = [], {key: [] for key in ("token", "expert", "src", "weight")}, [0]
        for s in range(G):
            lo, hi = int(sends[s]["send_offsets"][d]), int(sends[s]["send_offsets"][d + 1])
            seg_rows.append(sends[s]["rows"][lo:hi])
            for key in seg_meta:
                seg_meta[key].append(sends[s]["meta"][key][lo:hi])
            starts.append(starts[-1] + hi - lo)
        out.append(dict(rows=np.concatenate(seg_rows),
                        meta={key: np.concatenate(v) for key, v in seg_meta.items()},
                        recv_offsets=np.asarray(starts, dtype=np.int64)))
    return out


def expert_compute(recv, E: int, G: int, rank: int, expert) -> dict:
    """One rank's expert work on the assignments it received: group them by
    local expert (stable, ascending receive order: the single-GPU permutation
    of `ref.permute` over local expert ids), run each active local expert's
    SwiGLU FFN on its rows, and return the results in receive order.
    `expert(e)` gives (W1, W3, W2) of global expert e in float64."""
    El = E // G
    local = np.asarray(recv["meta"]["expert"], dtype=np.int64) - rank * El
    if local.size and (local.min() < 0 or local.max() >= El):
        raise ValueError("a record names an expert this rank does not hold")
    counts, offsets, row_src, assign_row = ref.permute(local.reshape(-1, 1), El)
    rows = np.asarray(recv["rows"], dtype=np.float64)
    Xp = rows[row_src]
    Yp = ref.grouped_ffn(Xp, offsets, lambda l: expert(rank * El + l))
    if local.size == 0:
        Yp = np.zeros((0, rows.shape[1]), dtype=np.float64)
    return dict(local_counts=counts, local_offsets=offsets, row_src=row_src, assign_row=assign_row,
                Yp=Yp, results=Yp[assign_row])


def give_back(results, recvs, sends) -> list:
    """The return all-to-all: result row i of rank d's receive segment from
    source s goes back to s at send row send_offsets_s[d] + i, so every source
    gets its results in its own send order."""
    G = len(sends)
    out = []
    for s in range(G):
        parts = []
        for d in range(G):
            lo, hi = int(recvs[d]["recv_offsets"][s]), int(recvs[d]["recv_offsets"][s + 1])
            parts.append(results[d][lo:hi])
        ret = np.concatenate(parts)
        assert ret.shape[0] == int(sends[s]["send_offsets"][G])
        out.append(ret)
    return out


def combine_at_source(ret, send_slot, w, k: int, S=None) -> np.ndarray:
    """Y[i] = sum_j w[i, j] * ret[send_slot[i*k + j]] (+ S[i]): restore token
    order through the saved send rows, weight and sum (ref.combine with the
    send rows as the inverse map)."""
    n = np.asarray(w).shape[0]
    return ref.combine(ret, send_slot, w, n, k, S)


def forward(layer: "ref.Layer", G: int) -> dict:
    """The whole layer with experts spread over G ranks: route on each rank,
    dispatch, exchange, expert compute, return, combine at the source (plus the
    shared expert, replicated on every rank). Y equals ref.forward's."""
    X = layer.X()
    T, k, E = layer.T, layer.k, layer.E
    logits, idx, w = ref.route(X, layer.Wg(), layer.gate_bias(), k)
    sends = []
    for r in range(G):
        tk = rank_tokens(T, G, r)
        sends.append(dispatch(idx[tk], w[tk], X[tk], tk, E, G, r))
    recvs = exchange(sends)
    outs = [expert_compute(recvs[d], E, G, d, layer.expert) for d in range(G)]
    rets = give_back([o["results"] for o in outs], recvs, sends)
    Y = np.zeros((T, layer.H), dtype=np.float64)
    for r in range(G):
        tk = rank_tokens(T, G, r)
        S = ref.swiglu_ffn(X[tk], *layer.shared()) if layer.has_shared() else None
        Y[tk] = combine_at_source(rets[r], sends[r]["send_slot"], w[tk], k, S)
    return dict(idx=idx, w=w, sends=sends, recvs=recvs, experts=outs, returns=rets, Y=Y)
