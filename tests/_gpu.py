"""Helpers shared by the GPU parity tests.

Inputs come from synth (seeded) and are screened with the oracle's fp64
logits: for every token the adjacent gaps among its top min(k+1, E) logits
must be at least GAP, otherwise the token's row is redrawn from its own
substream. Routing is then a clean decision that fp32 and fp64 agree on.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from synth import make_layer, redraw_rows

GAP = 1e-3
TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def small_gaps(logits: np.ndarray, k: int, gap: float = GAP) -> np.ndarray:
    """Tokens whose top min(k+1, E) sorted logits have an adjacent gap < gap."""
    n = min(k + 1, logits.shape[1])
    top = -np.sort(-logits, axis=1)[:, :n]
    if n < 2:
        return np.zeros(0, dtype=np.int64)
    return np.nonzero((top[:, :-1] - top[:, 1:]).min(axis=1) < gap)[0]


def screen_rows(cfg, d: dict, max_attempts: int = 16) -> None:
    for attempt in range(max_attempts):
        L = oracle.router_logits(d["X"], d["Wg"], d.get("gate_bias"))
        bad = small_gaps(L, cfg.k)
        if bad.size == 0:
            return
        redraw_rows(cfg, d["X"], bad, attempt)
    raise RuntimeError(f"{cfg.name}: gap screening did not converge")


def screened_layer(cfg, device="cuda", experts: bool = True) -> dict:
    d = make_layer(cfg, device=device, experts=experts)
    screen_rows(cfg, d)
    return d


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over the whole array (fp64)."""
    got = got.detach().float().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got.astype(np.float64) - ref).max() / (den if den > 0 else 1.0))


def tol_for(cfg) -> float:
    return TOL[cfg.w] if cfg.w == "fp8" else TOL[cfg.act]


def cover_tokens(idx: np.ndarray, extra=()) -> np.ndarray:
    """Tokens whose outputs are compared at full size: a greedy cover of the
    routed sets (each step adds the token that chooses the most experts not
    yet covered, until every touched expert is), plus the first and last row
    of every expert block (rows are in ascending token order, so the smallest
    and largest token that chose the expert), plus `extra`. Every token also
    passes through the shared expert, whose block's first and last rows are
    tokens 0 and T - 1 (in `extra` by the caller when there is one)."""
    idx = np.asarray(idx)
    T = idx.shape[0]
    uncovered = set(np.unique(idx).tolist())
    sets = [set(row.tolist()) for row in idx]
    chosen = []
    while uncovered:
        t = max(range(T), key=lambda i: len(sets[i] & uncovered))
        chosen.append(t)
        uncovered -= sets[t]
    ends = []
    for e in np.unique(idx):
        ts = np.nonzero((idx == e).any(axis=1))[0]
        ends += [ts[0], ts[-1]]
    return np.unique(np.concatenate([np.asarray(chosen, dtype=np.int64), np.asarray(ends, dtype=np.int64),
                                     np.asarray(list(extra), dtype=np.int64)]))

