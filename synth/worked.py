"""Inputs that reproduce the four-token worked example.

The page "MOE推理流程解析" (ffner.com), section 二, prints only the routing
outcome: each token's two experts and their weights. The inputs below are one
choice that yields exactly that outcome: X is the 4x4 identity (H = T = 4), so
the scores equal the gate rows, and the gate holds ln(weight) for each chosen
pair and ln(0.1) elsewhere. Softmax of those scores gives the printed weights
for the chosen pair (they already sum to 1) and 0.1 for the rest, which is below
every printed weight, so the printed pair is also the top-2 pair.
"""
from __future__ import annotations

import json
import math
import os

import torch

from .configs import LayerConfig
from .gen import _normal

FIXTURE = os.path.join(os.path.dirname(__file__), "..", "tests", "golden", "worked_example.json")


def load_fixture(path: str = FIXTURE) -> dict:
    with open(path, encoding="utf-8") as fh:
        return json.load(fh)


def worked_example_layer(F: int = 8, device="cpu", fixture: dict | None = None, H: int | None = None) -> dict:
    """H defaults to T; a larger H pads X with zero columns and the gate with
    zero rows, which leaves every score unchanged."""
    fx = fixture or load_fixture()
    T, E, k = fx["T"], fx["E"], fx["k"]
    H = T if H is None else H
    if H < T:
        raise ValueError("H must be at least T")
    cfg = LayerConfig("worked_example", T=T, H=H, F=F, E=E, k=k, act="f32", w="f32", w_std=0.5)
    Wg = torch.zeros((H, E), dtype=torch.float64)
    Wg[:T] = math.log(0.1)
    for t, pairs in enumerate(fx["choices"]):
        for e1, w in pairs:
            Wg[t, e1 - 1] = math.log(w)
    out = {"cfg": cfg,
           "X": torch.eye(T, H, dtype=torch.float32, device=device),
           "Wg": Wg.to(torch.float32).to(device),
           "gate_bias": None}
    for name, r, c in (("W1", H, F), ("W3", H, F), ("W2", F, H)):
        out[name] = torch.stack([_normal(cfg, name, (r, c), cfg.w_std, device, e)
                                 for e in range(E)]).contiguous()
        out["S" + name[1:]] = None
    for name in ("Ws1", "Ws3", "Ws2", "Ss1", "Ss3", "Ss2"):
        out[name] = None
    return out
