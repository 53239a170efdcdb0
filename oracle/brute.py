"""Brute-force per-token MoE layer in pure Python (test infrastructure only).

An independent second statement of the layer for tiny inputs: no matrices, no
permutation, no inverse map. For each token it scores every expert, sorts all
scores, keeps the first k, renormalises their softmax probabilities and adds up
the chosen experts' SwiGLU outputs computed element by element (page
"MOE推理流程解析", §一: the output is the routing-weighted sum over the chosen
experts, plus any always-on shared expert).
"""
from __future__ import annotations

import math


def _ffn(x, W1, W3, W2):
    H, F = len(W1), len(W1[0])
    h = []
    for f in range(F):
        g = 0.0
        u = 0.0
        for i in range(H):
            g += x[i] * W1[i][f]
            u += x[i] * W3[i][f]
        h.append(g / (1.0 + math.exp(-g)) * u)
    return [sum(h[f] * W2[f][o] for f in range(F)) for o in range(len(W2[0]))]


def brute_force_forward(X, Wg, gate_bias, k, experts, shared=None):
    """X: T lists of H floats; Wg: H lists of E floats; gate_bias: E floats or
    None; experts: E triples (W1, W3, W2) of nested lists; shared: a triple or
    None. Returns (chosen [T][k], weights [T][k], Y [T][H]) as Python lists.
    """
    E = len(Wg[0])
    chosen, weights, Y = [], [], []
    for x in X:
        scores = []
        for e in range(E):
            s = sum(x[i] * Wg[i][e] for i in range(len(x)))
            if gate_bias is not None:
                s += gate_bias[e]
            scores.append(s)
        ranked = sorted(range(E), key=lambda e: (-scores[e], e))
        top = ranked[:k]
        m = max(scores)
        p = [math.exp(s - m) for s in scores]
        z = sum(p)
        p = [v / z for v in p]
        kept = sum(p[e] for e in top)
        w = [p[e] / kept for e in top]
        y = [0.0] * len(x)
        for wj, e in zip(w, top):
            ye = _ffn(x, *experts[e])
            y = [a + wj * b for a, b in zip(y, ye)]
        if shared is not None:
            ys = _ffn(x, *shared)
            y = [a + b for a, b in zip(y, ys)]
        chosen.append(top)
        weights.append(w)
        Y.append(y)
    return chosen, weights, Y
