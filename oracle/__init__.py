"""Plain fp64 CPU oracle for the MoE layer forward.

TEST INFRASTRUCTURE ONLY. This package is the checker the HIP path is compared
against. Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import it; the library and its Python binding never do, and it shares
no code with them.

Sources: the page "MOE推理流程解析" (ffner.com), sections 一 (the layer computes
a routing-weighted sum over the chosen experts, plus any always-on shared
experts), 二 (assignments are grouped into per-expert matrices, the token id
travels with each row, combine weights and sums the contributions), 三 (router
scores, top-k keeps indices and weights, permutation with an inverse map, expert
activation and output projection, unpermute) and 九 (kept weights are
renormalised); the page "MoE serving production quirks" (tianpan.co), section
on the memory paradox (the gate runs a linear projection and a softmax over all
experts); the page "MoE-推理部署" (zzmblog.top), section on expert quantisation
(per-expert FP8 scales; MXFP4 as a single-GPU weight format). oracle.ep follows
"MOE推理流程解析" §五 (expert-parallel dispatch and combine).

Parity pins: see the functions' docstrings and tests/test_oracle_*.py. The
whole-layer output at model scale has no printed values on the pages; it is
pinned by the worked example, closed forms, special cases and a brute-force
per-token loop on small inputs.
"""
from .ref import (
    to_f64, e4m3_decode, e4m3_encode, quantize_rows_e4m3, dequant_rows, round_bf16, dequant_blocks,
    e2m1_decode, e8m0_decode, dequant_mxfp4, router_logits, softmax, select_topk,
    route, routing_weights, permute, silu, swiglu_ffn, grouped_ffn, combine,
    Layer, forward, forward_tokens,
)
from .brute import brute_force_forward
from . import ep

__all__ = [
    "to_f64", "e4m3_decode", "e4m3_encode", "quantize_rows_e4m3", "dequant_rows", "round_bf16", "dequant_blocks", "router_logits", "softmax",
    "select_topk", "route", "routing_weights", "permute", "silu", "swiglu_ffn",
    "grouped_ffn", "combine", "Layer", "forward", "forward_tokens",
    "brute_force_forward", "ep",
]
