"""MoE layer forward on one AMD Instinct MI355X (gfx950).

The layer: router (gate projection, softmax, top-k, renormalised weights) ->
dispatch (per-expert counts, offsets, stable permutation, inverse map) ->
grouped SwiGLU expert FFN (+ optional shared expert) -> combine. Every stage
is a HIP kernel in libmoe.so (C ABI: include/moe.h); this package is its thin
Python binding, with torch providing device memory and streams.
"""
from ._lib import (
    EP_STAGES, LIB_PATH, MOE_N_EVENTS, STAGES, EPLoopback, MoEError, MoELayer, StageEvents, combine, ep_dispatch,
    ep_exchange, ep_local_experts, ep_recv_offsets, grouped_ffn, lib, permute, quantize_e4m3_rows, rank_tokens,
    route,
)

__all__ = ["EP_STAGES", "LIB_PATH", "MOE_N_EVENTS", "STAGES", "EPLoopback", "MoEError", "MoELayer", "StageEvents",
           "combine", "ep_dispatch", "ep_exchange", "ep_local_experts", "ep_recv_offsets", "grouped_ffn", "lib",
           "permute", "quantize_e4m3_rows", "rank_tokens", "route"]
