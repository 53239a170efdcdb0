"""Seeded synthetic inputs for the MoE layer forward.

This package draws inputs only: token rows, gate weights, expert weights and
the fp8 storage format of those weights. It performs none of the layer's
arithmetic (no routing, no permutation, no expert FFN, no combine). Both the
CPU oracle and the HIP path are fed from here.
"""
from .configs import CONFIGS, MINI_CONFIGS, LayerConfig, get_config
from .gen import make_layer, redraw_rows, quantize_e4m3_blocks, quantize_mxfp4, spread_block_scales, tensor_seed

__all__ = ["CONFIGS", "MINI_CONFIGS", "LayerConfig", "get_config", "make_layer",
           "redraw_rows", "quantize_e4m3_blocks", "quantize_mxfp4", "spread_block_scales", "tensor_seed"]
