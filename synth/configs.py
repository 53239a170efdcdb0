"""Layer shapes for the synthetic workloads.

Names follow the pages' notation: T tokens, H hidden size, F per-expert FFN
width, E routed experts, k experts chosen per token, Fs the width of the
always-on shared expert (0 = none).

Model shapes: Mixtral-8x7B (E=8, top-2), Qwen3-30B-A3B (E=128, top-8) and
DeepSeek-V3 (E=256 routed + 1 shared, top-8), stated on the pages
"MOE推理流程解析" (section 一, model card figures) and the ai-master page's
expert-parallel paragraph; H and F are the published layer widths of those
models.
"""
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    F: int
    E: int
    k: int
    Fs: int = 0            # shared-expert width; 0 = no shared expert
    act: str = "bf16"      # activation / gate dtype: "f32" or "bf16"
    w: str = "bf16"        # expert weight dtype: "f32", "bf16", "fp8" or "mxfp4"
    ws: str = ""           # shared-expert weight dtype ("" = w; "bf16" beside fp8)
    wg: str = ""           # gate dtype ("" = act; "f32" beside bf16: higher-precision router)
    zipf_s: float = 0.0    # > 0: gate bias b[e] = -s*ln(e+1) (hot low experts)
    x_std: float = 1.0
    w_std: float = 0.02
    seed: int = 0

    @property
    def shared_w(self) -> str:
        """Storage dtype of the shared expert's weights."""
        return self.ws or self.w

    @property
    def A(self) -> int:
        """Number of (token, expert) assignments, T*k."""
        return self.T * self.k

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


# Full-size workloads (one MoE layer each).
CONFIGS = {
    c.name: c for c in [
        LayerConfig("toy_fp32", T=64, H=128, F=256, E=8, k=2, act="f32", w="f32"),
        LayerConfig("mixtral_decode", T=16, H=4096, F=14336, E=8, k=2),
        LayerConfig("mixtral_prefill", T=4096, H=4096, F=14336, E=8, k=2, zipf_s=1.1),
        LayerConfig("qwen3_decode", T=32, H=2048, F=768, E=128, k=8),
        LayerConfig("qwen3_prefill", T=8192, H=2048, F=768, E=128, k=8),
        LayerConfig("dsv3_decode", T=64, H=7168, F=2048, E=256, k=8, Fs=2048, w="fp8"),
        LayerConfig("dsv3_prefill", T=4096, H=7168, F=2048, E=256, k=8, Fs=2048, w="fp8"),
        # the shared expert kept in bf16 beside the fp8 routed experts (same draws)
        LayerConfig("dsv3_decode_bf16_shared", T=64, H=7168, F=2048, E=256, k=8, Fs=2048, w="fp8", ws="bf16"),
        LayerConfig("dsv3_prefill_bf16_shared", T=4096, H=7168, F=2048, E=256, k=8, Fs=2048, w="fp8",
                    ws="bf16"),
        # the router kept in fp32 beside bf16 tokens (same draws)
        LayerConfig("qwen3_prefill_f32_router", T=8192, H=2048, F=768, E=128, k=8, wg="f32"),
        # MXFP4 experts (row-streaming kernel), decode batches
        LayerConfig("mixtral_decode_mxfp4", T=16, H=4096, F=14336, E=8, k=2, w="mxfp4"),
        LayerConfig("qwen3_decode_mxfp4", T=32, H=2048, F=768, E=128, k=8, w="mxfp4"),
        # MXFP4 experts at prefill sizes: decoded to bf16 for the tiled kernels
        LayerConfig("mixtral_prefill_mxfp4", T=4096, H=4096, F=14336, E=8, k=2, zipf_s=1.1, w="mxfp4"),
        LayerConfig("qwen3_prefill_mxfp4", T=8192, H=2048, F=768, E=128, k=8, w="mxfp4"),
    ]
}

# Reduced shapes with the same dtypes and routing structure, small enough for
# the oracle to compute every output in seconds, with ragged tails (T, F and H
# not multiples of the kernels' tiles where the format allows it).
MINI_CONFIGS = {
    c.name: c for c in [
        LayerConfig("mini_f32", T=37, H=96, F=160, E=12, k=2, act="f32", w="f32", seed=1),
        LayerConfig("mini_bf16_decode", T=13, H=544, F=672, E=8, k=2, seed=2),
        LayerConfig("mini_bf16_prefill", T=700, H=512, F=384, E=8, k=2, zipf_s=1.1, seed=3),
        LayerConfig("mini_bf16_wide", T=300, H=256, F=192, E=64, k=8, seed=4),
        # enough rows per expert for 256-row tiles, ragged in rows, N and K
        LayerConfig("mini_bf16_tall", T=1536, H=640, F=416, E=8, k=2, zipf_s=1.1, seed=7),
        # bf16 shared expert as wide as the routed experts (one more group of
        # the routed launches), with 256-row tiles and whole 256-column down
        # tiles: the persistent down projection's shared-expert rows
        LayerConfig("mini_bf16_shared_prefill", T=800, H=512, F=384, E=8, k=2, Fs=384, seed=16),
        LayerConfig("mini_fp8_decode", T=20, H=384, F=256, E=16, k=4, Fs=256, w="fp8", seed=5),
        LayerConfig("mini_fp8_prefill", T=520, H=512, F=384, E=16, k=4, Fs=384, w="fp8", seed=6),
        # down projection over several 256-column tiles (H = 11 x 128: a
        # half tile at the end) with an even count of 128-deep K blocks
        LayerConfig("mini_fp8_wide", T=640, H=1408, F=512, E=16, k=4, Fs=512, w="fp8", seed=8),
        # bf16 shared expert beside fp8 routed experts: as wide as the routed
        # experts (decode), and narrower, ragged against the tiles (prefill)
        LayerConfig("mini_fp8_bf16s_decode", T=20, H=384, F=256, E=16, k=4, Fs=256, w="fp8", ws="bf16",
                    seed=9),
        LayerConfig("mini_fp8_bf16s_prefill", T=520, H=512, F=384, E=16, k=4, Fs=160, w="fp8", ws="bf16",
                    seed=10),
        # fp32 gate beside bf16 tokens, few tokens and many (where a bf16
        # gate would take the tiled router)
        LayerConfig("mini_bf16_f32gate_decode", T=13, H=544, F=672, E=8, k=2, wg="f32", seed=11),
        LayerConfig("mini_fp8_f32gate_prefill", T=600, H=512, F=384, E=16, k=4, Fs=384, w="fp8", wg="f32",
                    seed=12),
        # MXFP4 experts: ragged K splits and N tails (F = 352 = 5.5 slices),
        # and with an MXFP4 shared expert in the routed launch
        LayerConfig("mini_mxfp4_decode", T=13, H=544, F=352, E=8, k=2, w="mxfp4", seed=13),
        LayerConfig("mini_mxfp4_shared", T=40, H=384, F=256, E=16, k=4, Fs=256, w="mxfp4", seed=14),
        # prefill-sized MXFP4 (tiled after decoding), with a wider MXFP4 shared
        # expert in launches of its own
        LayerConfig("mini_mxfp4_prefill", T=256, H=384, F=256, E=8, k=2, Fs=512, w="mxfp4", seed=15),
    ]
}


def get_config(name: str) -> LayerConfig:
    if name in CONFIGS:
        return CONFIGS[name]
    if name in MINI_CONFIGS:
        return MINI_CONFIGS[name]
    raise KeyError(f"unknown layer config {name!r}")
