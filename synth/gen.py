"""Seeded synthetic inputs for one MoE layer.

Every tensor has its own seeded torch generator, so any expert's weights can be
drawn on its own and on the device that will hold them. The values are drawn
once, in float32, and then stored in the layer's storage dtype; the stored
values (bf16 numbers, or fp8 codes plus fp32 block scales) are the canonical
inputs that both the HIP path and the oracle consume.

Distributions: token rows X ~ N(0, x_std^2); gate and expert weights
~ N(0, w_std^2) (standard deviation w_std). For the hot-expert workload the gate
carries the bias b[e] = -s*ln(e+1), which adds log-Zipf(s) offsets to the
expert scores (the Zipf normaliser is a constant shift and cancels in softmax).

The fp8 storage format is OCP E4M3 ("e4m3fn": bias 7, largest finite 448, no
infinities) with one fp32 scale per 128x128 block: s = amax/448 (1 when the
block is all zero) and code = round-to-nearest-even(w/s), saturated to +-448.
This is the storage format of the synthetic weights, not a step of the layer.
"""
from __future__ import annotations

import hashlib

import torch

from .configs import LayerConfig

_E4M3_MAX = 448.0
_BLOCK = 128

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def tensor_seed(cfg: LayerConfig, name: str, *idx: int) -> int:
    """Stable 63-bit seed for one tensor (or one expert of a tensor)."""
    key = "/".join([str(cfg.seed), cfg.name, name] + [str(i) for i in idx])
    digest = hashlib.blake2b(key.encode(), digest_size=8).digest()
    return int.from_bytes(digest, "little") & ((1 << 63) - 1)


def _normal(cfg: LayerConfig, name: str, shape, std: float, device, *idx: int) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(tensor_seed(cfg, name, *idx))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x


def quantize_e4m3_blocks(w: torch.Tensor):
    """Store a float32 matrix [R, C] as E4M3 codes with 128x128 fp32 scales.

    Returns (codes uint8 [R, C], scales float32 [R/128, C/128]).
    """
    R, C = w.shape
    if R % _BLOCK or C % _BLOCK:
        raise ValueError(f"fp8 block storage needs dims divisible by {_BLOCK}, got {R}x{C}")
    w = w.to(torch.float32)
    blk = w.reshape(R // _BLOCK, _BLOCK, C // _BLOCK, _BLOCK)
    amax = blk.abs().amax(dim=(1, 3))
    scale = amax / _E4M3_MAX
    scale = torch.where(amax == 0, torch.ones_like(scale), scale)
    q = blk / scale[:, None, :, None]
    q = q.clamp(-_E4M3_MAX, _E4M3_MAX)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(R, C)
    return codes.contiguous(), scale.contiguous()


# magnitudes of the OCP FP4 E2M1 codes 0..7 (a code's sign is bit 3)
_E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
_MX_BLOCK = 32


def quantize_mxfp4(w: torch.Tensor):
    """Store a float32 matrix [K, N] as MXFP4: E2M1 codes with one E8M0 scale
    per 32 consecutive K rows of a column.

    Per block: shared exponent floor(log2(amax)) - 2 (2 is E2M1's largest
    exponent), clamped to the E8M0 range; each value divided by the scale goes
    to the nearest E2M1 magnitude, ties to the even code, saturating at 6 (a
    zero block gets the scale 1). Returns (packed uint8 [K/2, N], byte (i, n)
    holding rows 2i (low nibble) and 2i + 1 (high nibble) of column n; scales
    uint8 [K/32, N] as E8M0 codes).
    """
    K, N = w.shape
    if K % _MX_BLOCK:
        raise ValueError("MXFP4 needs K to be a multiple of 32")
    w64 = w.to(torch.float64)
    blk = w64.reshape(K // _MX_BLOCK, _MX_BLOCK, N)
    amax = blk.abs().amax(dim=1)
    e = torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 2.0
    e = torch.where(amax > 0, e, torch.zeros_like(e)).clamp(-127.0, 127.0)
    scale_codes = (e + 127.0).to(torch.uint8)
    x = blk / torch.exp2(e)[:, None, :]
    mags = torch.tensor(_E2M1_MAG, dtype=torch.float64, device=w.device)
    d = (x.abs()[..., None] - mags).abs()
    # exact midpoints go to the even code (its mantissa bit clear)
    d = d + (torch.arange(8, device=w.device) % 2).to(torch.float64) * 1e-12
    code = d.argmin(dim=-1).to(torch.uint8)
    code = code | torch.where(x < 0, 8, 0).to(torch.uint8)
    code = code.reshape(K, N)
    packed = (code[0::2] | (code[1::2] << 4)).contiguous()
    return packed, scale_codes.contiguous()


def _store(w32: torch.Tensor, wdt: str):
    """Cast a float32 weight matrix to its storage format."""
    if wdt == "fp8":
        return quantize_e4m3_blocks(w32)
    if wdt == "mxfp4":
        return quantize_mxfp4(w32)
    return w32.to(_DTYPES[wdt]).contiguous(), None


def _expert_stack(cfg: LayerConfig, name: str, n: int, rows: int, cols: int, device):
    """[n, rows, cols] expert weights (+ [n, rows/128, cols/128] scales for fp8;
    MXFP4: [n, rows/2, cols] packed codes and [n, rows/32, cols] E8M0 scales)."""
    if cfg.w == "fp8":
        W = torch.empty((n, rows, cols), dtype=torch.uint8, device=device)
        S = torch.empty((n, rows // _BLOCK, cols // _BLOCK), dtype=torch.float32, device=device)
    elif cfg.w == "mxfp4":
        W = torch.empty((n, rows // 2, cols), dtype=torch.uint8, device=device)
        S = torch.empty((n, rows // _MX_BLOCK, cols), dtype=torch.uint8, device=device)
    else:
        W = torch.empty((n, rows, cols), dtype=_DTYPES[cfg.w], device=device)
        S = None
    for e in range(n):
        w32 = _normal(cfg, name, (rows, cols), cfg.w_std, device, e)
        q, s = _store(w32, cfg.w)
        W[e].copy_(q)
        if S is not None:
            S[e].copy_(s)
        del w32, q, s
    return W, S


def gate_bias(cfg: LayerConfig, device="cpu"):
    """Log-Zipf(s) per-expert offsets, or None when the workload has none."""
    if cfg.zipf_s <= 0:
        return None
    e = torch.arange(cfg.E, dtype=torch.float64)
    return (-cfg.zipf_s * torch.log1p(e)).to(torch.float32).to(device)


def make_layer(cfg: LayerConfig, device="cpu", experts: bool = True) -> dict:
    """Draw one layer's inputs on `device`.

    Keys: X [T,H]; Wg [H,E]; gate_bias [E] or None; W1, W3 [E,H,F]; W2 [E,F,H];
    S1, S3 [E,H/128,F/128], S2 [E,F/128,H/128] (fp8 only, else None); and for a
    shared expert Ws1, Ws3 [H,Fs], Ws2 [Fs,H] with Ss1, Ss3, Ss2.
    With experts=False only X, Wg and gate_bias are drawn.
    """
    act = _DTYPES[cfg.act]
    out = {"cfg": cfg}
    out["X"] = _normal(cfg, "X", (cfg.T, cfg.H), cfg.x_std, device).to(act).contiguous()
    out["Wg"] = _normal(cfg, "Wg", (cfg.H, cfg.E), cfg.w_std, device).to(_DTYPES[cfg.wg or cfg.act]).contiguous()
    out["gate_bias"] = gate_bias(cfg, device)
    if not experts:
        return out
    out["W1"], out["S1"] = _expert_stack(cfg, "W1", cfg.E, cfg.H, cfg.F, device)
    out["W3"], out["S3"] = _expert_stack(cfg, "W3", cfg.E, cfg.H, cfg.F, device)
    out["W2"], out["S2"] = _expert_stack(cfg, "W2", cfg.E, cfg.F, cfg.H, device)
    if cfg.Fs > 0:
        for name, r, c in (("Ws1", cfg.H, cfg.Fs), ("Ws3", cfg.H, cfg.Fs), ("Ws2", cfg.Fs, cfg.H)):
            w, s = _store(_normal(cfg, name, (r, c), cfg.w_std, device), cfg.shared_w)
            out[name] = w
            out["S" + name[1:]] = s
    else:
        for name in ("Ws1", "Ws3", "Ws2", "Ss1", "Ss3", "Ss2"):
            out[name] = None
    return out


def redraw_rows(cfg: LayerConfig, X: torch.Tensor, rows, attempt: int) -> None:
    """Replace token rows of X in place with fresh draws from per-row substreams."""
    for t in rows:
        t = int(t)
        x = _normal(cfg, "X-redraw", (cfg.H,), cfg.x_std, X.device, t, attempt)
        X[t].copy_(x.to(X.dtype))


def spread_block_scales(d: dict, seed: int, lo: int = -4, hi: int = 4) -> dict:
    """A copy of layer `d` whose fp32 128x128 block scales (S1, S3, S2 and the
    shared expert's Ss1, Ss3, Ss2) are each multiplied by a seeded power of two
    2^u, u uniform in [lo, hi]. The E4M3 codes are unchanged, so the stored
    weights stay exact; blocks then differ in scale by up to 2^(hi - lo), and a
    weight read with another block's scale is far off."""
    out = dict(d)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    for key in ("S1", "S3", "S2", "Ss1", "Ss3", "Ss2"):
        s = d.get(key)
        if s is None or s.dtype != torch.float32:
            continue
        u = torch.randint(lo, hi + 1, tuple(s.shape), generator=g).to(torch.float32)
        out[key] = (s * torch.exp2(u).to(s.device)).contiguous()
    return out

