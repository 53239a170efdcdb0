"""fp64 reference for the MoE layer forward (test infrastructure only).

Each function is the plain definition of one step, in the pages' order:
router scores -> softmax -> top-k -> renormalise -> group assignments by expert
(counts, offsets, stable permutation, inverse map) -> per-expert SwiGLU FFN ->
combine (unpermute, weight, sum) [+ shared expert].

Inputs are the canonical stored values (f32 / bf16 numbers, E4M3 codes with
fp32 block scales, or MXFP4 codes with E8M0 scales); they are upcast exactly to
float64 and every step runs in float64. Nothing here is blocked, fused or reordered beyond what each
definition states.
"""
from __future__ import annotations

import numpy as np

try:  # torch is only used as a container for the canonical inputs
    import torch
except ImportError:  # pragma: no cover
    torch = None


# ----------------------------------------------------------------------------
# Canonical values
# ----------------------------------------------------------------------------

def to_f64(x) -> np.ndarray:
    """Exact float64 copy of a float tensor/array (f32 and bf16 embed exactly)."""
    if torch is not None and isinstance(x, torch.Tensor):
        if x.dtype == torch.uint8:
            raise TypeError("uint8 tensors are fp8 codes: use dequant_blocks")
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """OCP E4M3 ("e4m3fn") code -> float64, from the format definition.

    Bit layout s|eeee|mmm, exponent bias 7. Exponent field 0 encodes subnormals
    m * 2^-9; exponent field 15 with mantissa 7 is NaN (no infinities); every
    other code is (-1)^s * (1 + m/8) * 2^(e-7). Largest finite value 448.
    FP8 storage of expert weights is the format the page "MoE-推理部署" names in
    its expert-quantisation section.
    """
    if torch is not None and isinstance(codes, torch.Tensor):
        codes = codes.detach().to("cpu").numpy()
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    sub = m.astype(np.float64) * 2.0 ** -9
    nor = (1.0 + m.astype(np.float64) / 8.0) * np.exp2((e - 7).astype(np.float64))
    val = sign * np.where(e == 0, sub, nor)
    return np.where((e == 15) & (m == 7), np.nan, val)


_E4M3_TABLE = None


def _e4m3_table() -> np.ndarray:
    """The 256 decoded E4M3 values (e4m3_decode of every code), tabulated once."""
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        _E4M3_TABLE = e4m3_decode(np.arange(256, dtype=np.uint8))
    return _E4M3_TABLE


def dequant_blocks(codes, scales, block: int = 128) -> np.ndarray:
    """W[r, c] = decode(code[r, c]) * scale[r // block, c // block], in float64.

    Every E4M3 value times an fp32 scale is exact in float64 (4 + 24 significand
    bits), so this is the exact value of the stored weight. The scales are per
    expert and per 128x128 block, the per-expert granularity the page
    "MoE-推理部署" asks for in its expert-quantisation section.
    """
    if torch is not None and isinstance(codes, torch.Tensor):
        codes = codes.detach().to("cpu").numpy()
    q = _e4m3_table()[np.asarray(codes, dtype=np.uint8)]
    s = to_f64(scales)
    R, C = q.shape
    q = q.reshape(R // block, block, C // block, block)
    return (q * s[:, None, :, None]).reshape(R, C)


def _u8(x) -> np.ndarray:
    if torch is not None and isinstance(x, torch.Tensor):
        x = x.detach().to("cpu").numpy()
    return np.asarray(x, dtype=np.uint8)


def e2m1_decode(codes) -> np.ndarray:
    """OCP FP4 E2M1 code (low 4 bits) -> float64, from the format definition.

    Bit layout s|ee|m, exponent bias 1. Exponent field 0 encodes the subnormals
    m * 2^-1; every other code is (-1)^s * (1 + m/2) * 2^(e-1). No infinities
    or NaN; largest magnitude 6. MXFP4 is one of the expert-weight formats the
    page "MoE-推理部署" names for single-GPU serving.
    """
    c = _u8(codes) & 0xF
    s = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e.astype(np.float64) - 1.0))
    return s * mag


def e8m0_decode(codes) -> np.ndarray:
    """OCP E8M0 scale code -> float64: 2^(e - 127), code 255 is NaN."""
    e = _u8(codes).astype(np.float64)
    return np.where(e == 255.0, np.nan, np.exp2(e - 127.0))


def dequant_mxfp4(packed, scales, block: int = 32) -> np.ndarray:
    """MXFP4 weights [K, N] in float64 from packed codes [K/2, N] and E8M0
    scales [K/block, N].

    Byte (i, n) holds column n's rows 2i (low nibble) and 2i + 1 (high nibble),
    so the two values of a byte share one scale; every `block` consecutive K
    rows of a column share one scale (the microscaling block runs along the
    reduction dimension). An E2M1 value times a power of two is exact in
    float64, so this is the exact stored weight.
    """
    b = _u8(packed)
    K2, N = b.shape
    q = np.empty((2 * K2, N), dtype=np.float64)
    q[0::2] = e2m1_decode(b & 0xF)
    q[1::2] = e2m1_decode(b >> 4)
    sc = e8m0_decode(scales)
    return q * np.repeat(sc, block, axis=0)[: 2 * K2]


def e4m3_encode(x) -> np.ndarray:
    """float -> OCP E4M3 code: the representable value nearest to x, ties to
    the code with an even mantissa (its lowest bit clear), magnitudes at or
    above the largest finite value 448 saturating to it; the sign bit is x's
    (so -0.0 -> 0x80). NaN -> 0x7f. From the format definition in
    `e4m3_decode`; the decoded values are searched, nothing is computed by
    bit manipulation.
    """
    x = np.asarray(x, dtype=np.float64)
    pos_codes = np.arange(0x7f, dtype=np.int64)          # 0x00..0x7e: the finite non-negative codes
    pos_vals = _e4m3_table()[pos_codes]                   # ascending
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(pos_vals, a, side="left"), 0, pos_codes.size - 1)
    lo = np.clip(hi - 1, 0, pos_codes.size - 1)
    d_lo, d_hi = a - pos_vals[lo], pos_vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (pos_codes[hi] % 2 == 0))
    code = np.where(pick_hi, pos_codes[hi], pos_codes[lo])
    code = np.where(np.signbit(x), code | 0x80, code)
    return np.where(np.isnan(x), 0x7f, code).astype(np.uint8)


def quantize_rows_e4m3(x, group: int = 128):
    """Activation quantisation before expert compute (page "MOE推理流程解析"
    §三 names the choice of quantising activations before dispatch or just
    before the expert GEMM; both give these values for per-row scales).

    Per row and `group`-column block, in float32 as a kernel would compute it:
    amax = max |x|, s = amax / 448 (s = 1 when amax = 0), q = E4M3(x / s)
    (round to nearest even, saturating). Returns (codes uint8 [R, C], scales
    float32 [R, C / group]).
    """
    x32 = np.asarray(to_f64(x), dtype=np.float32)
    R, C = x32.shape
    xg = x32.reshape(R, C // group, group)
    amax = np.abs(xg).max(axis=2)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = e4m3_encode((xg / s[:, :, None]).astype(np.float32)).reshape(R, C)
    return q, s


def dequant_rows(codes, scales, group: int = 128) -> np.ndarray:
    """x[r, c] = decode(code[r, c]) * scale[r, c // group], exact in float64."""
    q = _e4m3_table()[np.asarray(codes, dtype=np.uint8)]
    s = np.asarray(scales, dtype=np.float64)
    R, C = q.shape
    return (q.reshape(R, C // group, group) * s[:, :, None]).reshape(R, C)


def round_bf16(x) -> np.ndarray:
    """float64 -> float32 -> bfloat16 value, each rounding to nearest even
    (bfloat16: the float32 bit pattern's upper 16 bits, rounded on the lower
    16 with ties to an even upper half). NaN stays NaN."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    out = u.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isnan(f), np.nan, out)


def _act_quant(x) -> np.ndarray:
    """x rounded through quantize_rows_e4m3 and back (float64)."""
    q, s = quantize_rows_e4m3(np.asarray(x, dtype=np.float64).astype(np.float32))
    return dequant_rows(q, s)


# ----------------------------------------------------------------------------
# Router: page "MoE serving production quirks", memory-paradox section (linear
# projection and softmax over all experts); page "MOE推理流程解析" §三 (top-k
# keeps the selected indices and their weights) and §九 (kept weights are
# renormalised).
# ----------------------------------------------------------------------------

def router_logits(X, Wg, gate_bias=None) -> np.ndarray:
    """logits[t, e] = sum_h X[t, h] * Wg[h, e] (+ b[e]), float64."""
    logits = to_f64(X) @ to_f64(Wg)
    if gate_bias is not None:
        logits = logits + to_f64(gate_bias)[None, :]
    return logits


def softmax(logits) -> np.ndarray:
    """Row softmax with the row maximum subtracted, float64."""
    z = np.asarray(logits, dtype=np.float64)
    z = z - z.max(axis=1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=1, keepdims=True)


def select_topk(logits, k: int) -> np.ndarray:
    """Indices of the k largest scores per token, best first; a tie goes to the
    lower expert index. Comparisons happen in the dtype of `logits` (pass the
    fp32 logits of another implementation to take the same decision it took).
    Softmax is monotone, so the k largest logits are the k largest
    probabilities.
    """
    L = np.asarray(logits)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    idx = np.empty((T, k), dtype=np.int64)
    experts = np.arange(E)
    for t in range(T):
        # primary key: score, descending; secondary key: expert index, ascending
        order = np.lexsort((experts, -L[t].astype(np.float64)))
        idx[t] = order[:k]
    return idx


def routing_weights(logits, idx) -> np.ndarray:
    """w[t, j] = p[t, idx[t, j]] / sum_j' p[t, idx[t, j']] with p = softmax over
    all E experts (float64)."""
    p = softmax(logits)
    sel = np.take_along_axis(p, np.asarray(idx), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route(X, Wg, gate_bias, k: int):
    """Returns (logits [T,E], idx [T,k], w [T,k]) in float64 / int64."""
    logits = router_logits(X, Wg, gate_bias)
    idx = select_topk(logits, k)
    return logits, idx, routing_weights(logits, idx)


# ----------------------------------------------------------------------------
# Dispatch on one GPU: page "MOE推理流程解析" §二 (T*k assignments grouped into
# per-expert matrices; the token id stays beside each row) and §三 (the
# permutation writes rows in expert order and records an inverse map).
# ----------------------------------------------------------------------------

def permute(idx, E: int):
    """Group the T*k assignments a = t*k + j by expert.

    counts[e]     = number of assignments with expert e
    offsets[e]    = sum of counts[:e]  (offsets[E] = T*k)
    row_src[r]    = assignment held by row r; rows of expert e are
                    offsets[e] .. offsets[e+1]-1, in ascending assignment order
    assign_row[a] = row holding assignment a (inverse of row_src)
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    A = flat.size
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    row_src = np.argsort(flat, kind="stable").astype(np.int64)
    assign_row = np.empty(A, dtype=np.int64)
    assign_row[row_src] = np.arange(A)
    return counts, offsets, row_src, assign_row


# ----------------------------------------------------------------------------
# Expert FFN: page "MOE推理流程解析" §三 (each expert applies its activation and
# output projection). SwiGLU form: h = silu(x W1) * (x W3), y = h W2.
# ----------------------------------------------------------------------------

def silu(z):
    """silu(z) = z / (1 + exp(-z)) (float64). For z below about -709 exp(-z)
    overflows to inf and the quotient is -0, the function's limit."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(x, W1, W3, W2, act_quant: bool = False) -> np.ndarray:
    """y = (silu(x @ W1) * (x @ W3)) @ W2 for rows x [n, H].

    act_quant (diagnosis only: the exact result is the reference): x and h
    pass through E4M3 activation quantisation (`quantize_rows_e4m3`) before
    their projections, as a W8A8 kernel computes; h is first stored in
    bfloat16 (the intermediate's storage precision), so its codes are decided
    on the values the kernel quantises.
    """
    x = np.asarray(x, dtype=np.float64)
    if act_quant:
        x = _act_quant(x)
    h = silu(x @ W1) * (x @ W3)
    if act_quant:
        h = _act_quant(round_bf16(h))
    return h @ W2


def grouped_ffn(Xrows, offsets, expert, act_quant: bool = False) -> np.ndarray:
    """Yp[r] = FFN_e(Xrows[r]) for the rows r of each group e.

    `expert(e)` returns (W1, W3, W2) as float64 arrays. Groups with no rows are
    skipped (their weights are never touched). `act_quant`: see swiglu_ffn.
    """
    Xrows = np.asarray(Xrows, dtype=np.float64)
    offsets = np.asarray(offsets)
    G = offsets.size - 1
    Yp = None
    for e in range(G):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        W1, W3, W2 = expert(e)
        y = swiglu_ffn(Xrows[lo:hi], W1, W3, W2, act_quant)
        if Yp is None:
            Yp = np.zeros((Xrows.shape[0], y.shape[1]), dtype=np.float64)
        Yp[lo:hi] = y
    if Yp is None:
        Yp = np.zeros((Xrows.shape[0], 0), dtype=np.float64)
    return Yp


# ----------------------------------------------------------------------------
# Combine: page "MOE推理流程解析" §二 (each contribution times its routing
# weight, summed per token) and §三 (the inverse map restores token order).
# ----------------------------------------------------------------------------

def combine(Yp, assign_row, w, T: int, k: int, S=None) -> np.ndarray:
    """Y[t] = sum_{j<k} w[t,j] * Yp[assign_row[t*k+j]] (+ S[t]), j ascending."""
    Yp = np.asarray(Yp, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64).reshape(T, k)
    assign_row = np.asarray(assign_row).reshape(T, k)
    Y = np.zeros((T, Yp.shape[1]), dtype=np.float64)
    for j in range(k):
        Y += w[:, j:j + 1] * Yp[assign_row[:, j]]
    if S is not None:
        Y = Y + np.asarray(S, dtype=np.float64)
    return Y


# ----------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------

class Layer:
    """Read-only view of one layer's canonical inputs, upcast on demand.

    `d` holds torch tensors (any device) or numpy arrays under the keys X, Wg,
    gate_bias, W1, W3, W2, S1, S3, S2 (scales only for fp8 codes) and,
    optionally, the shared expert Ws1, Ws3, Ws2, Ss1, Ss3, Ss2. Experts are
    converted one at a time so model-sized weights never sit in RAM as float64
    all at once.
    """

    def __init__(self, d: dict, k: int):
        self.d = d
        self.k = int(k)
        self.E = int(d["W1"].shape[0])
        self.T, self.H = (int(s) for s in d["X"].shape)

    def X(self):
        return to_f64(self.d["X"])

    def Wg(self):
        return to_f64(self.d["Wg"])

    def gate_bias(self):
        b = self.d.get("gate_bias")
        return None if b is None else to_f64(b)

    def _mat(self, wkey, skey, e=None):
        W = self.d[wkey] if e is None else self.d[wkey][e]
        S = self.d.get(skey)
        if S is not None:
            S = S if e is None else S[e]
            # E8M0 byte scales mark MXFP4 codes, fp32 scales E4M3 codes
            if getattr(S, "dtype", None) in (np.uint8,) or (torch is not None and getattr(S, "dtype", None) == torch.uint8):
                return dequant_mxfp4(W, S)
            return dequant_blocks(W, S)
        return to_f64(W)

    def expert(self, e: int):
        return (self._mat("W1", "S1", e), self._mat("W3", "S3", e), self._mat("W2", "S2", e))

    def has_shared(self) -> bool:
        return self.d.get("Ws1") is not None

    def shared_is_fp8(self) -> bool:
        """The shared expert is stored as E4M3 codes with block scales (it may
        instead be bf16 beside fp8 routed experts)."""
        return self.d.get("Ss1") is not None

    def shared(self):
        return (self._mat("Ws1", "Ss1"), self._mat("Ws3", "Ss3"), self._mat("Ws2", "Ss2"))


def forward(layer: Layer) -> dict:
    """Full fp64 forward. Returns every intermediate of the pages' pipeline."""
    X = layer.X()
    T, k, E = layer.T, layer.k, layer.E
    logits, idx, w = route(X, layer.Wg(), layer.gate_bias(), k)
    counts, offsets, row_src, assign_row = permute(idx, E)
    Xp = X[row_src // k]
    Yp = grouped_ffn(Xp, offsets, layer.expert)
    S = swiglu_ffn(X, *layer.shared()) if layer.has_shared() else None
    Y = combine(Yp, assign_row, w, T, k, S)
    return dict(logits=logits, idx=idx, w=w, counts=counts, offsets=offsets,
                row_src=row_src, assign_row=assign_row, Xp=Xp, Yp=Yp, S=S, Y=Y)


def forward_tokens(layer: Layer, tokens, idx=None, act_quant: bool = False, workers: int = 1) -> dict:
    """fp64 outputs for a subset of tokens only (the layer is per-token
    independent: each token's output depends on its own row, its own routing
    and the shared weights). `idx` optionally fixes the routing decision
    (rows for the sampled tokens) instead of re-deriving it. `act_quant`
    mirrors activation quantisation in the expert FFNs (see swiglu_ffn).
    `workers` > 1 evaluates the chosen experts on that many threads: each
    expert fills its own (token, slot) entries of y with the same
    expressions, so the result does not depend on it.
    Returns logits, idx, w, per-token expert outputs y[t, j] and Y for the
    sampled tokens, in the given order.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    X = layer.X()[tokens]
    logits = router_logits(X, layer.Wg(), layer.gate_bias())
    if idx is None:
        idx = select_topk(logits, layer.k)
    idx = np.asarray(idx, dtype=np.int64).reshape(len(tokens), layer.k)
    w = routing_weights(logits, idx)
    n = len(tokens)
    y = np.zeros((n, layer.k, layer.H), dtype=np.float64)

    def one_expert(e):
        W1, W3, W2 = layer.expert(int(e))
        ts, js = np.nonzero(idx == e)
        y[ts, js] = swiglu_ffn(X[ts], W1, W3, W2, act_quant)

    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one_expert, np.unique(idx)))
    else:
        for e in np.unique(idx):
            one_expert(e)
    Y = np.einsum("tj,tjh->th", w, y)
    S = None
    if layer.has_shared():
        # activation quantisation belongs to the W8A8 form of fp8 experts: a
        # bf16 shared expert is mirrored without it
        S = swiglu_ffn(X, *layer.shared(), act_quant and layer.shared_is_fp8())
        Y = Y + S
    return dict(tokens=tokens, logits=logits, idx=idx, w=w, y=y, S=S, Y=Y)
