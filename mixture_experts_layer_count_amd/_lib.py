"""ctypes binding of libmoe (include/moe.h).

Argument marshalling only: torch tensors provide device memory and the HIP
stream; every computation runs in libmoe's HIP kernels. The library must be
built (python -m mixture_experts_layer_count_amd.build); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

(MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP,
 MOE_ERR_SCRATCH_LIMIT) = range(6)
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4 = 0, 1, 2, 3
PATHS = {"auto": 0, "gemv": 1, "tiled": 2, "tiled_a8": 3}
# bits of moe_debug_bounds() (the bounds-checked build)
(MOE_BOUNDS_TILE, MOE_BOUNDS_A_ROW, MOE_BOUNDS_SCALE_ROW, MOE_BOUNDS_TAIL_SLOT, MOE_BOUNDS_PERM_ROW,
 MOE_BOUNDS_COMBINE_ROW, MOE_BOUNDS_QUANT_ROW, MOE_BOUNDS_EP_ROW) = (1 << i for i in range(8))

# Every function include/moe.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_route_workspace_bytes": (_SZ, [_I, _I, _I]),
    "moe_route": (_I, [_P, _I, _P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute_workspace_bytes": (_SZ, [_I, _I, _I]),
    "moe_permute": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _P, _I, _I, _P, _P, _SZ, _P]),
    "moe_grouped_ffn_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "moe_grouped_ffn": (_I, [_P, _P, _I, _I, _P, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _I, _P, _I,
                             _P, _SZ, _P]),
    "moe_quantize_e4m3_rows": (_I, [_P, _I, ctypes.c_longlong, _P, _I, _I, _I, _P, _P, _P]),
    "moe_combine": (_I, [_P, _P, _P, _I, _I, _I, _P, _I, _P, _P]),
    "moe_forward_workspace_bytes": (_SZ, [_P, _I]),
    "moe_forward": (_I, [_P, _P, _I, _P, _P, _SZ, _P, _P, _P, _P, _P, _P]),
    "moe_forward_noalloc_max_bytes": (_SZ, []),
    "moe_ep_dispatch_workspace_bytes": (_SZ, [_I, _I, _I]),
    "moe_ep_dispatch": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_ep_recv_offsets": (_I, [_P, _I, _P, _P]),
    "moe_ep_exchange": (_I, [_I, _P, ctypes.c_longlong, _P, _P, ctypes.c_longlong, _P, ctypes.c_longlong, _P, _I,
                             _I, _P]),
    "moe_ep_local_experts": (_I, [_P, _I, _I, _I, _I, _P, _P]),
    "moe_forward_noalloc": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _P, _P]),
    "moe_debug_bounds": (ctypes.c_uint, []),
}


class LayerDesc(ctypes.Structure):
    """Mirror of moe_layer_desc."""
    _fields_ = [
        ("H", _I), ("F", _I), ("E", _I), ("k", _I), ("Fs", _I),
        ("act_dt", _I), ("w_dt", _I), ("path", _I),
        ("Wg", _P), ("gate_bias", _P),
        ("W1", _P), ("W3", _P), ("W2", _P),
        ("S1", _P), ("S3", _P), ("S2", _P),
        ("Ws1", _P), ("Ws3", _P), ("Ws2", _P),
        ("Ss1", _P), ("Ss3", _P), ("Ss2", _P),
        ("ws_dt", _I), ("gate_f32", _I),
    ]


# the bounds-checked debug build of the same sources (-DMOE_BOUNDS_CHECK)
DEBUG_LIB_PATH = os.path.join(PKG, "libmoe_debug.so")

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """A handle on a built libmoe (release or debug) with every signature set."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m mixture_experts_layer_count_amd.build`")
    h = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(h, name)
        fn.restype = res
        fn.argtypes = args
    return h


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


class use_library:
    """Context manager: route every call of this binding to another libmoe
    handle (the bounds-checked build) inside the block."""

    def __init__(self, handle: ctypes.CDLL):
        self.handle, self.saved = handle, None

    def __enter__(self):
        global _lib
        self.saved, _lib = lib(), self.handle
        return self.handle

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().moe_status_string(status).decode()
        super().__init__(f"{fn}: {msg}")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoEError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def act_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"activation dtype must be float32 or bfloat16, got {t.dtype}")


def weight_dtype(t: torch.Tensor, scales=None) -> int:
    """uint8 codes with uint8 (E8M0) scales are MXFP4, with fp32 scales E4M3."""
    if t.dtype == torch.uint8 and scales is not None and scales.dtype == torch.uint8:
        return MOE_MXFP4
    if t.dtype == torch.uint8 or t.dtype == torch.float8_e4m3fn:
        return MOE_FP8_E4M3
    return act_dtype(t)


def _expert_dims(W1: torch.Tensor, wdt: int):
    """(experts, H, F) of W1: MXFP4 stores two K rows a byte ([E, H/2, F])."""
    G, K, F = W1.shape
    return G, (2 * K if wdt == MOE_MXFP4 else K), F


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libmoe takes device tensors")
        if not t.is_contiguous():
            raise ValueError("libmoe takes contiguous tensors")


def _i32(t):
    if t is not None and t.dtype != torch.int32:
        raise TypeError(f"expected int32 tensor, got {t.dtype}")
    return t


def route(X, Wg, k: int, gate_bias=None):
    """-> (logits [T,E] f32, topk_idx [T,k] i32, topk_w [T,k] f32)."""
    _dev(X, Wg, gate_bias)
    T, H = X.shape
    E = Wg.shape[1]
    logits = torch.empty((T, E), dtype=torch.float32, device=X.device)
    idx = torch.empty((T, k), dtype=torch.int32, device=X.device)
    w = torch.empty((T, k), dtype=torch.float32, device=X.device)
    nbytes = lib().moe_route_workspace_bytes(T, H, E)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=X.device)
    # the gate in X's dtype, or fp32 beside bf16 tokens (higher-precision router)
    _check("moe_route", lib().moe_route(_ptr(X), act_dtype(X), _ptr(Wg), act_dtype(Wg), _ptr(gate_bias), T, H, E, k,
                                        _ptr(logits), _ptr(idx), _ptr(w), _ptr(ws), nbytes, _stream()))
    return logits, idx, w


def permute(topk_idx, E: int, X=None, assign_row=None):
    """-> (counts [E], offsets [E+1], row_src [A], assign_row [A], Xp [A,H] or None).
    `assign_row`: optional int32 [A] output buffer."""
    _dev(topk_idx, X, assign_row)
    _i32(topk_idx)
    T, k = topk_idx.shape
    dev = topk_idx.device
    A = T * k
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_src = torch.empty(A, dtype=torch.int32, device=dev)
    if assign_row is None:
        assign_row = torch.empty(A, dtype=torch.int32, device=dev)
    elif assign_row.numel() != A or assign_row.dtype != torch.int32:
        raise ValueError("assign_row must be int32 with T*k elements")
    Xp = None
    H, xdt = 0, MOE_F32
    if X is not None:
        H = X.shape[1]
        xdt = act_dtype(X)
        Xp = torch.empty((A, H), dtype=X.dtype, device=dev)
    nbytes = lib().moe_permute_workspace_bytes(T, k, E)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check("moe_permute", lib().moe_permute(_ptr(topk_idx), T, k, E, _ptr(counts), _ptr(offsets),
                                            _ptr(row_src), _ptr(assign_row), _ptr(X), xdt, H, _ptr(Xp),
                                            _ptr(ws), nbytes, _stream()))
    return counts, offsets, row_src, assign_row, Xp


def grouped_ffn(Xin, offsets, W1, W3, W2, S1=None, S3=None, S2=None, row_src=None, k: int = 1,
                M: int | None = None, path: str = "auto", out=None):
    """Yp [M,H] = per-group SwiGLU FFN of the input rows (see moe_grouped_ffn).
    `out`: optional [M,H] output buffer."""
    _dev(Xin, offsets, W1, W3, W2, S1, S3, S2, row_src, out)
    _i32(offsets)
    _i32(row_src)
    adt, wdt = act_dtype(Xin), weight_dtype(W1, S1)
    G, H, F = _expert_dims(W1, wdt)
    if M is None:
        M = row_src.numel() if row_src is not None else Xin.shape[0]
    if out is None:
        Yp = torch.empty((M, H), dtype=Xin.dtype, device=Xin.device)
    elif tuple(out.shape) != (M, H) or out.dtype != Xin.dtype:
        raise ValueError("out must be [M, H] in the activation dtype")
    else:
        Yp = out
    p = PATHS[path]
    nbytes = lib().moe_grouped_ffn_workspace_bytes(M, G, H, F, adt, wdt, p)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=Xin.device)
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(
        _ptr(Xin), _ptr(row_src), k, M, _ptr(offsets), G, H, F, _ptr(W1), _ptr(W3), _ptr(W2), wdt,
        _ptr(S1), _ptr(S3), _ptr(S2), adt, _ptr(Yp), p, _ptr(ws), nbytes, _stream()))
    return Yp


def quantize_e4m3_rows(X, row_src=None, k: int = 1, R: int | None = None):
    """E4M3 codes [R, C] (uint8) and fp32 scales [R, C/128] of bf16 rows
    X[row_src[r] // k] (X[r] without row_src), per 128-column group."""
    _dev(X, row_src)
    if row_src is not None:
        _i32(row_src)
    R = (row_src.numel() if row_src is not None else X.shape[0]) if R is None else R
    C = X.shape[1]
    Q = torch.empty((R, C), dtype=torch.uint8, device=X.device)
    S = torch.empty((R, C // 128), dtype=torch.float32, device=X.device)
    _check("moe_quantize_e4m3_rows", lib().moe_quantize_e4m3_rows(
        _ptr(X), act_dtype(X), X.stride(0), _ptr(row_src), k, R, C, _ptr(Q), _ptr(S), _stream()))
    return Q, S


def combine(Yp, assign_row, topk_w, S=None, out=None):
    """Y [T,H] = sum_j w[t,j] * Yp[assign_row[t*k+j]] (+ S[t]). `out`: optional
    [T,H] output buffer."""
    _dev(Yp, assign_row, topk_w, S, out)
    _i32(assign_row)
    T, k = topk_w.shape
    H = Yp.shape[1]
    if out is None:
        Y = torch.empty((T, H), dtype=Yp.dtype, device=Yp.device)
    elif tuple(out.shape) != (T, H) or out.dtype != Yp.dtype:
        raise ValueError("out must be [T, H] in Yp's dtype")
    else:
        Y = out
    _check("moe_combine", lib().moe_combine(_ptr(Yp), _ptr(assign_row), _ptr(topk_w), T, k, H, _ptr(S),
                                            act_dtype(Yp), _ptr(Y), _stream()))
    return Y


class MoELayer:
    """One MoE layer's device weights plus a reusable workspace.

    `weights` holds device tensors under the keys Wg, gate_bias, W1, W3, W2,
    S1, S3, S2 and (shared expert, optional) Ws1, Ws3, Ws2, Ss1, Ss3, Ss2.
    """

    def __init__(self, weights: dict, k: int, path: str = "auto"):
        self.w = {key: weights.get(key) for key in
                  ("Wg", "gate_bias", "W1", "W3", "W2", "S1", "S3", "S2",
                   "Ws1", "Ws3", "Ws2", "Ss1", "Ss3", "Ss2")}
        _dev(*[v for v in self.w.values() if v is not None])
        W1 = self.w["W1"]
        E, H, F = _expert_dims(W1, weight_dtype(W1, self.w["S1"]))
        Fs = 0 if self.w["Ws1"] is None else self.w["Ws1"].shape[1]
        d = LayerDesc()
        d.H, d.F, d.E, d.k, d.Fs = H, F, E, k, Fs
        d.w_dt = weight_dtype(W1, self.w["S1"])
        # activations are f32 with f32 experts, else bf16; the gate may be
        # fp32 beside bf16 activations (higher-precision router)
        d.act_dt = MOE_F32 if d.w_dt == MOE_F32 else MOE_BF16
        gate_dt = act_dtype(self.w["Wg"])
        if gate_dt != d.act_dt and not (gate_dt == MOE_F32 and d.act_dt == MOE_BF16):
            raise TypeError("the gate must have the activation dtype, or be float32 beside bfloat16")
        d.gate_f32 = int(gate_dt == MOE_F32 and d.act_dt == MOE_BF16)
        # the shared expert's own dtype (bf16 beside fp8 routed experts allowed)
        d.ws_dt = weight_dtype(self.w["Ws1"], self.w["Ss1"]) if Fs > 0 else d.w_dt
        d.path = PATHS[path]
        for key in self.w:
            setattr(d, key, None if self.w[key] is None else self.w[key].data_ptr())
        self.desc = d
        self.k = k
        self.E, self.H, self.F, self.Fs = E, H, F, Fs
        self._ws = None

    def workspace_bytes(self, T: int) -> int:
        return lib().moe_forward_workspace_bytes(ctypes.byref(self.desc), T)

    def workspace(self, T: int, device) -> torch.Tensor:
        n = max(self.workspace_bytes(T), 1)
        if self._ws is None or self._ws.numel() < n or self._ws.device != device:
            self._ws = torch.empty(n, dtype=torch.uint8, device=device)
        return self._ws

    def forward(self, X, Y=None, aux: bool = False, events=None):
        """Y [T,H]; with aux=True also (logits, topk_idx, topk_w, counts).

        `events`: optional ctypes array of MOE_N_EVENTS hipEvent_t handles
        (see StageEvents) recorded after each stage."""
        _dev(X, Y)
        T = X.shape[0]
        dev = X.device
        if Y is None:
            Y = torch.empty_like(X)
        ws = self.workspace(T, dev)
        outs = [None] * 4
        if aux:
            outs = [torch.empty((T, self.E), dtype=torch.float32, device=dev),
                    torch.empty((T, self.k), dtype=torch.int32, device=dev),
                    torch.empty((T, self.k), dtype=torch.float32, device=dev),
                    torch.empty(self.E, dtype=torch.int32, device=dev)]
        _check("moe_forward", lib().moe_forward(ctypes.byref(self.desc), _ptr(X), T, _ptr(Y), _ptr(ws),
                                                ws.numel(), _stream(), *[_ptr(o) for o in outs], events))
        return (Y, *outs) if aux else Y


    def forward_noalloc(self, X, Y=None, aux: bool = False, events=None):
        """As forward(), through moe_forward_noalloc: no workspace is passed
        (the library's fixed device scratch is used instead)."""
        _dev(X, Y)
        T = X.shape[0]
        dev = X.device
        if Y is None:
            Y = torch.empty_like(X)
        outs = [None] * 4
        if aux:
            outs = [torch.empty((T, self.E), dtype=torch.float32, device=dev),
                    torch.empty((T, self.k), dtype=torch.int32, device=dev),
                    torch.empty((T, self.k), dtype=torch.float32, device=dev),
                    torch.empty(self.E, dtype=torch.int32, device=dev)]
        _check("moe_forward_noalloc", lib().moe_forward_noalloc(ctypes.byref(self.desc), _ptr(X), T, _ptr(Y),
                                                                _stream(), *[_ptr(o) for o in outs], events))
        return (Y, *outs) if aux else Y


# ---------------------------------------------------------------------------
# Expert-parallel dispatch and combine between G ranks on one device
# ---------------------------------------------------------------------------
RECORD_INTS = 4  # moe_ep_record: token, expert, src_rank (int32), weight (fp32 bits)


def ep_dispatch(topk_idx, topk_w, X, E: int, G: int, rank: int, token0: int = 0, out=None):
    """-> (send_offsets [G+1], send_slot [A], send_rows [A,H], send_meta [A,4]
    int32 records). `out` optionally gives those four output buffers."""
    _dev(topk_idx, topk_w, X)
    _i32(topk_idx)
    T, k = topk_idx.shape
    H = X.shape[1]
    A = T * k
    dev = X.device
    if out is None:
        out = (torch.empty(G + 1, dtype=torch.int32, device=dev), torch.empty(A, dtype=torch.int32, device=dev),
               torch.empty((A, H), dtype=X.dtype, device=dev),
               torch.empty((A, RECORD_INTS), dtype=torch.int32, device=dev))
    so, slot, rows, meta = out
    _dev(so, slot, rows, meta)
    if so.numel() != G + 1 or slot.numel() != A or tuple(rows.shape) != (A, H) or meta.numel() != A * RECORD_INTS:
        raise ValueError("ep_dispatch output buffers have the wrong sizes")
    nbytes = lib().moe_ep_dispatch_workspace_bytes(T, k, G)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check("moe_ep_dispatch", lib().moe_ep_dispatch(
        _ptr(topk_idx), _ptr(topk_w), _ptr(X), act_dtype(X), T, k, H, E, G, rank, token0, _ptr(so), _ptr(slot),
        _ptr(rows), _ptr(meta), _ptr(ws), nbytes, _stream()))
    return so, slot, rows, meta


def ep_recv_offsets(send_offsets):
    """[G][G+1] send offsets of every rank -> [G][G+1] receive offsets."""
    _dev(send_offsets)
    _i32(send_offsets)
    G = send_offsets.shape[0]
    recv = torch.empty_like(send_offsets)
    _check("moe_ep_recv_offsets", lib().moe_ep_recv_offsets(_ptr(send_offsets), G, _ptr(recv), _stream()))
    return recv


def ep_exchange(inp, in_offsets, out, out_offsets, max_rows: int, gather=None):
    """All-to-all between the G ranks' row blocks inp [G, *, ...] -> out
    [G, *, ...] (rows = the trailing dimensions; see moe_ep_exchange)."""
    _dev(inp, in_offsets, out, out_offsets, gather)
    _i32(in_offsets)
    _i32(out_offsets)
    G = inp.shape[0]
    row_bytes = inp[0, 0].numel() * inp.element_size() if inp.shape[1] > 0 else out[0, 0].numel() * out.element_size()
    _check("moe_ep_exchange", lib().moe_ep_exchange(
        G, _ptr(inp), inp.stride(0) * inp.element_size(), _ptr(in_offsets), _ptr(gather),
        0 if gather is None else gather.stride(0), _ptr(out), out.stride(0) * out.element_size(), _ptr(out_offsets),
        row_bytes, max_rows, _stream()))
    return out


def ep_local_experts(recv_meta, n: int, E: int, G: int, rank: int, out=None):
    """Local expert ids of the first n received records of rank `rank`."""
    _dev(recv_meta, out)
    local = torch.empty(n, dtype=torch.int32, device=recv_meta.device) if out is None else out
    _check("moe_ep_local_experts", lib().moe_ep_local_experts(_ptr(recv_meta), n, E, G, rank, _ptr(local),
                                                              _stream()))
    return local


def rank_tokens(T: int, G: int, r: int) -> slice:
    """Token slice of rank r: the r-th of G contiguous slices of ceil(T/G)."""
    n = -(-T // G)
    return slice(min(r * n, T), min((r + 1) * n, T))


class EPLoopback:
    """One MoE layer with its experts spread over G ranks that share one
    device (page "MOE推理流程解析" §五), each rank's steps issued in order:
    route its tokens -> dispatch (bucket by owner, pack records) -> all-to-all
    -> local permutation + grouped FFN of its experts -> return all-to-all ->
    combine at the source (+ the shared expert, replicated per rank).
    Between the two halves the host reads the G x G count matrix, as an
    all-to-all(v) needs its split sizes; every other step stays on the device.
    `events`: optional list of len(EP_STAGES) + 1 torch.cuda.Event, the
    first recorded before the first stage and event i + 1 after stage i of
    EP_STAGES ("counts" is the host's read of the count matrix)."""

    def __init__(self, weights: dict, k: int, G: int, path: str = "auto"):
        self.w = weights
        self.k, self.G, self.path = k, G, path
        W1 = weights["W1"]
        self.wdt = weight_dtype(W1, weights.get("S1"))
        self.E, self.H, self.F = _expert_dims(W1, self.wdt)
        if self.E % G:
            raise ValueError("E must be divisible by G")
        self.El = self.E // G

    def _experts(self, d: int):
        sl = slice(d * self.El, (d + 1) * self.El)
        get = lambda key: None if self.w.get(key) is None else self.w[key][sl]
        return [get(key) for key in ("W1", "W3", "W2", "S1", "S3", "S2")]

    def forward(self, X, Y=None, events=None, keep: bool = False):
        _dev(X, Y)
        T, H = X.shape
        G, k, E = self.G, self.k, self.E
        dev = X.device
        if Y is None:
            Y = torch.empty_like(X)
        mark = (lambda i: events[i].record()) if events else (lambda i: None)
        ranks = [rank_tokens(T, G, r) for r in range(G)]
        cap_s = max(max(sl.stop - sl.start for sl in ranks), 1) * k
        mark(0)
        # route on every rank (each on its own tokens)
        routes = [route(X[sl], self.w["Wg"], k, self.w.get("gate_bias")) if sl.stop > sl.start else None
                  for sl in ranks]
        mark(1)
        # dispatch: buckets by owner and records, into rank-strided buffers
        send_off = torch.zeros((G, G + 1), dtype=torch.int32, device=dev)
        send_slot = torch.empty((G, cap_s), dtype=torch.int32, device=dev)
        send_rows = torch.empty((G, cap_s, H), dtype=X.dtype, device=dev)
        send_meta = torch.empty((G, cap_s, RECORD_INTS), dtype=torch.int32, device=dev)
        for r, sl in enumerate(ranks):
            n = (sl.stop - sl.start) * k
            if n == 0:
                continue
            ep_dispatch(routes[r][1], routes[r][2], X[sl], E, G, r, sl.start,
                        out=(send_off[r], send_slot[r, :n], send_rows[r, :n], send_meta[r, :n]))
        recv_off = ep_recv_offsets(send_off)
        mark(2)
        # the count matrix on the host (an all-to-all(v) needs its split sizes)
        recv_h = recv_off.cpu()
        n_recv = [int(recv_h[d, G]) for d in range(G)]
        cap_r = max(max(n_recv), 1)
        recv_rows = torch.empty((G, cap_r, H), dtype=X.dtype, device=dev)
        recv_meta = torch.empty((G, cap_r, RECORD_INTS), dtype=torch.int32, device=dev)
        mark(3)
        ep_exchange(send_rows, send_off, recv_rows, recv_off, cap_s)
        ep_exchange(send_meta, send_off, recv_meta, recv_off, cap_s)
        mark(4)
        # each rank's experts on what it received
        Yp = torch.empty((G, cap_r, H), dtype=X.dtype, device=dev)
        assign = torch.empty((G, cap_r), dtype=torch.int32, device=dev)
        local = []
        for d in range(G):
            n = n_recv[d]
            if n == 0:
                local.append(None)
                continue
            lidx = ep_local_experts(recv_meta[d, :n], n, E, G, d)
            counts, offsets, row_src, _, _ = permute(lidx.view(n, 1), self.El, assign_row=assign[d, :n])
            W1, W3, W2, S1, S3, S2 = self._experts(d)
            grouped_ffn(recv_rows[d, :n], offsets, W1, W3, W2, S1, S3, S2, row_src=row_src, k=1, path=self.path,
                        out=Yp[d, :n])
            local.append((lidx, counts, offsets, row_src))
        mark(5)
        # results back to their sources, in send order
        ret = torch.empty((G, cap_s, H), dtype=X.dtype, device=dev)
        ep_exchange(Yp, recv_off, ret, send_off, cap_s, gather=assign)
        mark(6)
        # combine at the source (+ the shared expert on the rank's own tokens)
        shared = self.w.get("Ws1") is not None
        for r, sl in enumerate(ranks):
            nt = sl.stop - sl.start
            if nt == 0:
                continue
            S = None
            if shared:
                off = torch.tensor([0, nt], dtype=torch.int32, device=dev)
                sw = [None if self.w.get(key) is None else self.w[key].unsqueeze(0)
                      for key in ("Ws1", "Ws3", "Ws2", "Ss1", "Ss3", "Ss2")]
                S = grouped_ffn(X[sl], off, *sw, path=self.path)
            combine(ret[r, :nt * k], send_slot[r, :nt * k], routes[r][2], S, out=Y[sl])
        mark(7)
        if keep:
            self.last = dict(routes=routes, send_off=send_off, send_slot=send_slot, send_rows=send_rows,
                             send_meta=send_meta, recv_off=recv_off, n_recv=n_recv, recv_rows=recv_rows,
                             recv_meta=recv_meta, Yp=Yp, assign=assign, local=local, ret=ret)
        return Y


EP_STAGES = ["route", "dispatch", "counts", "exchange", "experts", "return", "combine"]


# ---------------------------------------------------------------------------
# Stage timing with HIP events (plumbing for measurement only)
# ---------------------------------------------------------------------------
MOE_N_EVENTS = 9
STAGES = ["route", "permute", "schedule", "gate_up", "shared_gate_up", "down", "shared_down", "combine"]

_hip = None


def hip_runtime() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        # the runtime torch already loaded (same soname as libmoe's dependency)
        for name in ("libamdhip64.so.7", "libamdhip64.so"):
            try:
                _hip = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if _hip is None:
            raise RuntimeError("libamdhip64.so not found")
        # event handles are pointers: declare every signature so ctypes never
        # narrows them to C int
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventCreate.restype = ctypes.c_int
        _hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        _hip.hipEventCreateWithFlags.restype = ctypes.c_int
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventDestroy.restype = ctypes.c_int
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipEventSynchronize.restype = ctypes.c_int
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipEventElapsedTime.restype = ctypes.c_int
    return _hip


# hipEventDisableSystemFence (hip_runtime_api.h): a timing-only event whose
# record skips the system-scope fence (an L2 writeback and invalidation), which
# otherwise adds several microseconds to the measured work per marker. Elapsed
# times stay valid; callers synchronise the device before reading them.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class StageEvents:
    """MOE_N_EVENTS timing events; `want` selects which markers are recorded."""

    def __init__(self, want=None):
        hip = hip_runtime()
        self.handles = (ctypes.c_void_p * MOE_N_EVENTS)()
        self._owned = []
        want = range(MOE_N_EVENTS) if want is None else want
        for i in want:
            ev = ctypes.c_void_p()
            if hip.hipEventCreateWithFlags(ctypes.byref(ev), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.handles[i] = ev
            self._owned.append(ev)

    def elapsed_ms(self, i: int, j: int) -> float:
        """Milliseconds between markers i and j (both must have been recorded)."""
        hip = hip_runtime()
        ms = ctypes.c_float()
        if hip.hipEventSynchronize(self.handles[j]) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        if hip.hipEventElapsedTime(ctypes.byref(ms), self.handles[i], self.handles[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        try:
            hip = hip_runtime()
            for ev in self._owned:
                hip.hipEventDestroy(ev)
        except Exception:
            pass
