/*
 * moe.h - C ABI of libmoe: the forward pass of one Mixture-of-Experts layer on
 * one AMD Instinct MI355X (gfx950).
 *
 * The layer, as the page "MOE推理流程解析" (ffner.com) describes it:
 *   section 三: the router scores every expert and top-k keeps the chosen
 *     indices and their weights; a permutation writes token rows in expert
 *     order and records an inverse map; the grouped expert computation runs
 *     all experts' row blocks in one launch; experts apply their activation
 *     and output projection; the inverse map restores token order and the
 *     weighted contributions are summed per token.
 *   section 二: T*k assignments, each (token row, expert, weight), grouped
 *     into per-expert matrices; the token id stays beside each row.
 *   section 一: an optional shared expert processes every token with weight 1.
 *   section 九: the kept top-k weights are renormalised.
 * The page "MoE serving production quirks" (tianpan.co, memory-paradox
 * section) states the gate as a linear projection plus a softmax over all
 * experts; the page "MoE-推理部署" (zzmblog.top, expert-quantisation section)
 * asks for per-expert FP8 scales.
 *
 * Expert FFN form (SwiGLU): h = silu(x W1) * (x W3), y = h W2, with
 * silu(z) = z / (1 + exp(-z)).
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless stated; all buffers are owned by the
 *    caller, including workspaces. The library never allocates or frees device
 *    memory and keeps no pointer after a call returns.
 *  - Calls are asynchronous on `stream` (NULL = the null stream). There is no
 *    device-to-host synchronisation inside any call, so every call can be
 *    captured into a HIP graph. Inputs must stay valid until the work ends.
 *  - Matrices are row-major and densely packed.
 *  - Shapes and pointers are validated on the host before anything is
 *    launched; on error nothing is enqueued and a status is returned.
 *    T == 0 returns MOE_OK without launching. Launch failures return
 *    MOE_ERR_HIP. No call throws.
 *  - Routing order: the k slots of a token hold its experts best score first;
 *    equal scores go to the lower expert index. Rows of an expert block are in
 *    ascending assignment order a = t*k + j (so ascending token order).
 *  - dtype combinations (activation, expert weights): (F32, F32), (BF16,
 *    BF16), (BF16, FP8_E4M3), (BF16, MXFP4). The gate matrix has the
 *    activation dtype (or fp32, see moe_route).
 *    FP8 weights are OCP E4M3 codes with one fp32 scale per 128x128 block,
 *    so their dimensions must be multiples of 128.
 *    MXFP4 weights (the page "MoE-推理部署", expert-quantisation section, names
 *    MXFP4 beside FP8): a [K, N] matrix is stored as [K/2, N] bytes, byte
 *    (i, n) holding rows 2i (low nibble) and 2i + 1 (high nibble) of column
 *    n as E2M1 codes, with [K/32, N] E8M0 scale bytes (2^(e - 127)), one per
 *    32 K rows of a column; the S* pointers then point to these bytes. So W1,
 *    W3 are [E, H/2, F] and W2 [E, F/2, H] bytes, S1, S3 [E, H/32, F] and S2
 *    [E, F/32, H]. Both kernels decode the codes on chip (the row-streaming
 *    path in registers, the tiled path after staging codes and scales in LDS)
 *    and multiply in bf16; the workspace is the bf16 one. Scale code 0 is
 *    2^-127; code 255 (NaN) makes the outputs that depend on it non-finite.
 *    TILED_A8 is refused.
 *    H and F must be multiples of 32 and at most 2^20; E <= 1024;
 *    1 <= k <= min(E, 64); moe_route needs T*E < 2^31, moe_permute T*k < 2^31,
 *    moe_forward T <= 65535. Larger sizes return MOE_ERR_UNSUPPORTED (and the
 *    *_workspace_bytes calls 0).
 *  - Thread safety: no mutable global state; concurrent calls on different
 *    streams with disjoint outputs and workspaces are safe.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,         /* null pointer, bad size, k > E, ... */
    MOE_ERR_UNSUPPORTED = 2,         /* valid but not implemented: dtype pair, alignment */
    MOE_ERR_WORKSPACE_TOO_SMALL = 3, /* ws_bytes below the *_workspace_bytes() value */
    MOE_ERR_HIP = 4,                 /* a HIP launch failed */
    MOE_ERR_SCRATCH_LIMIT = 5        /* moe_forward_noalloc: the layer's workspace exceeds
                                        moe_forward_noalloc_max_bytes() */
} moe_status;

typedef enum {
    MOE_F32 = 0,
    MOE_BF16 = 1,
    MOE_FP8_E4M3 = 2, /* OCP E4M3 ("e4m3fn"), 1 byte per value, weights only */
    MOE_MXFP4 = 3     /* OCP MXFP4 weights only: E2M1 codes, two K-consecutive values
                         a byte, one E8M0 scale per 32 K rows of a column (below) */
} moe_dtype;

/* Expert-FFN kernel choice. AUTO picks the row-streaming (batched GEMV) path
 * when the experts average fewer than 15 rows (48 for MXFP4 weights) and the
 * LDS-tiled grouped GEMM otherwise (prefill); for FP8 weights the tiled choice
 * is TILED_A8. All give results within the same tolerance of the exact layer;
 * the forced values exist for testing and comparison.
 *  GEMV, TILED: activations stay in act_dt; FP8 weights are decoded exactly
 *    and each 128-deep K block is scaled (W8A16).
 *  TILED_A8 (FP8 weights only, H and F multiples of 128): the expert inputs
 *    (token rows, then h) are quantised to E4M3 per row and 128-column group
 *    with scale amax/448 (page "MOE推理流程解析" §三: activations quantised
 *    before the expert GEMM) and multiplied on the FP8 matrix cores (W8A8);
 *    h is quantised inside the gate/up GEMM, from its bf16 values.
 *    In moe_forward it needs Fs == 0 or Fs == F. */
typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_GEMV = 1, MOE_PATH_TILED = 2, MOE_PATH_TILED_A8 = 3 } moe_ffn_path;

/* Static string for a status code (host memory, never NULL). */
const char *moe_status_string(moe_status s);

/* ---------------------------------------------------------------------------
 * Router: logits, softmax, top-k, renormalised weights.
 *   logits[t,e] = sum_h X[t,h] * Wg[h,e] + gate_bias[e]   (fp32 accumulate)
 *   topk_idx[t,:] = the k experts with the largest logits (softmax is
 *     monotone), best first, ties to the lower index
 *   topk_w[t,j]   = p[t,topk_idx[t,j]] / sum_j' p[t,topk_idx[t,j']], p the
 *     softmax over all E logits; computed as the identical softmax over the
 *     k kept logits, in fp32.
 * X [T,H] in x_dt (F32 or BF16); Wg [H,E] in wg_dt: x_dt, or F32 beside
 * BF16 tokens (the page "MoE-推理部署", expert-quantisation section: the
 * router is usually kept at higher precision than the experts; every
 * product is then taken in fp32); other pairs return MOE_ERR_UNSUPPORTED.
 * gate_bias [E] fp32 or NULL.
 * Outputs: logits [T,E] fp32, topk_idx [T,k] int32, topk_w [T,k] fp32.
 * NaN logits are never selected while a non-NaN logit is left.
 * The sum over h is split into fixed K ranges whose fp32 partial sums are
 * added in a fixed order, so results are identical run to run.
 * Workspace: moe_route_workspace_bytes(T, H, E) bytes (may be 0; then ws may
 * be NULL).
 * ------------------------------------------------------------------------- */
size_t moe_route_workspace_bytes(int T, int H, int E);
moe_status moe_route(const void *X, moe_dtype x_dt, const void *Wg, moe_dtype wg_dt, const float *gate_bias,
                     int T, int H, int E, int k,
                     float *logits, int32_t *topk_idx, float *topk_w,
                     void *ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Dispatch on one GPU: group the A = T*k assignments by expert.
 *   counts[e]     = #{a : topk_idx[a] == e}                  [E]
 *   offsets[e]    = sum_{e' < e} counts[e'], offsets[E] = A  [E+1]
 *   row_src[r]    = assignment a held by row r (stable: ascending a within
 *                   each expert block)                        [A]
 *   assign_row[a] = row r with row_src[r] == a (inverse map)  [A]
 *   Xp[r, :]      = X[row_src[r] / k, :] if Xp != NULL        [A, H] (x_dt)
 * topk_idx entries must lie in [0, E) (the kernel skips others, leaving their
 * rows unset). Bit-exact and deterministic (no atomics decide any order).
 * Workspace: moe_permute_workspace_bytes(T, k, E) bytes (device, any
 * contents, 256-byte aligned).
 * ------------------------------------------------------------------------- */
size_t moe_permute_workspace_bytes(int T, int k, int E);
moe_status moe_permute(const int32_t *topk_idx, int T, int k, int E,
                       int32_t *counts, int32_t *offsets, int32_t *row_src, int32_t *assign_row,
                       const void *X, moe_dtype x_dt, int H, void *Xp,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Grouped expert FFN over G row blocks (one per expert):
 *   for each group g and row r in [offsets[g], offsets[g+1]):
 *     x  = row r of the input (see below)
 *     h  = silu(x W1[g]) * (x W3[g])
 *     Yp[r, :] = h W2[g]
 * Input rows: if row_src == NULL, Xin is [M, H] already permuted and row r is
 * Xin[r]; otherwise Xin is the token matrix [T, H] and row r is
 * Xin[row_src[r] / k] (the permutation is fused into the load).
 * offsets [G+1] int32 on the device with offsets[0] = 0 and offsets[G] = M.
 * W1, W3 [G, H, F]; W2 [G, F, H] in w_dt. For FP8 weights, S1, S3
 * [G, H/128, F/128] and S2 [G, F/128, H/128] are fp32 block scales
 * (weight = decode(code) * scale); they must be NULL otherwise.
 * Yp [M, H] in act_dt. Accumulation is fp32; h is rounded to act_dt.
 * Workspace: moe_grouped_ffn_workspace_bytes(...) bytes.
 * ------------------------------------------------------------------------- */
size_t moe_grouped_ffn_workspace_bytes(int M, int G, int H, int F, moe_dtype act_dt,
                                       moe_dtype w_dt, moe_ffn_path path);
moe_status moe_grouped_ffn(const void *Xin, const int32_t *row_src, int k, int M,
                           const int32_t *offsets, int G, int H, int F,
                           const void *W1, const void *W3, const void *W2, moe_dtype w_dt,
                           const float *S1, const float *S3, const float *S2,
                           moe_dtype act_dt, void *Yp, moe_ffn_path path,
                           void *ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * E4M3 activation quantisation (the W8A8 path's input step; page
 * "MOE推理流程解析" §三: activations may be quantised before dispatch or
 * before the expert GEMM). For output row r (input row row_src[r] / gk, or r
 * when row_src is NULL) and each 128-column group c:
 *   s = amax / 448 over the group's |x| (s = 1 when amax = 0),
 *   Q[r, j] = E4M3(x[j] / s) rounded to nearest, ties to even, saturating
 *   at +-448;  S[r, c] = s.
 * All arithmetic fp32 (correctly rounded division). X [*, ldx] bf16 with
 * ldx >= C and ldx % 8 == 0; C a multiple of 128; Q [R, C] uint8 codes,
 * S [R, C/128] fp32. Deterministic, bit-exact.
 * ------------------------------------------------------------------------- */
moe_status moe_quantize_e4m3_rows(const void *X, moe_dtype x_dt, long long ldx, const int32_t *row_src,
                                  int gk, int R, int C, uint8_t *Q, float *S, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Combine / unpermute:
 *   Y[t, :] = sum_{j<k} topk_w[t,j] * Yp[assign_row[t*k+j], :]  (+ S[t, :])
 * summed in fp32 in ascending j, then S added with weight 1, then rounded to
 * act_dt. Yp [A, H], S [T, H] (or NULL), Y [T, H] in act_dt.
 * ------------------------------------------------------------------------- */
moe_status moe_combine(const void *Yp, const int32_t *assign_row, const float *topk_w,
                       int T, int k, int H, const void *S, moe_dtype act_dt, void *Y,
                       hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Whole layer: route -> permute -> grouped FFN (+ shared expert) -> combine.
 * Weights are borrowed device pointers described by moe_layer_desc. The
 * shared expert (Fs > 0) uses Ws1, Ws3 [H, Fs], Ws2 [Fs, H] in ws_dt (+ Ss*
 * scales when ws_dt is FP8) and is added with weight 1. ws_dt equals w_dt,
 * or is BF16 beside FP8 routed experts: the page "MoE-推理部署"
 * (expert-quantisation section) notes that the shared expert, like the
 * router, is usually kept at higher precision than the routed experts. A
 * shared expert whose dtype or width differs from the routed experts' runs
 * as its own one-group launches; otherwise it is one more group of the routed
 * launches. ws_dt is ignored when Fs == 0. Unsupported pairs return
 * MOE_ERR_UNSUPPORTED; scale pointers that do not match ws_dt return
 * MOE_ERR_INVALID_ARG. X [T, H] and Y [T, H] in act_dt.
 * Optional outputs (NULL to skip): logits [T,E], topk_idx [T,k],
 * topk_w [T,k], counts [E]. Optional `events`: see MOE_EV_* below.
 * Workspace: moe_forward_workspace_bytes(desc, T) bytes.
 * ------------------------------------------------------------------------- */
typedef struct moe_layer_desc {
    int H, F, E, k, Fs;
    moe_dtype act_dt, w_dt;
    moe_ffn_path path;
    const void *Wg;          /* [H, E], act_dt (fp32 when gate_f32) */
    const float *gate_bias;  /* [E] or NULL */
    const void *W1, *W3, *W2;
    const float *S1, *S3, *S2;
    const void *Ws1, *Ws3, *Ws2;
    const float *Ss1, *Ss3, *Ss2;
    moe_dtype ws_dt;         /* shared expert weights: w_dt, or BF16 beside FP8 */
    int gate_f32;            /* 0: Wg in act_dt; 1: Wg fp32 (higher-precision
                                router, see moe_route); other values rejected */
} moe_layer_desc;

/* Stage markers for moe_forward's `events` argument: events[i] is recorded on
 * `stream` right after stage i (events[MOE_EV_START] before the first
 * launch). The page "MOE推理流程解析" (sections 三 and 十) asks for routing,
 * permutation, expert GEMM and combine to be timed separately; elapsed time
 * between consecutive markers is exactly one stage. Entries may be NULL. */
enum {
    MOE_EV_START = 0,
    MOE_EV_ROUTE,          /* router GEMM + top-k done */
    MOE_EV_PERMUTE,        /* counts / offsets / permutation done */
    MOE_EV_SCHEDULE,       /* tile list built (and, on TILED_A8, X quantised) */
    MOE_EV_GATE_UP,        /* routed gate/up GEMM + SwiGLU done (TILED_A8: h written as E4M3) */
    MOE_EV_SHARED_GATE_UP, /* shared expert gate/up done (no-op without one) */
    MOE_EV_DOWN,           /* routed down projection done */
    MOE_EV_SHARED_DOWN,    /* shared expert down projection done */
    MOE_EV_COMBINE,        /* combine done: Y written */
    MOE_N_EVENTS
};

size_t moe_forward_workspace_bytes(const moe_layer_desc *desc, int T);
moe_status moe_forward(const moe_layer_desc *desc, const void *X, int T, void *Y,
                       void *ws, size_t ws_bytes, hipStream_t stream,
                       float *logits_out, int32_t *topk_idx_out, float *topk_w_out,
                       int32_t *counts_out, hipEvent_t const *events /* [MOE_N_EVENTS] or NULL */);

/* ---------------------------------------------------------------------------
 * Expert-parallel dispatch and combine (page "MOE推理流程解析" §五): experts
 * are placed on G ranks in contiguous blocks, expert e on rank e / (E/G)
 * (E divisible by G); an assignment whose expert is on another rank travels
 * there as a record of the token row plus (token id, expert, source rank,
 * routing weight); each rank groups what it received by expert and runs one
 * matrix per active local expert (moe_permute + moe_grouped_ffn on the local
 * expert ids); the results travel back and the source restores token order,
 * weights and sums (moe_combine with send_slot as the inverse map). Here the
 * G ranks share one device and moe_ep_exchange is the all-to-all between
 * their buffers; on several GPUs it would be an RCCL all-to-all(v), whose
 * split sizes are the count matrix below. Per-rank buffers of the exchange
 * are laid out at a fixed stride from one base pointer.
 * ------------------------------------------------------------------------- */
typedef struct moe_ep_record {
    int32_t token;    /* token id: token0 + local token index */
    int32_t expert;   /* global expert index */
    int32_t src_rank; /* rank the token lives on */
    float weight;     /* routing weight of the assignment */
} moe_ep_record;      /* 16 bytes */

/* Dispatch on source rank `rank` of G: bucket its A = T*k assignments a =
 * t*k + j (topk_idx, topk_w [T,k], as moe_route writes them) by destination
 * rank, stably (ascending a within a destination), and pack them.
 *   send_offsets [G+1]: first send row of each destination, send_offsets[G] = A
 *   send_slot [A]:      send row of assignment a
 *   send_rows [A, H]:   send row r holds X[a/k] (x_dt: F32 or BF16; H*size
 *                       a multiple of 16 bytes)
 *   send_meta [A]:      the record of that assignment (token = token0 + a/k)
 * Assignments naming an expert outside [0, E) are left out (their rows and
 * slots unset; send_offsets[G] counts the others). Deterministic.
 * Workspace: moe_ep_dispatch_workspace_bytes(T, k, G). */
size_t moe_ep_dispatch_workspace_bytes(int T, int k, int G);
moe_status moe_ep_dispatch(const int32_t *topk_idx, const float *topk_w, const void *X, moe_dtype x_dt, int T,
                           int k, int H, int E, int G, int rank, int token0, int32_t *send_offsets,
                           int32_t *send_slot, void *send_rows, moe_ep_record *send_meta, void *ws,
                           size_t ws_bytes, hipStream_t stream);

/* Receive layout from every rank's send_offsets (device [G][G+1], row s =
 * rank s's send_offsets): recv_offsets[d][s] = first receive row of rank d
 * holding rank s's rows (sum of what ranks s' < s send to d),
 * recv_offsets[d][G] = rows rank d receives. G <= 1024. */
moe_status moe_ep_recv_offsets(const int32_t *send_offsets, int G, int32_t *recv_offsets, hipStream_t stream);

/* All-to-all between G ranks' buffers on this device. Rank r's input rows
 * start at in + r*in_rank_stride, its output rows at out + r*out_rank_stride
 * (strides in bytes). For every ordered pair (s, d) and i < in_offsets[s][d+1]
 * - in_offsets[s][d]:
 *   out row out_offsets[d][s] + i of rank d = in row g(in_offsets[s][d] + i) of rank s,
 * g(j) = gather[s*gather_rank_stride + j] when gather != NULL, else j.
 * Offsets are device [G][G+1] arrays. Dispatch: in/out = send/receive rows
 * (or records, 16 bytes), in_offsets = send_offsets, out_offsets =
 * recv_offsets. Return: in = each expert rank's grouped-FFN output (local
 * permuted order), gather = its moe_permute assign_row, in_offsets =
 * recv_offsets, out_offsets = send_offsets, so results land in send order.
 * row_bytes, the strides and the base pointers must be multiples of 16;
 * max_rows bounds every pair's row count (rows beyond it are not copied);
 * G*G <= 65535. The caller sizes every buffer for the rows the offsets
 * name. */
moe_status moe_ep_exchange(int G, const void *in, long long in_rank_stride, const int32_t *in_offsets,
                           const int32_t *gather, long long gather_rank_stride, void *out,
                           long long out_rank_stride, const int32_t *out_offsets, int row_bytes, int max_rows,
                           hipStream_t stream);

/* Receiver side of rank `rank`: local_idx[i] = recv_meta[i].expert - rank*E/G
 * for the n received records (-1 for a record naming another rank's expert),
 * the expert ids moe_permute groups the received rows by (T = n, k = 1,
 * E = E/G). */
moe_status moe_ep_local_experts(const moe_ep_record *recv_meta, int n, int E, int G, int rank, int32_t *local_idx,
                                hipStream_t stream);

/* ---------------------------------------------------------------------------
 * moe_forward without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same arguments, kernels and results as moe_forward
 * (bit for bit); the workspace is a fixed array of
 * moe_forward_noalloc_max_bytes() bytes (256 MiB) in device global memory that
 * the library's code object holds on every GPU it is loaded on, until the
 * process ends. Nothing is allocated or freed, on the device or by any
 * library routine.
 *  - The layer's workspace (moe_forward_workspace_bytes(desc, T)) must fit:
 *    otherwise MOE_ERR_SCRATCH_LIMIT, returned on the host before the device
 *    is touched. Every decode batch of the Mixtral-, Qwen3- and
 *    DeepSeek-V3-shaped layers fits; prefill batches of thousands of tokens
 *    do not (use moe_forward with a workspace).
 *  - The work runs on the current device; `stream` (NULL = null stream) must
 *    belong to it, else MOE_ERR_INVALID_ARG.
 *  - Every call on one GPU uses that GPU's one array, and no kernel relies on
 *    its contents at entry (each writes what it later reads, as with a fresh
 *    workspace). Calls that overlap in time on one GPU (on different streams,
 *    or from several threads without ordering) race on the array and give
 *    undefined results: order them, e.g. on one stream.
 * ------------------------------------------------------------------------- */
size_t moe_forward_noalloc_max_bytes(void);
moe_status moe_forward_noalloc(const moe_layer_desc *desc, const void *X, int T, void *Y, hipStream_t stream,
                               float *logits_out, int32_t *topk_idx_out, float *topk_w_out,
                               int32_t *counts_out, hipEvent_t const *events);

/* ---------------------------------------------------------------------------
 * Bounds-checked debug build (libmoe_debug.so: every source compiled with
 * -DMOE_BOUNDS_CHECK). Its kernels check the indices they address memory
 * with -- tile records, gathered and permuted rows, combine rows, scale rows,
 * tail-split slots, exchange rows -- and on a failed check record a bit
 * (below) instead of trapping, and keep the access in bounds (results are
 * then wrong, but nothing faults). Same arguments and results as the release
 * library otherwise.
 * moe_debug_bounds(): waits for the current device, returns the union of the
 * bits recorded since the previous call and clears them; ~0u if a HIP call
 * failed. The release library returns 0 and touches no device.
 * ------------------------------------------------------------------------- */
#define MOE_BOUNDS_TILE 1u          /* tile record: group, first or end row */
#define MOE_BOUNDS_A_ROW 2u         /* gathered input row of a GEMM */
#define MOE_BOUNDS_SCALE_ROW 4u     /* activation-scale row of the W8A8 GEMM */
#define MOE_BOUNDS_TAIL_SLOT 8u     /* tail-split partial slot or counter */
#define MOE_BOUNDS_PERM_ROW 16u     /* permuted row of an assignment */
#define MOE_BOUNDS_COMBINE_ROW 32u  /* Yp row read by combine */
#define MOE_BOUNDS_QUANT_ROW 64u    /* scale row written by the quantiser */
#define MOE_BOUNDS_EP_ROW 128u      /* row of an expert-parallel exchange */
unsigned moe_debug_bounds(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
