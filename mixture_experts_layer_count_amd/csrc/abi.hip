// libmoe public entry points: argument validation, workspace layout and the
// order of stage launches. Every launch goes to the caller's stream; nothing
// here synchronises with the device or allocates device memory.
#include <string.h>

#include "common.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
constexpr int kGemvBM = 16;  // rows per tile of the row-streaming GEMM

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Bump allocator over a caller-provided workspace. With base == NULL it only
// measures.
struct Carver {
    char *base;
    size_t used = 0;
    explicit Carver(void *b) : base(static_cast<char *>(b)) {}
    void *take(size_t bytes) {
        void *p = base ? base + used : nullptr;
        used += align_up(bytes);
        return p;
    }
};

size_t dt_size(moe_dtype d) { return d == MOE_F32 ? 4 : d == MOE_BF16 ? 2 : 1; }

bool act_ok(moe_dtype a) { return a == MOE_F32 || a == MOE_BF16; }

bool pair_ok(moe_dtype act, moe_dtype w) {
    return (act == MOE_F32 && w == MOE_F32) || (act == MOE_BF16 && w == MOE_BF16) ||
           (act == MOE_BF16 && w == MOE_FP8_E4M3) || (act == MOE_BF16 && w == MOE_MXFP4);
}

// weights stored as codes with scales (E4M3 + fp32 block scales, or MXFP4
// E2M1 + E8M0 scales)
bool scaled(moe_dtype w) { return w == MOE_FP8_E4M3 || w == MOE_MXFP4; }

WType wtype(moe_dtype w) {
    return w == MOE_F32 ? W_F32 : w == MOE_BF16 ? W_BF16 : w == MOE_MXFP4 ? W_MXFP4 : W_FP8;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                                  \
    do {                                               \
        hipError_t e_ = (expr);                        \
        if (e_ != hipSuccess) return MOE_ERR_HIP;      \
    } while (0)

// Shape rules for expert matrices [K][N].
constexpr int kMaxDim = 1 << 20;  // largest H or F (keeps every size product in range)

moe_status check_ffn_dims(int H, int F, moe_dtype w_dt) {
    if (H < 1 || F < 1) return MOE_ERR_INVALID_ARG;
    if (H % 32 || F % 32 || H > kMaxDim || F > kMaxDim) return MOE_ERR_UNSUPPORTED;
    if (w_dt == MOE_FP8_E4M3 && (H % 128 || F % 128)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// ---------------------------------------------------------------------------
// Expert FFN planning (shared by moe_grouped_ffn and moe_forward)
// ---------------------------------------------------------------------------
struct FfnPlan {
    bool tiled;
    bool a8;      // tiled with E4M3 activations (W8A8)
    bool tail;    // tiled with the tail split (bf16 and MXFP4 weights)
    int bm;
    int ksplit1;  // split-K of gate/up (row-streaming path; 1: none)
    int kchunk1;
    int ksplit2;  // split-K of the down projection (row-streaming path)
    int kchunk2;
};

bool path_ok(moe_ffn_path path) {
    return path == MOE_PATH_AUTO || path == MOE_PATH_GEMV || path == MOE_PATH_TILED || path == MOE_PATH_TILED_A8;
}

// a8_ok: the caller can run the W8A8 form (AUTO picks it for FP8 weights
// whenever it picks the tiled path).
FfnPlan plan_ffn(int M, int G, int H, int F, moe_dtype w_dt, moe_ffn_path path, bool a8_ok = true) {
    FfnPlan p{};
    const WType wt = wtype(w_dt);
    const bool can_tile = tiled_gemm_supports(wt, F, H) && tiled_gemm_supports(wt, H, F);
    const bool can_a8 = a8_ok && w_dt == MOE_FP8_E4M3 && tiled_a8_supports(F, H) && tiled_a8_supports(H, F);
    if (path == MOE_PATH_TILED_A8) {
        p.tiled = p.a8 = can_a8;
    } else if (path == MOE_PATH_TILED) {
        p.tiled = can_tile;
    } else if (path == MOE_PATH_GEMV) {
        p.tiled = false;
    } else {
        // the tiled kernels win from about 12-25 rows per group (measured by
        // token-count sweeps of the Mixtral-, Qwen3- and DeepSeek-shaped
        // layers); with MXFP4 weights the row-streaming kernel reads a quarter
        // of bf16's bytes, and the sweeps put the crossover at 32-64 rows
        const long long min_rows = w_dt == MOE_MXFP4 ? 48 : 15;
        p.tiled = can_tile && (long long)M >= min_rows * G;
        p.a8 = p.tiled && can_a8;
    }
    p.bm = p.a8 ? tiled_a8_bm(M, G) : p.tiled ? tiled_gemm_bm(wt, M, G) : kGemvBM;
    p.tail = p.tiled && !p.a8 && (w_dt == MOE_BF16 || w_dt == MOE_MXFP4);
    p.ksplit1 = 1;
    p.kchunk1 = H;
    p.ksplit2 = 1;
    p.kchunk2 = F;
    if (!p.tiled) {
        // enough wavefronts in flight to cover HBM latency: ~2048
        const long long tiles_est = M < G ? M : G;
        // gate/up: split over H only when its slices alone leave most SIMDs
        // idle (few touched experts); its fp32 partials are summed and passed
        // through SwiGLU by one small pass
        const int slice = (w_dt == MOE_FP8_E4M3 || w_dt == MOE_MXFP4) ? 128 : 64;
        const long long waves1 = tiles_est * ((F + slice - 1) / slice);
        if (waves1 < 1024) {
            int ks1 = (int)((2048 + waves1 - 1) / (waves1 > 0 ? waves1 : 1));
            ks1 = ks1 < 1 ? 1 : ks1 > 8 ? 8 : ks1;
            const int gran1 = w_dt == MOE_FP8_E4M3 ? 128 : 32;
            int chunk1 = (H + ks1 - 1) / ks1;
            chunk1 = (chunk1 + gran1 - 1) / gran1 * gran1;
            p.kchunk1 = chunk1;
            p.ksplit1 = (H + chunk1 - 1) / chunk1;
        }
        const long long waves = tiles_est * ((H + slice - 1) / slice);
        int ks = (int)((2048 + waves - 1) / (waves > 0 ? waves : 1));
        ks = ks < 1 ? 1 : ks > 8 ? 8 : ks;
        const int gran = w_dt == MOE_FP8_E4M3 ? 128 : 32;
        int chunk = (F + ks - 1) / ks;
        chunk = (chunk + gran - 1) / gran * gran;
        p.kchunk2 = chunk;
        p.ksplit2 = (F + chunk - 1) / chunk;
    }
    return p;
}

struct FfnWs {
    int32_t *tiles, *n_tiles, *group_tile_start;
    void *h;     // [rows][hw] SwiGLU activations
    void *part;  // Yp: [ksplit][rows][H] fp32 (row-streaming) or [rows][H] act_dt (tiled)
    float *part1;  // gate/up split-K partials [ksplit1][rows][2 hw] (g then u), or null
    uint8_t *xq, *hq;  // W8A8: E4M3 codes of the expert inputs [xrows][H] and of h [rows][hw]
    float *xs, *hs;    // and their per-row 128-column scales
    float *tail_part;  // tail split: partial sums and counters (or null)
    int32_t *tail_cnt;
};

// Weights of the optional extra group: the always-on shared expert run in
// the same grouped launch as the routed experts (same width F).
struct ExtraGroup {
    int rows = 0;
    const void *W1 = nullptr, *W3 = nullptr, *W2 = nullptr;
    const float *S1 = nullptr, *S3 = nullptr, *S2 = nullptr;
};

long long max_tiles_for(long long rows, int groups, int bm) { return (rows + bm - 1) / bm + groups; }

// xrows: rows of quantised expert input (W8A8 only).
size_t ffn_ws_carve(Carver &c, FfnWs &w, const FfnPlan &p, int rows, int groups, int H, int hw,
                    moe_dtype act_dt, int xrows) {
    const long long max_tiles = max_tiles_for(rows, groups, p.bm);
    w.tiles = static_cast<int32_t *>(c.take(sizeof(int32_t) * 4 * max_tiles));
    w.n_tiles = static_cast<int32_t *>(c.take(sizeof(int32_t)));
    w.group_tile_start = static_cast<int32_t *>(c.take(sizeof(int32_t) * (groups + 1)));
    w.h = c.take(dt_size(act_dt) * (size_t)rows * hw);
    w.part = p.tiled ? c.take(dt_size(act_dt) * (size_t)rows * H)
                     : c.take(sizeof(float) * (size_t)p.ksplit2 * rows * H);
    w.part1 = p.ksplit1 > 1 ? static_cast<float *>(c.take(sizeof(float) * (size_t)p.ksplit1 * rows * 2 * hw))
                            : nullptr;
    if (p.a8) {
        // codes per input row; scales per GEMM row, transposed [H/128][rows]
        w.xq = static_cast<uint8_t *>(c.take((size_t)xrows * H));
        w.xs = static_cast<float *>(c.take(sizeof(float) * (size_t)rows * (H / 128)));
        w.hq = static_cast<uint8_t *>(c.take((size_t)rows * hw));
        w.hs = static_cast<float *>(c.take(sizeof(float) * (size_t)rows * (hw / 128)));
    }
    if (p.tail) {
        w.tail_part = static_cast<float *>(c.take(tiled_tail_bytes(p.bm)));
        w.tail_cnt = static_cast<int32_t *>(c.take(sizeof(int32_t) * tiled_tail_counters));
    }
    return c.used;
}

GemmProblem base_problem(const FfnWs *ws, int G, int max_tiles, const ExtraGroup &ex, int extra_row0) {
    GemmProblem g{};
    g.tiles = ws ? ws->tiles : nullptr;
    g.n_tiles = ws ? ws->n_tiles : nullptr;
    g.group_tile_start = ws ? ws->group_tile_start : nullptr;
    g.n_groups = G + (ex.rows > 0 ? 1 : 0);
    g.max_tiles = max_tiles;
    g.extra_group = ex.rows > 0 ? G : -1;
    g.extra_row0 = extra_row0;
    g.tail_part = ws ? ws->tail_part : nullptr;
    g.tail_cnt = ws ? ws->tail_cnt : nullptr;
    return g;
}

// h[r] = silu(x_r W1) * (x_r W3) for M rows (routed rows, then extra rows).
GemmProblem gate_up_problem(const void *X, const int32_t *row_src, int gk, const FfnWs *ws, int G,
                            int max_tiles, int M, int H, int F, const void *W1, const void *W3,
                            const float *S1, const float *S3, const ExtraGroup &ex, int extra_row0,
                            void *h) {
    GemmProblem g = base_problem(ws, G, max_tiles, ex, extra_row0);
    g.A = X;
    g.row_src = row_src;
    g.gk = gk;
    g.lda = H;
    g.M = M;
    g.a_rows = row_src ? 0 : M;  // gathered: the caller knows X's rows
    g.N = F;
    g.K = H;
    g.B0 = W1;
    g.B1 = W3;
    g.tail_part = nullptr;  // the tail split is for down projections
    g.tail_cnt = nullptr;
    g.b_stride = (long long)H * F;
    g.S0 = S1;
    g.S1 = S3;
    g.s_stride = (long long)(H / 128) * (F / 128);
    g.Bx0 = ex.W1;
    g.Bx1 = ex.W3;
    g.Sx0 = ex.S1;
    g.Sx1 = ex.S3;
    g.C = h;
    g.ldc = F;
    g.c_split_stride = 0;
    g.ksplit = 1;
    g.kchunk = H;
    return g;
}

// Yp[r] = h[r] W2 for M rows.
GemmProblem down_problem(const void *h, const FfnWs *ws, int G, int max_tiles, int M, int H, int F,
                         const void *W2, const float *S2, const ExtraGroup &ex, int extra_row0, void *C,
                         long long split_stride, int ksplit, int kchunk) {
    GemmProblem g = base_problem(ws, G, max_tiles, ex, extra_row0);
    g.A = h;
    g.row_src = nullptr;
    g.gk = 1;
    g.lda = F;
    g.M = M;
    g.a_rows = M;
    g.N = H;
    g.K = F;
    g.B0 = W2;
    g.B1 = nullptr;
    g.b_stride = (long long)F * H;
    g.S0 = S2;
    g.s_stride = (long long)(F / 128) * (H / 128);
    g.Bx0 = ex.W2;
    g.Sx0 = ex.S2;
    g.C = C;
    g.ldc = H;
    g.c_split_stride = split_stride;
    g.ksplit = ksplit;
    g.kchunk = kchunk;
    return g;
}

// Split-K chunk (rounded to the kernel granule) for a fixed split count.
int chunk_for(int K, int nsplit, moe_dtype w_dt) {
    const int gran = w_dt == MOE_FP8_E4M3 ? 128 : 32;
    int c = (K + nsplit - 1) / nsplit;
    return (c + gran - 1) / gran * gran;
}

// MXFP4 expert strides: [K/2][N] packed code bytes and [K/32][N] scale bytes
void mxfp4_strides(GemmProblem &g) {
    g.b_stride = (long long)g.K / 2 * g.N;
    g.s_stride = (long long)(g.K / 32) * g.N;
}

hipError_t run_gemm(const FfnPlan &p, GemmProblem g, WType wt, bool swiglu, bool out_bf16, hipStream_t s) {
    if (wt == W_MXFP4) mxfp4_strides(g);
    if (p.a8) return out_bf16 ? launch_tiled_a8(g, swiglu, p.bm, s) : hipErrorInvalidValue;
    return p.tiled ? launch_tiled_gemm(g, wt, swiglu, out_bf16, p.bm, s)
                   : launch_stream_gemm(g, wt, swiglu, out_bf16, s);
}

// Row-streaming gate/up into h (rows x F, row stride F). With a split plan
// the GEMM writes fp32 partials of x W1 and x W3 and one pass sums them in
// fixed order and applies SwiGLU.
hipError_t run_gate_up_rows(const FfnPlan &p, GemmProblem g, const FfnWs &w, int rows, int F, WType wt,
                            moe_dtype act_dt, hipStream_t s) {
    if (wt == W_MXFP4) mxfp4_strides(g);
    if (p.ksplit1 <= 1) return launch_stream_gemm(g, wt, true, act_dt == MOE_BF16, s);
    void *h = g.C;
    g.C = w.part1;
    g.ldc = 2 * F;
    g.c_split_stride = (long long)rows * 2 * F;
    g.ksplit = p.ksplit1;
    g.kchunk = p.kchunk1;
    hipError_t e = launch_stream_gemm(g, wt, true, act_dt == MOE_BF16, s);
    if (e != hipSuccess) return e;
    return launch_swiglu_splits(w.part1, g.c_split_stride, p.ksplit1, rows, F, act_dt, h, s);
}

// W8A8 operands: A holds E4M3 codes of rows of `width` values; As their
// scales, transposed, one per GEMM row of `rows` and 128 columns.
void set_a8(GemmProblem &g, const uint8_t *q, const float *sc, int width, int rows) {
    g.A = q;
    g.lda = width;
    g.As = sc;
    g.as_ld = rows;
}

}  // namespace

extern "C" {

unsigned moe_debug_bounds(void) {
#ifdef MOE_BOUNDS_CHECK
    if (hipDeviceSynchronize() != hipSuccess) return ~0u;
    return bounds_take_tiled128() | bounds_take_tiled256() | bounds_take_tiledf32() | bounds_take_a8() |
           bounds_take_stream() | bounds_take_permute() | bounds_take_combine() | bounds_take_quant() |
           bounds_take_ep() | bounds_take_persist();
#else
    return 0u;
#endif
}

const char *moe_status_string(moe_status s) {
    switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: unsupported dtype or shape";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL: workspace too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP launch failed";
    case MOE_ERR_SCRATCH_LIMIT:
        return "MOE_ERR_SCRATCH_LIMIT: the layer's workspace exceeds the fixed scratch of moe_forward_noalloc";
    }
    return "unknown moe_status";
}

// ---------------------------------------------------------------------------
namespace {

// The router GEMM: for many bf16 tokens (and at least 16 experts) the
// LDS-tiled GEMM with 128-row tiles, split over h into at most 256
// workgroups (one round on the CUs) of at least 8 K steps; otherwise the row-streaming form, split so that
// enough wavefronts (16 rows x 64 experts each) keep the gate and token reads
// in flight, at least 4 K steps each.
struct RoutePlan {
    int ksplit, kchunk;
    bool tiled;
};

RoutePlan plan_route(int T, int H, int E, moe_dtype x_dt, moe_dtype wg_dt) {
    if (x_dt == MOE_BF16 && wg_dt == MOE_BF16 && T >= 512 && tiled_f32_supports(T, E, H, 1, H)) {
        const long long tiles = (((long long)T + 127) / 128) * (((long long)E + 255) / 256);
        long long ks = 256 / tiles;  // one workgroup per CU, one round
        long long max_ks = H / 256 > 0 ? H / 256 : 1;
        if (max_ks > 16) max_ks = 16;
        if (ks > max_ks) ks = max_ks;
        if (ks < 1) ks = 1;
        int chunk = (int)((H + ks - 1) / ks);
        chunk = (chunk + 31) / 32 * 32;
        return RoutePlan{(H + chunk - 1) / chunk, chunk, true};
    }
    long long base = (((long long)T + 15) / 16) * (((long long)E + 63) / 64);
    if (base < 1) base = 1;
    long long ks = (4096 + base - 1) / base;
    long long max_ks = H / 128 > 0 ? H / 128 : 1;
    if (max_ks > 16) max_ks = 16;
    if (ks > max_ks) ks = max_ks;
    if (ks < 1) ks = 1;
    int chunk = (int)((H + ks - 1) / ks);
    chunk = (chunk + 31) / 32 * 32;
    return RoutePlan{(H + chunk - 1) / chunk, chunk, false};
}

// split-K partials of the router; the larger of the two forms' needs, so the
// size depends on neither the token nor the gate dtype
size_t route_ws_bytes(int T, int H, int E) {
    size_t need = 0;
    for (moe_dtype dt : {MOE_BF16, MOE_F32}) {
        const RoutePlan r = plan_route(T, H, E, dt, dt);
        const size_t b = r.ksplit > 1 ? (size_t)r.ksplit * T * E * sizeof(float) : 0;
        if (b > need) need = b;
    }
    return need;
}

moe_status route_impl(const void *X, moe_dtype x_dt, const void *Wg, moe_dtype wg_dt, const float *gate_bias,
                      int T, int H, int E, int k, float *logits, int32_t *topk_idx, float *topk_w, void *ws,
                      hipStream_t stream) {
    const RoutePlan r = plan_route(T, H, E, x_dt, wg_dt);
    float *part = r.ksplit > 1 ? static_cast<float *>(ws) : logits;
    GemmProblem g{};
    g.extra_group = -1;
    g.A = X;
    g.gk = 1;
    g.lda = H;
    g.M = T;
    g.N = E;
    g.K = H;
    g.B0 = Wg;
    g.C = part;
    g.ldc = E;
    g.c_split_stride = (long long)T * E;
    g.ksplit = r.ksplit;
    g.kchunk = r.kchunk;
    if (r.tiled) MOE_TRY(launch_tiled_f32(g, stream));
    else {
        // fp32 gate against bf16 tokens: the higher-precision router
        const WType wt = x_dt == MOE_F32 ? W_F32 : (wg_dt == MOE_F32 ? W_F32_XBF16 : W_BF16);
        MOE_TRY(launch_stream_gemm(g, wt, false, false, stream));
    }
    return hip_status(launch_topk(part, r.ksplit, (long long)T * E, gate_bias, T, E, k, logits, topk_idx,
                                  topk_w, stream));
}

moe_status check_route(moe_dtype x_dt, moe_dtype wg_dt, int T, int H, int E, int k) {
    if (T < 0 || H < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
    if (!act_ok(x_dt)) return MOE_ERR_UNSUPPORTED;
    // the gate in the token dtype, or fp32 beside bf16 tokens
    if (wg_dt != x_dt && !(x_dt == MOE_BF16 && wg_dt == MOE_F32)) return MOE_ERR_UNSUPPORTED;
    if (E > 1024 || k > 64 || E % 4 || H % 32 || H > kMaxDim) return MOE_ERR_UNSUPPORTED;
    if ((long long)T * E > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

}  // namespace

size_t moe_route_workspace_bytes(int T, int H, int E) {
    if (T < 0 || H < 1 || E < 1 || E > 1024 || H > kMaxDim || (long long)T * E > 0x7fffffffLL) return 0;
    return align_up(route_ws_bytes(T, H, E));
}

moe_status moe_route(const void *X, moe_dtype x_dt, const void *Wg, moe_dtype wg_dt, const float *gate_bias,
                     int T, int H, int E, int k, float *logits, int32_t *topk_idx, float *topk_w, void *ws,
                     size_t ws_bytes, hipStream_t stream) {
    moe_status st = check_route(x_dt, wg_dt, T, H, E, k);
    if (st != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if (!X || !Wg || !logits || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
    const size_t need = route_ws_bytes(T, H, E);
    if (need && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    return route_impl(X, x_dt, Wg, wg_dt, gate_bias, T, H, E, k, logits, topk_idx, topk_w, ws, stream);
}

// ---------------------------------------------------------------------------
size_t moe_permute_workspace_bytes(int T, int k, int E) {
    if (T < 0 || k < 1 || E < 1) return 0;
    if ((long long)T * k > 0x7fffffffLL) return 0;  // moe_permute refuses such sizes
    return align_up(permute_ws_bytes(T * k, E));
}

moe_status moe_permute(const int32_t *topk_idx, int T, int k, int E, int32_t *counts,
                       int32_t *offsets, int32_t *row_src, int32_t *assign_row, const void *X,
                       moe_dtype x_dt, int H, void *Xp, void *ws, size_t ws_bytes,
                       hipStream_t stream) {
    if (T < 0 || k < 1 || E < 1 || k > E) return MOE_ERR_INVALID_ARG;
    if (E > 1024) return MOE_ERR_UNSUPPORTED;
    if ((long long)T * k > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!topk_idx || !counts || !offsets || !row_src || !assign_row) return MOE_ERR_INVALID_ARG;
    if (Xp) {
        if (!X || H < 1) return MOE_ERR_INVALID_ARG;
        if (!act_ok(x_dt)) return MOE_ERR_UNSUPPORTED;
        if ((H * dt_size(x_dt)) % 16) return MOE_ERR_UNSUPPORTED;
    }
    const size_t need = permute_ws_bytes(T * k, E);
    if (need && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    MOE_TRY(launch_permute(topk_idx, T * k, E, counts, offsets, row_src, assign_row, ws, stream));
    // rows past offsets[E] (assignments of experts outside [0, E)) stay unset
    if (Xp) MOE_TRY(launch_gather_rows(X, (int)dt_size(x_dt), H, row_src, k, T * k, Xp, stream, offsets + E));
    return MOE_OK;
}

// ---------------------------------------------------------------------------
size_t moe_grouped_ffn_workspace_bytes(int M, int G, int H, int F, moe_dtype act_dt,
                                       moe_dtype w_dt, moe_ffn_path path) {
    if (M < 0 || G < 1 || H < 1 || F < 1 || H > kMaxDim || F > kMaxDim) return 0;
    const FfnPlan p = plan_ffn(M, G, H, F, w_dt, path);
    Carver c(nullptr);
    FfnWs w{};
    size_t bytes = ffn_ws_carve(c, w, p, M, G, H, F, act_dt, M);
    FfnPlan q = p;  // the fp32 partials of the row-streaming form can be larger
    q.tiled = q.a8 = false;
    Carver c2(nullptr);
    const size_t b2 = ffn_ws_carve(c2, w, q, M, G, H, F, act_dt, M);
    return bytes > b2 ? bytes : b2;
}

moe_status moe_grouped_ffn(const void *Xin, const int32_t *row_src, int k, int M,
                           const int32_t *offsets, int G, int H, int F, const void *W1,
                           const void *W3, const void *W2, moe_dtype w_dt, const float *S1,
                           const float *S3, const float *S2, moe_dtype act_dt, void *Yp,
                           moe_ffn_path path, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (M < 0 || G < 1 || k < 1) return MOE_ERR_INVALID_ARG;
    if (!pair_ok(act_dt, w_dt)) return MOE_ERR_UNSUPPORTED;
    moe_status st = check_ffn_dims(H, F, w_dt);
    if (st != MOE_OK) return st;
    if (!path_ok(path)) return MOE_ERR_INVALID_ARG;
    if (path == MOE_PATH_TILED_A8 && w_dt != MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
    if (M == 0) return MOE_OK;
    if (!Xin || !offsets || !W1 || !W3 || !W2 || !Yp) return MOE_ERR_INVALID_ARG;
    const bool sc = scaled(w_dt);
    if (sc != (S1 != nullptr) || sc != (S3 != nullptr) || sc != (S2 != nullptr))
        return MOE_ERR_INVALID_ARG;
    const FfnPlan p = plan_ffn(M, G, H, F, w_dt, path);
    if ((path == MOE_PATH_TILED || path == MOE_PATH_TILED_A8) && !p.tiled) return MOE_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < moe_grouped_ffn_workspace_bytes(M, G, H, F, act_dt, w_dt, path))
        return MOE_ERR_WORKSPACE_TOO_SMALL;
    Carver c(ws);
    FfnWs w{};
    ffn_ws_carve(c, w, p, M, G, H, F, act_dt, M);
    const WType wt = wtype(w_dt);
    const bool bf = act_dt == MOE_BF16;
    const int max_tiles = (int)max_tiles_for(M, G, p.bm);
    const ExtraGroup none{};

    MOE_TRY(launch_build_tiles(offsets, G, 0, p.bm, w.tiles, w.n_tiles, w.group_tile_start, stream, w.tail_cnt,
                               w.tail_cnt ? tiled_tail_counters : 0));
    if (p.a8) {
        // E4M3 input rows (gathered here), gate/up writing E4M3 h, down
        ScaleLayout sl;  // the gathered rows' scales, transposed
        sl.ld = M;
        MOE_TRY(launch_quant_rows(Xin, H, row_src, k, M, H, w.xq, w.xs, stream, &sl));
        GemmProblem g1 = gate_up_problem(nullptr, nullptr, 1, &w, G, max_tiles, M, H, F, W1, W3, S1, S3, none, M,
                                         w.h);
        set_a8(g1, w.xq, w.xs, H, M);
        g1.Cq = w.hq;
        g1.Cqs = w.hs;
        g1.cqs_ld = M;
        MOE_TRY(run_gemm(p, g1, wt, true, true, stream));
        GemmProblem g2 = down_problem(nullptr, &w, G, max_tiles, M, H, F, W2, S2, none, M, Yp, 0, 1, F);
        set_a8(g2, w.hq, w.hs, F, M);
        MOE_TRY(run_gemm(p, g2, wt, false, true, stream));
        return MOE_OK;
    }
    GemmProblem g1 = gate_up_problem(Xin, row_src, k, &w, G, max_tiles, M, H, F, W1, W3, S1, S3, none, M, w.h);
    if (p.tiled) MOE_TRY(run_gemm(p, g1, wt, true, bf, stream));
    else MOE_TRY(run_gate_up_rows(p, g1, w, M, F, wt, act_dt, stream));
    if (p.tiled) {
        GemmProblem g2 = down_problem(w.h, &w, G, max_tiles, M, H, F, W2, S2, none, M, Yp, 0, 1, F);
        MOE_TRY(run_gemm(p, g2, wt, false, bf, stream));
    } else {
        const long long split_stride = (long long)M * H;
        GemmProblem g2 = down_problem(w.h, &w, G, max_tiles, M, H, F, W2, S2, none, M, w.part, split_stride,
                                      p.ksplit2, p.kchunk2);
        MOE_TRY(run_gemm(p, g2, wt, false, false, stream));
        MOE_TRY(launch_reduce_splits(static_cast<const float *>(w.part), split_stride, p.ksplit2, M, H,
                                     act_dt, Yp, stream));
    }
    return MOE_OK;
}

// ---------------------------------------------------------------------------
moe_status moe_quantize_e4m3_rows(const void *X, moe_dtype x_dt, long long ldx, const int32_t *row_src,
                                  int gk, int R, int C, uint8_t *Q, float *S, hipStream_t stream) {
    if (R < 0 || C < 1 || gk < 1 || ldx < C) return MOE_ERR_INVALID_ARG;
    if (x_dt != MOE_BF16 || C % 128 || ldx % 8) return MOE_ERR_UNSUPPORTED;
    if (R == 0) return MOE_OK;
    if (!X || !Q || !S) return MOE_ERR_INVALID_ARG;
    return hip_status(launch_quant_rows(X, ldx, row_src, gk, R, C, Q, S, stream));
}

// ---------------------------------------------------------------------------
moe_status moe_combine(const void *Yp, const int32_t *assign_row, const float *topk_w, int T, int k,
                       int H, const void *S, moe_dtype act_dt, void *Y, hipStream_t stream) {
    if (T < 0 || k < 1 || H < 1) return MOE_ERR_INVALID_ARG;
    if (!act_ok(act_dt)) return MOE_ERR_UNSUPPORTED;
    if (H % 4 || T > 65535) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!Yp || !assign_row || !topk_w || !Y) return MOE_ERR_INVALID_ARG;
    return hip_status(
        launch_combine(Yp, S, 0, 1, 1, act_dt, assign_row, topk_w, T, k, H, act_dt, Y, stream, (long long)T * k));
}

// ---------------------------------------------------------------------------
namespace {

moe_status check_desc(const moe_layer_desc *d) {
    if (!d) return MOE_ERR_INVALID_ARG;
    if (d->E < 1 || d->k < 1 || d->k > d->E || d->Fs < 0) return MOE_ERR_INVALID_ARG;
    if (!pair_ok(d->act_dt, d->w_dt)) return MOE_ERR_UNSUPPORTED;
    if (d->E > 1024 || d->k > 64 || d->E % 4) return MOE_ERR_UNSUPPORTED;
    moe_status st = check_ffn_dims(d->H, d->F, d->w_dt);
    if (st != MOE_OK) return st;
    // the shared expert: the routed experts' dtype, or bf16 beside fp8 or MXFP4
    if (d->Fs > 0 && d->ws_dt != d->w_dt && !(scaled(d->w_dt) && d->ws_dt == MOE_BF16))
        return MOE_ERR_UNSUPPORTED;
    if (d->Fs > 0 && (st = check_ffn_dims(d->H, d->Fs, d->ws_dt)) != MOE_OK) return st;
    if (!path_ok(d->path)) return MOE_ERR_INVALID_ARG;
    if (d->gate_f32 != 0 && d->gate_f32 != 1) return MOE_ERR_INVALID_ARG;
    // W8A8 takes an fp8 shared expert only inside its routed launches
    if (d->path == MOE_PATH_TILED_A8 &&
        (d->w_dt != MOE_FP8_E4M3 || (d->Fs > 0 && d->ws_dt == MOE_FP8_E4M3 && d->Fs != d->F)))
        return MOE_ERR_UNSUPPORTED;
    if (!d->Wg || !d->W1 || !d->W3 || !d->W2) return MOE_ERR_INVALID_ARG;
    const bool sc = scaled(d->w_dt);
    if (sc != (d->S1 != nullptr) || sc != (d->S3 != nullptr) || sc != (d->S2 != nullptr))
        return MOE_ERR_INVALID_ARG;
    if (d->Fs > 0) {
        const bool sfp8 = scaled(d->ws_dt);
        if (!d->Ws1 || !d->Ws3 || !d->Ws2) return MOE_ERR_INVALID_ARG;
        if (sfp8 != (d->Ss1 != nullptr) || sfp8 != (d->Ss3 != nullptr) || sfp8 != (d->Ss2 != nullptr))
            return MOE_ERR_INVALID_ARG;
    }
    return MOE_OK;
}

struct ForwardWs {
    float *logits, *w;
    int32_t *idx, *counts, *offsets, *row_src, *assign_row;
    void *perm_ws, *route_ws;
    FfnWs ffn;
    FfnPlan plan, plan_s;
    float *part1_s;  // split-K partials of a separate shared-expert gate/up, or null
    bool combined;   // shared expert runs as an extra group of the routed launches
    size_t bytes;
};

ForwardWs carve_forward(const moe_layer_desc *d, int T, void *base) {
    ForwardWs f{};
    Carver c(base);
    const int A = T * d->k;
    f.logits = static_cast<float *>(c.take(sizeof(float) * (size_t)T * d->E));
    f.w = static_cast<float *>(c.take(sizeof(float) * (size_t)A));
    f.idx = static_cast<int32_t *>(c.take(sizeof(int32_t) * (size_t)A));
    f.counts = static_cast<int32_t *>(c.take(sizeof(int32_t) * (size_t)d->E));
    f.offsets = static_cast<int32_t *>(c.take(sizeof(int32_t) * (size_t)(d->E + 1)));
    f.row_src = static_cast<int32_t *>(c.take(sizeof(int32_t) * (size_t)A));
    f.assign_row = static_cast<int32_t *>(c.take(sizeof(int32_t) * (size_t)A));
    f.perm_ws = c.take(permute_ws_bytes(A, d->E));
    f.route_ws = c.take(route_ws_bytes(T, d->H, d->E));
    f.combined = d->Fs > 0 && d->Fs == d->F && d->ws_dt == d->w_dt;
    // W8A8 keeps an fp8 shared expert inside the routed launches (a bf16
    // one runs on its own, on the bf16 path)
    f.plan = plan_ffn(A, d->E, d->H, d->F, d->w_dt, d->path,
                      d->Fs == 0 || f.combined || d->ws_dt == MOE_BF16);
    if (d->Fs > 0 && !f.combined) {
        // separate shared-expert launches; one Yp buffer holds routed rows
        // then shared rows, so both use one format
        f.plan_s = plan_ffn(T, 1, d->H, d->Fs, d->ws_dt, f.plan.tiled ? MOE_PATH_TILED : MOE_PATH_GEMV);
        if (f.plan_s.tiled != f.plan.tiled) {
            f.plan = plan_ffn(A, d->E, d->H, d->F, d->w_dt, MOE_PATH_GEMV);
            f.plan_s = plan_ffn(T, 1, d->H, d->Fs, d->ws_dt, MOE_PATH_GEMV);
        }
    }
    const int rows = A + (d->Fs > 0 ? T : 0);
    const int groups = d->E + (f.combined ? 1 : 0);
    const int hw = d->F > d->Fs ? d->F : d->Fs;
    // row-streaming: the routed and a separate shared down projection keep
    // their own split counts; the partial buffer holds the larger count
    FfnPlan carve = f.plan;
    const bool separate = d->Fs > 0 && !f.combined;
    if (separate && !f.plan.tiled && f.plan_s.ksplit2 > carve.ksplit2) carve.ksplit2 = f.plan_s.ksplit2;
    ffn_ws_carve(c, f.ffn, carve, rows, groups, d->H, hw, d->act_dt, T);
    f.part1_s = nullptr;
    if (separate && !f.plan_s.tiled && f.plan_s.ksplit1 > 1)
        f.part1_s = static_cast<float *>(c.take(sizeof(float) * (size_t)f.plan_s.ksplit1 * T * 2 * d->Fs));
    f.bytes = c.used;
    return f;
}

}  // namespace

size_t moe_forward_workspace_bytes(const moe_layer_desc *desc, int T) {
    // moe_forward takes at most 65535 tokens
    if (check_desc(desc) != MOE_OK || T < 0 || T > 65535) return 0;
    return carve_forward(desc, T, nullptr).bytes;
}

moe_status moe_forward(const moe_layer_desc *d, const void *X, int T, void *Y, void *ws,
                       size_t ws_bytes, hipStream_t stream, float *logits_out,
                       int32_t *topk_idx_out, float *topk_w_out, int32_t *counts_out,
                       hipEvent_t const *events) {
    auto mark = [&](int i) -> hipError_t {
        return (events && events[i]) ? hipEventRecord(events[i], stream) : hipSuccess;
    };
    moe_status st = check_desc(d);
    if (st != MOE_OK) return st;
    if (T < 0) return MOE_ERR_INVALID_ARG;
    if ((long long)T * d->k > 0x7fffffffLL || T > 65535) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!X || !Y) return MOE_ERR_INVALID_ARG;
    ForwardWs f = carve_forward(d, T, ws);
    if (!ws || ws_bytes < f.bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (logits_out) f.logits = logits_out;
    if (topk_idx_out) f.idx = topk_idx_out;
    if (topk_w_out) f.w = topk_w_out;
    if (counts_out) f.counts = counts_out;

    const int A = T * d->k, H = d->H, F = d->F, E = d->E;
    const WType wt = wtype(d->w_dt);
    // separate shared-expert launches
    const WType wts = wtype(d->Fs > 0 ? d->ws_dt : d->w_dt);
    const void *W1 = d->W1, *W3 = d->W3, *W2 = d->W2, *Ws1 = d->Ws1, *Ws3 = d->Ws3, *Ws2 = d->Ws2;
    const float *S1 = d->S1, *S3 = d->S3, *S2 = d->S2, *Ss1 = d->Ss1, *Ss3 = d->Ss3, *Ss2 = d->Ss2;
    const bool bf = d->act_dt == MOE_BF16;
    const FfnPlan &p = f.plan;
    const int rows = A + (d->Fs > 0 ? T : 0);
    const size_t hb = dt_size(d->act_dt);
    const int hw = d->F > d->Fs ? d->F : d->Fs;

    ExtraGroup ex{};
    if (f.combined) {
        ex.rows = T;
        ex.W1 = Ws1;
        ex.W3 = Ws3;
        ex.W2 = Ws2;
        ex.S1 = Ss1;
        ex.S3 = Ss3;
        ex.S2 = Ss2;
    }
    const int M = A + ex.rows;  // rows of the grouped launches
    const int max_tiles = (int)max_tiles_for(M, E + (f.combined ? 1 : 0), p.bm);

    MOE_TRY(mark(MOE_EV_START));
    // 1. router
    st = route_impl(X, d->act_dt, d->Wg, d->gate_f32 ? MOE_F32 : d->act_dt, d->gate_bias, T, H, E, d->k,
                    f.logits, f.idx, f.w, f.route_ws, stream);
    if (st != MOE_OK) return st;
    MOE_TRY(mark(MOE_EV_ROUTE));
    // 2. dispatch (the row gather is fused into the gate/up GEMM's loads);
    // a one-block permutation also writes the GEMMs' tile list
    TileRequest tr;
    tr.tiles = f.ffn.tiles;
    tr.n_tiles = f.ffn.n_tiles;
    tr.group_tile_start = f.ffn.group_tile_start;
    tr.extra_rows = ex.rows;
    tr.bm = p.bm;
    tr.zero = f.ffn.tail_cnt;
    tr.n_zero = f.ffn.tail_cnt ? tiled_tail_counters : 0;
    bool tiles_built = false;
    MOE_TRY(launch_permute(f.idx, A, E, f.counts, f.offsets, f.row_src, f.assign_row, f.perm_ws, stream, &tr,
                           &tiles_built));
    MOE_TRY(mark(MOE_EV_PERMUTE));
    // 3. expert FFN; with `combined` the shared expert is group E of the same launches
    if (!tiles_built)
        MOE_TRY(launch_build_tiles(f.offsets, E, ex.rows, p.bm, f.ffn.tiles, f.ffn.n_tiles,
                                   f.ffn.group_tile_start, stream, tr.zero, tr.n_zero));
    // W8A8: the token rows are quantised once (per-row scales, so the gather
    // in the GEMM's loads picks the same codes as quantising gathered rows)
    if (p.a8) {
        // the scales go, transposed, to the rows of each token's assignments
        // (and of its shared-expert row), where the GEMM's tiles read them
        ScaleLayout sl;
        sl.ld = M;
        sl.scatter = f.assign_row;
        sl.k = d->k;
        sl.extra0 = ex.rows > 0 ? A : -1;
        MOE_TRY(launch_quant_rows(X, H, nullptr, 1, T, H, f.ffn.xq, f.ffn.xs, stream, &sl));
    }
    MOE_TRY(mark(MOE_EV_SCHEDULE));
    GemmProblem g1 = gate_up_problem(X, f.row_src, d->k, &f.ffn, E, max_tiles, M, H, F, W1, W3, S1, S3, ex, A,
                                     f.ffn.h);
    g1.a_rows = T;  // token rows (bf16) or their E4M3 codes
    if (p.a8) {
        set_a8(g1, f.ffn.xq, f.ffn.xs, H, M);
        g1.Cq = f.ffn.hq;  // h leaves the gate/up GEMM as E4M3 codes
        g1.Cqs = f.ffn.hs;
        g1.cqs_ld = M;
    }
    if (p.tiled) MOE_TRY(run_gemm(p, g1, wt, true, bf, stream));
    else MOE_TRY(run_gate_up_rows(p, g1, f.ffn, M, F, wt, d->act_dt, stream));
    MOE_TRY(mark(MOE_EV_GATE_UP));
    void *h_s = static_cast<char *>(f.ffn.h) + hb * (size_t)A * hw;
    const ExtraGroup none{};
    if (d->Fs > 0 && !f.combined) {
        GemmProblem gs = gate_up_problem(X, nullptr, 1, nullptr, 1, 0, T, H, d->Fs, Ws1, Ws3, Ss1, Ss3, none, 0,
                                         h_s);
        if (f.plan_s.tiled) {
            MOE_TRY(run_gemm(f.plan_s, gs, wts, true, bf, stream));
        } else {
            // few rows: split over H like a small routed launch (own partials)
            FfnWs ws_s = f.ffn;
            ws_s.part1 = f.part1_s;
            MOE_TRY(run_gate_up_rows(f.plan_s, gs, ws_s, T, d->Fs, wts, d->act_dt, stream));
        }
    }
    MOE_TRY(mark(MOE_EV_SHARED_GATE_UP));
    const void *S = nullptr;
    long long split_stride = 0;
    int nsplit = 1, nsplit_s = 1;
    moe_dtype yp_dt = d->act_dt;
    if (p.tiled) {
        GemmProblem g2 = down_problem(f.ffn.h, &f.ffn, E, max_tiles, M, H, F, W2, S2, ex, A, f.ffn.part, 0, 1,
                                      F);
        if (p.a8) set_a8(g2, f.ffn.hq, f.ffn.hs, F, M);
        MOE_TRY(run_gemm(p, g2, wt, false, bf, stream));
        MOE_TRY(mark(MOE_EV_DOWN));
        void *Sp = static_cast<char *>(f.ffn.part) + hb * (size_t)A * H;
        if (d->Fs > 0 && !f.combined) {
            GemmProblem g2s = down_problem(h_s, nullptr, 1, 0, T, H, d->Fs, Ws2, Ss2, none, 0, Sp, 0, 1, d->Fs);
            MOE_TRY(run_gemm(f.plan_s, g2s, wts, false, bf, stream));
        }
        if (d->Fs > 0) S = Sp;
    } else {
        // every down projection writes all nsplit slices (an empty K range
        // writes zeros), so combine sums a fixed number of slices
        split_stride = (long long)rows * H;
        nsplit = p.ksplit2;
        nsplit_s = (d->Fs > 0 && !f.combined) ? f.plan_s.ksplit2 : nsplit;
        yp_dt = MOE_F32;
        GemmProblem g2 = down_problem(f.ffn.h, &f.ffn, E, max_tiles, M, H, F, W2, S2, ex, A, f.ffn.part,
                                      split_stride, nsplit, chunk_for(F, nsplit, d->w_dt));
        MOE_TRY(run_gemm(p, g2, wt, false, false, stream));
        MOE_TRY(mark(MOE_EV_DOWN));
        float *Sp = static_cast<float *>(f.ffn.part) + (size_t)A * H;
        if (d->Fs > 0 && !f.combined) {
            GemmProblem g2s = down_problem(h_s, nullptr, 1, 0, T, H, d->Fs, Ws2, Ss2, none, 0, Sp, split_stride,
                                           nsplit_s, chunk_for(d->Fs, nsplit_s, d->ws_dt));
            MOE_TRY(run_gemm(f.plan_s, g2s, wts, false, false, stream));
        }
        if (d->Fs > 0) S = Sp;
    }
    MOE_TRY(mark(MOE_EV_SHARED_DOWN));
    // 4. combine
    MOE_TRY(launch_combine(f.ffn.part, S, split_stride, nsplit, nsplit_s, yp_dt, f.assign_row, f.w, T, d->k, H,
                           d->act_dt, Y, stream, A));
    MOE_TRY(mark(MOE_EV_COMBINE));
    return MOE_OK;
}

}  // extern "C"
