// Internal helpers shared by the libmoe HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// Bounds-checked debug build (-DMOE_BOUNDS_CHECK, libmoe_debug.so). Kernels
// check the indices they address memory with; a failed check sets its bit in
// a flag of the source file (atomicOr, no trap) and the access is clamped in
// bounds. moe_debug_bounds() returns the union of every file's flags and
// clears them. In the release build the checks compile to nothing.
// ---------------------------------------------------------------------------
enum BoundsBit : unsigned {
    BOUNDS_TILE = 1u,        // tile record: group, first and end row
    BOUNDS_A_ROW = 2u,       // gathered input row of a GEMM
    BOUNDS_SCALE_ROW = 4u,   // activation-scale row of the W8A8 GEMM
    BOUNDS_TAIL_SLOT = 8u,   // tail-split partial slot or counter
    BOUNDS_PERM_ROW = 16u,   // permuted row of an assignment
    BOUNDS_COMBINE_ROW = 32u,  // Yp row read by combine
    BOUNDS_QUANT_ROW = 64u,  // scale row written by the quantiser
    BOUNDS_EP_ROW = 128u,    // row of an expert-parallel exchange
};
#ifdef MOE_BOUNDS_CHECK
namespace {
__device__ unsigned bounds_flag;  // this source file's failed checks
}
#define MOE_BOUNDS_FILE(tag)                                                        \
    unsigned bounds_take_##tag() {                                                  \
        unsigned v = 0;                                                             \
        if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(bounds_flag), sizeof(v)) != hipSuccess) \
            return ~0u;                                                             \
        const unsigned z = 0;                                                       \
        if (hipMemcpyToSymbol(HIP_SYMBOL(bounds_flag), &z, sizeof(z)) != hipSuccess)  \
            return ~0u;                                                             \
        return v;                                                                   \
    }
// true when cond fails (the caller then clamps the index)
#define MOE_BOUNDS_FAIL(cond, bit) (!(cond) ? (atomicOr(&bounds_flag, (unsigned)(bit)), true) : false)
#else
#define MOE_BOUNDS_FILE(tag) \
    unsigned bounds_take_##tag() { return 0u; }
#define MOE_BOUNDS_FAIL(cond, bit) false
#endif
unsigned bounds_take_tiled128();
unsigned bounds_take_tiled256();
unsigned bounds_take_tiledf32();
unsigned bounds_take_a8();
unsigned bounds_take_stream();
unsigned bounds_take_permute();
unsigned bounds_take_combine();
unsigned bounds_take_quant();
unsigned bounds_take_ep();
unsigned bounds_take_persist();

// ---------------------------------------------------------------------------
// Vector types for MFMA operands and wide loads
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// bf16 <-> f32 (bf16 is carried as raw uint16 bits)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even f32 -> bf16 bits; NaN stays NaN (quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
// Two f32 -> packed bf16 pair (round to nearest even: v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// silu(z) = z / (1 + e^-z), with the hardware exp2 and reciprocal
// (v_exp_f32, v_rcp_f32, about 1 ulp each: a few fp32 ulps in all, far below
// the bf16 rounding of h that follows) in 4 VALU instructions instead of a
// library exp and an IEEE divide (measured: the SwiGLU epilogues of the tiled
// kernels 2-10 % faster). Large negative z: e^-z = inf, 1 / inf = 0, z * 0 =
// -0 (the limit).
__device__ __forceinline__ float silu_f32(float z) {
    const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * z);
    return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// ---------------------------------------------------------------------------
// Block-wide exclusive scan of one int per thread (blockDim.x <= 1024,
// multiple of 64). `lds` must hold 16 ints. Returns the exclusive prefix;
// *total receives the block sum. Contains barriers: all threads must call.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int block_exclusive_scan(int v, int *lds, int *total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) lds[wid] = x;
    __syncthreads();
    if (wid == 0) {
        int s = lane < nw ? lds[lane] : 0;
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) {
            int y = __shfl_up(s, d, 64);
            if (lane >= d) s += y;
        }
        if (lane < 16) lds[lane] = s;  // inclusive prefix over waves
    }
    __syncthreads();
    int base = wid > 0 ? lds[wid - 1] : 0;
    *total = lds[nw - 1];
    __syncthreads();  // lds may be reused by the caller
    return base + x - v;
}

// ---------------------------------------------------------------------------
// Internal launchers (host side). All enqueue on `s` and return hipError_t.
// ---------------------------------------------------------------------------

// Weight element type of a GEMM: matches moe_dtype for the B operand.
// W_F32_XBF16: fp32 weights against bf16 token rows (the higher-precision
// router gate; row-streaming kernel, fp32 output only).
// W_MXFP4: E2M1 codes packed two K-consecutive values a byte ([K/2][N]) with
// one E8M0 scale per 32 K rows of a column ([K/32][N] bytes), decoded to bf16
// inside the row-streaming and the tiled kernels.
enum WType { W_F32 = 0, W_BF16 = 1, W_FP8 = 2, W_F32_XBF16 = 3, W_MXFP4 = 4 };

// Row-streaming grouped GEMM (small rows per group).
//   C[r, n] = sum_k A(r)[k] * B_g[k, n]   (PLAIN)      or
//   C[r, n] = silu(A(r) B0_g)[n] * (A(r) B1_g)[n]   (SWIGLU)
// A(r) = A[row_src[r]/gk] if row_src else A[r].
struct GemmProblem {
    const void *A;
    const int32_t *row_src;
    int gk;
    int lda;
    const int32_t *tiles;     // (group, row0, row_end, 0) per tile; NULL: one group of M rows
    const int32_t *n_tiles;   // device count of tiles
    const int32_t *group_tile_start;  // [n_groups+1] first tile of each group (tiled kernel)
    int n_groups;             // groups in the tile list (incl. the extra group)
    int max_tiles;            // host upper bound on tiles
    // optional extra group (the always-on shared expert run in the same
    // launch): its tiles carry group index extra_group; it uses the Bx/Sx
    // weights, and its input rows r map to A[r - extra_row0] (no row_src)
    int extra_group = -1;     // -1: none (never 0 by default: 0 is a real group)
    int extra_row0 = 0;
    const void *Bx0 = nullptr, *Bx1 = nullptr;
    const float *Sx0 = nullptr, *Sx1 = nullptr;
    int M, N, K;
    const void *B0, *B1;      // [G][K][N]
    long long b_stride;       // elements per group
    const float *S0, *S1;     // fp8 block scales [G][K/128][N/128]
    long long s_stride;
    void *C;                  // output rows; split s at C + s * c_split_stride
    int ldc;
    long long c_split_stride;
    int ksplit;
    int kchunk;               // K elements per split (multiple of 32, or 128 for fp8)
    // fp8 activations (W8A8 tiled path): A holds E4M3 codes (rows mapped
    // through row_src as for bf16) and As their scales, one per GEMM row r
    // and 128 K, transposed: As[kb * as_ld + r], as_ld >= M
    const float *As = nullptr;
    long long as_ld = 0;
    // W8A8 gate/up: when Cq is set, h is written as E4M3 codes (Cq, ldc bytes
    // a row) with one fp32 scale per row and 128 columns, transposed:
    // Cqs[(column / 128) * cqs_ld + row], instead of bf16 to C
    uint8_t *Cq = nullptr;
    float *Cqs = nullptr;
    long long cqs_ld = 0;
    // tail split (LDS-tiled plain GEMM with a tile list, bf16 and MXFP4 weights):
    // the items of each XCD's last, partial round are split over K; the parts
    // leave fp32 partial sums in tail_part (tiled_tail_bytes(bm) bytes) and
    // count themselves in tail_cnt (tiled_tail_counters ints, zero at launch
    // and left zero). NULL: no split.
    float *tail_part = nullptr;
    int32_t *tail_cnt = nullptr;
    // rows of A (the bounds-checked build's checks only; 0: not known)
    long long a_rows = 0;
};

hipError_t launch_stream_gemm(const GemmProblem &p, WType wt, bool swiglu, bool out_bf16,
                              hipStream_t s);
// h = silu(sum of G partials) * (sum of U partials), rows [M][2N] per split
hipError_t launch_swiglu_splits(const float *part, long long split_stride, int nsplit, int M, int N,
                                moe_dtype out_dt, void *out, hipStream_t s);

// Plain bf16 GEMM of M rows (no tile list, no gather) with fp32 output and
// split-K over blockIdx.y (C + s c_split_stride); every split non-empty.
bool tiled_f32_supports(int M, int N, int K, int ksplit, int kchunk);
hipError_t launch_tiled_f32(const GemmProblem &p, hipStream_t s);

// LDS-tiled grouped GEMM (many rows per group). Same problem statement;
// ksplit must be 1; bm (rows per tile) must be tiled_gemm_bm(wt, rows, groups) and
// the tile list must have been built with it. Returns hipErrorInvalidValue
// for unsupported shapes.
hipError_t launch_tiled_gemm(const GemmProblem &p, WType wt, bool swiglu, bool out_bf16, int bm,
                             hipStream_t s);
int tiled_gemm_bm(WType wt, long long rows, int groups);  // rows per tile for this row distribution
bool tiled_gemm_supports(WType wt, int N, int K);
// persistent form of the 256-row bf16 tiled GEMM (tiled_persist.hip): shapes
// it takes, and its launcher (N a multiple of the tile width)
bool tiled_persist_fits(const GemmProblem &p, WType wt, bool swiglu, int bm);
hipError_t launch_tiled_persist(const GemmProblem &p, bool swiglu, hipStream_t s);
// tail-split scratch of the tiled kernel: partial sums for tiles of bm rows,
// and the number of counters
size_t tiled_tail_bytes(int bm);
constexpr int tiled_tail_counters = 256;

// W8A8 variant of the LDS-tiled grouped GEMM (fp8 weights and fp8
// activations with per-row 128-column scales, p.As transposed by GEMM row):
// tiles of bm = 128 or 160 rows; output bf16, or E4M3 h with transposed
// scales (gate/up). Returns hipErrorInvalidValue for unsupported shapes.
hipError_t launch_tiled_a8(const GemmProblem &p, bool swiglu, int bm, hipStream_t s);
int tiled_a8_bm(long long rows, int groups);  // rows per W8A8 tile (160)
bool tiled_a8_supports(int N, int K);

// E4M3 quantisation of bf16 rows: for each row and 128-column group,
// s = amax / 448 (1 when amax is 0), q = E4M3(x / s) rounded to nearest even
// and saturated. Output row r reads X[row_src[r] / gk] (X[r] if row_src is
// NULL; row stride ldx elements) -> Q [R][C], S [R][C/128].
// Scale output layout (NULL: row-major S[R][C/128]): transposed,
// S[g * ld + row]; with `scatter`, input row r's scales go to rows
// scatter[r * k + j] (j < k) and, when extra0 >= 0, extra0 + r.
struct ScaleLayout {
    long long ld = 0;
    const int32_t *scatter = nullptr;
    int k = 0;
    int extra0 = -1;
};
hipError_t launch_quant_rows(const void *X, long long ldx, const int32_t *row_src, int gk, int R, int C,
                             uint8_t *Q, float *S, hipStream_t s, const ScaleLayout *sl = nullptr);

// Tile list (group, row0, row_end, 0) for G groups of rows given by offsets
// plus, when extra_rows > 0, group G = rows [offsets[G], offsets[G] +
// extra_rows); bm rows per tile. Also the first tile index of every group,
// [groups + 1] (optional).
hipError_t launch_build_tiles(const int32_t *offsets, int G, int extra_rows, int bm, int32_t *tiles,
                              int32_t *n_tiles, int32_t *group_tile_start, hipStream_t s,
                              int32_t *zero = nullptr, int n_zero = 0);

// Router top-k. logits[t,e] = sum_s part[s][t][e] (s ascending) + bias[e] is
// written to `logits`, then the k best are selected. part may alias logits
// when nsplit == 1.
hipError_t launch_topk(const float *part, int nsplit, long long split_stride, const float *bias,
                       int T, int E, int k, float *logits, int32_t *idx, float *w, hipStream_t s);

// Tile list requested from the permutation (same records as
// launch_build_tiles for the E expert groups plus an extra group of
// extra_rows rows).
struct TileRequest {
    int32_t *tiles = nullptr, *n_tiles = nullptr, *group_tile_start = nullptr;
    int extra_rows = 0, bm = 0;
    int32_t *zero = nullptr;  // n_zero ints cleared with the list (tail-split counters)
    int n_zero = 0;
};

// Permutation (count / scan / scatter) and optional row gather. With `tr`,
// a permutation that runs in one block also writes the tile list; then
// *tiles_built is set and no launch_build_tiles is needed.
size_t permute_ws_bytes(int A, int E);
hipError_t launch_permute(const int32_t *idx, int A, int E, int32_t *counts, int32_t *offsets,
                          int32_t *row_src, int32_t *assign_row, void *ws, hipStream_t s,
                          const TileRequest *tr = nullptr, bool *tiles_built = nullptr);
// Xp[r] = X[row_src[r] / gk] for r < A, or r < *n_rows when n_rows is given
hipError_t launch_gather_rows(const void *X, int elem_bytes, int H, const int32_t *row_src,
                              int gk, int A, void *Xp, hipStream_t s, const int32_t *n_rows = nullptr);

// Combine: Y[t] = sum_j w[t,j] * sum_{s<nsplit} Yp_s[assign_row[t*k+j]]
//               (+ sum_{s<nsplit_s} S_s[t]).
// in_dt/out_dt: MOE_F32 or MOE_BF16.
hipError_t launch_combine(const void *Yp, const void *S, long long split_stride, int nsplit, int nsplit_s,
                          moe_dtype in_dt, const int32_t *assign_row, const float *w, int T,
                          int k, int H, moe_dtype out_dt, void *Y, hipStream_t s, long long yp_rows = 0);

// Sum fp32 split partials [nsplit][M][N] into out [M][N] (f32 or bf16).
hipError_t launch_reduce_splits(const float *part, long long split_stride, int nsplit, int M,
                                int N, moe_dtype out_dt, void *out, hipStream_t s);

}  // namespace moe
