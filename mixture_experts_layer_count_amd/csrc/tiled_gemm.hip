// LDS-tiled grouped GEMM for many rows per expert (prefill).
//
// The grouped GEMM of the page "MoE-推理部署" (operator section) and the page
// "MOE推理流程解析" §二/§三: every expert's block of rows runs in one launch,
// with row counts that differ per expert; §三 also asks that fusion keep
// intermediates out of HBM, so the row gather (permutation) is fused into the
// A-tile load and SwiGLU into the gate/up epilogue.
//
// Tile: 128 rows x 256 B-columns x 64 deep, 256 threads = 4 wavefronts in a
// 2 x 2 grid, each owning 64 rows x 128 columns (two 64-column halves).
//  * gate/up (SWIGLU): B-columns 0..127 are W1[:, n0:n0+128] and 128..255 are
//    W3[:, n0:n0+128]; a wavefront holds the W1 and W3 accumulators of the
//    same 64 output columns, so h = silu(g) * u is formed in registers.
//  * down (PLAIN): B-columns are W2[:, n0:n0+256].
// MI355X mapping:
//  * v_mfma_f32_16x16x32_bf16 throughout (fp32 accumulators: 128 per lane).
//  * weights are [K][N] in HBM; each thread loads 8 K-rows x 8 columns
//    (16-byte rows, 256 contiguous bytes per 16 threads), transposes them in
//    registers with v_perm into K-contiguous column fragments, and writes
//    those to LDS, so every MFMA operand is one ds_read_b128.
//  * fp8 E4M3 weights are decoded to f32 (v_cvt_pk_f32_fp8), multiplied by
//    their 128x128 block scale and rounded once to bf16 on the way in.
//  * A rows are gathered through row_src while loading (no permuted copy of
//    the tokens is ever written).
//  * next K tile is prefetched into registers during the MFMAs of the
//    current one (one LDS buffer, two blocks per CU).
//  * workgroups are remapped so that each XCD (own L2) receives a contiguous
//    range of tiles: consecutive tiles share one weight column tile across
//    the row tiles of an expert, so weights are read from HBM about once.
//  * the epilogue stages the bf16 tile in LDS and writes 16-byte rows.
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;       // rows per tile
constexpr int kBNH = 128;      // B-columns per half
constexpr int kBK = 64;        // K depth per tile
constexpr int kLD = kBK + 8;   // LDS row stride (elements) of the A and B^T tiles
constexpr int kCLD = 2 * kBNH + 8;  // LDS row stride of the output staging tile
constexpr int kAElems = kBM * kLD;
constexpr int kBElems = 2 * kBNH * kLD;
constexpr int kCElems = kBM * kCLD;
constexpr int kLdsElems = (kAElems + kBElems) > kCElems ? (kAElems + kBElems) : kCElems;
constexpr int kThreads = 256;
constexpr int kXcds = 8;

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// 8 fp8 codes (one K row, 8 columns) -> 8 bf16 of code * scale.
__device__ __forceinline__ u32x4 fp8x8_scaled(u32x2 q, float s) {
    u32x4 o;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(q[d], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(q[d], true);
        o[2 * d] = pack2(lo[0] * s, lo[1] * s);
        o[2 * d + 1] = pack2(hi[0] * s, hi[1] * s);
    }
    return o;
}

template <int WT, bool SWIGLU>
__global__ __launch_bounds__(kThreads, 2) void tiled_gemm_kernel(GemmProblem p, int n_ntiles,
                                                                 int mt_cap) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[kLdsElems];
    uint16_t *As = lds;
    uint16_t *Bs = lds + kAElems;

    // ---- tile selection (XCD-contiguous) ----
    const int nblk = gridDim.x;
    const int per = nblk / kXcds;
    const int lid = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    const int mt = lid % mt_cap;
    const int nt = lid / mt_cap;
    if (nt >= n_ntiles) return;
    int g, row0, row_end;
    if (p.tiles) {
        if (mt >= *p.n_tiles) return;
        g = p.tiles[2 * mt];
        row0 = p.tiles[2 * mt + 1];
        row_end = min(row0 + kBM, p.offsets[g + 1]);
    } else {
        g = 0;
        row0 = mt * kBM;
        if (row0 >= p.M) return;
        row_end = min(row0 + kBM, p.M);
    }
    const int n0 = SWIGLU ? nt * kBNH : nt * 2 * kBNH;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, wr = w >> 1, wc = w & 1;

    // ---- A loader: 4 rows x one 8-element K chunk per thread ----
    const int a_kc = tid & 7;
    const uint16_t *a_src[4];
    bool a_ok[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = row0 + (tid >> 3) + 32 * q;
        a_ok[q] = r < row_end;
        long long src = 0;
        if (a_ok[q]) src = p.row_src ? (long long)(p.row_src[r] / p.gk) : (long long)r;
        a_src[q] = reinterpret_cast<const uint16_t *>(p.A) + src * p.lda + 8 * a_kc;
    }

    // ---- B loader: 8 K rows x 8 columns per thread ----
    const int b_cg = tid & 31, b_kg = tid >> 5;
    const int b_half = b_cg >> 4;
    const int b_col = (SWIGLU ? n0 : n0 + b_half * kBNH) + 8 * (b_cg & 15);
    const bool b_ok = b_col < p.N;
    typedef typename std::conditional<WT == W_FP8, uint8_t, uint16_t>::type E;
    const E *b_base = reinterpret_cast<const E *>((SWIGLU && b_half) ? p.B1 : p.B0) +
                      (long long)g * p.b_stride + b_col;
    const float *b_scale = (SWIGLU && b_half) ? p.S1 : p.S0;
    const long long b_sidx = (long long)g * p.s_stride + (b_col >> 7);

    u32x4 a_reg[4];
    u32x4 b_reg[8];  // bf16: raw 8 columns per K row; fp8: scaled bf16

    auto load_tile = [&](int k0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool ok = a_ok[q] && (k0 + 8 * a_kc < p.K);
            a_reg[q] = ok ? *reinterpret_cast<const u32x4 *>(a_src[q] + k0) : u32x4{};
        }
        const int kr0 = k0 + 8 * b_kg;
        if constexpr (WT == W_FP8) {
            float s = 0.0f;
            if (b_ok && kr0 < p.K) s = b_scale[b_sidx + (long long)(kr0 >> 7) * (p.N >> 7)];
            u32x2 q8[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool ok = b_ok && (kr0 + i < p.K);
                q8[i] = ok ? *reinterpret_cast<const u32x2 *>(b_base + (long long)(kr0 + i) * p.N) : u32x2{};
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) b_reg[i] = fp8x8_scaled(q8[i], s);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool ok = b_ok && (kr0 + i < p.K);
                b_reg[i] = ok ? *reinterpret_cast<const u32x4 *>(b_base + (long long)(kr0 + i) * p.N) : u32x4{};
            }
        }
    };

    auto store_tile = [&]() {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<u32x4 *>(As + ((tid >> 3) + 32 * q) * kLD + 8 * a_kc) = a_reg[q];
        // transpose 8 (K) x 8 (column) bf16 into 8 K-contiguous column vectors
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
            u32x4 v;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp)
                v[pp] = __builtin_amdgcn_perm(b_reg[2 * pp + 1][c >> 1], b_reg[2 * pp][c >> 1], sel);
            *reinterpret_cast<u32x4 *>(Bs + (b_cg * 8 + c) * kLD + 8 * b_kg) = v;
        }
    };

    f32x4 acc[2][4][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) acc[h][mi][ni] = f32x4{};

    const int nk = (p.K + kBK - 1) / kBK;
    load_tile(0);
    store_tile();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) load_tile((kt + 1) * kBK);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 a[4], b[2][4];
            const int kof = ks * 32 + 8 * (lane >> 4);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                a[mi] = *reinterpret_cast<const bf16x8 *>(As + (wr * 64 + mi * 16 + (lane & 15)) * kLD + kof);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    b[h][ni] = *reinterpret_cast<const bf16x8 *>(
                        Bs + (h * kBNH + wc * 64 + ni * 16 + (lane & 15)) * kLD + kof);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        acc[h][mi][ni] =
                            __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi], b[h][ni], acc[h][mi][ni], 0, 0, 0);
        }
        __syncthreads();
        if (kt + 1 < nk) {
            store_tile();
            __syncthreads();
        }
    }

    // ---- epilogue: stage the bf16 tile in LDS, then 16-byte row stores ----
    uint16_t *Cs = lds;
    constexpr int W = SWIGLU ? kBNH : 2 * kBNH;  // output tile width
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wr * 64 + mi * 16 + 4 * (lane >> 4) + i;
                const int c = wc * 64 + ni * 16 + (lane & 15);
                if (SWIGLU) {
                    const float v = silu_f32(acc[0][mi][ni][i]) * acc[1][mi][ni][i];
                    Cs[r * kCLD + c] = __builtin_bit_cast(uint16_t, (__bf16)v);
                } else {
                    Cs[r * kCLD + c] = __builtin_bit_cast(uint16_t, (__bf16)acc[0][mi][ni][i]);
                    Cs[r * kCLD + kBNH + c] = __builtin_bit_cast(uint16_t, (__bf16)acc[1][mi][ni][i]);
                }
            }
    __syncthreads();
    constexpr int chunks_per_row = W / 8;
    uint16_t *Cg = reinterpret_cast<uint16_t *>(p.C);
    for (int idx = tid; idx < kBM * chunks_per_row; idx += kThreads) {
        const int r = idx / chunks_per_row, cc = idx % chunks_per_row;
        const int row = row0 + r, col = n0 + 8 * cc;
        if (row < row_end && col < p.N)
            *reinterpret_cast<u32x4 *>(Cg + (long long)row * p.ldc + col) =
                *reinterpret_cast<const u32x4 *>(Cs + r * kCLD + 8 * cc);
    }
}

template <int WT, bool SWIGLU>
hipError_t launch_t(const GemmProblem &p, hipStream_t s) {
    const int W = SWIGLU ? kBNH : 2 * kBNH;
    const int n_ntiles = (p.N + W - 1) / W;
    const int mt_cap = p.tiles ? p.max_tiles : (p.M + kBM - 1) / kBM;
    long long blocks = (long long)mt_cap * n_ntiles;
    blocks = (blocks + kXcds - 1) / kXcds * kXcds;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((tiled_gemm_kernel<WT, SWIGLU>), dim3((unsigned)blocks), dim3(kThreads), 0, s, p,
                       n_ntiles, mt_cap);
    return hipGetLastError();
}

}  // namespace

int tiled_gemm_bm() { return kBM; }

bool tiled_gemm_supports(WType wt, int N, int K) {
    if (wt == W_F32) return false;
    if (N % 8 || K % 32) return false;
    if (wt == W_FP8 && (N % 128 || K % 128)) return false;
    return true;
}

hipError_t launch_tiled_gemm(const GemmProblem &p, WType wt, bool swiglu, bool out_bf16, hipStream_t s) {
    if (!out_bf16 || p.ksplit != 1 || !tiled_gemm_supports(wt, p.N, p.K)) return hipErrorInvalidValue;
    switch (wt) {
    case W_BF16: return swiglu ? launch_t<W_BF16, true>(p, s) : launch_t<W_BF16, false>(p, s);
    case W_FP8: return swiglu ? launch_t<W_FP8, true>(p, s) : launch_t<W_FP8, false>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
