// LDS-tiled grouped GEMM for many rows per expert (prefill).
//
// The grouped GEMM of the page "MoE-推理部署" (operator section) and the page
// "MOE推理流程解析" §二/§三: every expert's block of rows runs in one launch,
// with row counts that differ per expert; §三 also asks that fusion keep
// intermediates out of HBM, so the row gather (permutation) is fused into the
// A-tile load and SwiGLU into the gate/up epilogue.
//
// Tile: BM rows (256, or 128 when experts hold few rows) x 256 B-columns x 64
// deep; 256 threads = 4 wavefronts in a 2 x 2 grid, each owning BM/2 rows x
// 128 B-columns (64 columns of each half, interleaved: columns 8j + 4wc + q).
//  * gate/up (SWIGLU): B-columns 0..127 are W1[:, n0:n0+128] and 128..255 are
//    W3[:, n0:n0+128]; a wavefront holds the W1 and W3 accumulators of the
//    same 64 output columns, so h = silu(g) * u is formed in registers.
//  * down (PLAIN): B-columns are W2[:, n0:n0+256].
// MI355X mapping:
//  * v_mfma_f32_16x16x32_bf16; a wavefront holds up to 256 fp32 accumulators
//    per lane (the unified 512-register file at one wavefront per SIMD).
//  * weights are [K][N] in HBM; each thread loads 8 K-rows x 8 columns
//    (16-byte rows, 256 contiguous bytes per 16 threads), transposes them in
//    registers with v_perm into K-contiguous column vectors and writes those
//    to LDS, so every MFMA operand is one ds_read_b128. The 16-byte chunk of
//    a B^T row is XOR-swizzled by its row index so both the transposing
//    writes and the operand reads spread over the LDS banks.
//  * fp8 E4M3 weights are decoded to f32 (v_cvt_pk_f32_fp8), multiplied by
//    their 128x128 block scale and rounded once to bf16 when staged.
//  * A rows are gathered through row_src while loading (the permuted token
//    matrix is never written).
//  * two LDS stages: the next K tile is loaded into registers during the
//    current tile's MFMAs and written to the other stage; one barrier per
//    K tile.
//  * tile order: the row tiles of one expert times a band of column tiles
//    are consecutive, and each XCD (own L2) takes a contiguous run of that
//    order, so an expert's weight tiles and its gathered rows are read from
//    beyond L2 about once. The real tile count is read on the device, so
//    surplus workgroups of the worst-case grid exit without unbalancing the
//    XCDs.
//  * the epilogue stages the bf16 tile in LDS and writes 16-byte rows.
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kBNH = 128;           // B-columns per half
constexpr int kBK = 64;             // K depth per tile
constexpr int kALD = kBK;           // LDS row stride (elements) of the A tile
constexpr int kLD = kBK + 8;        // LDS row stride (elements) of the B^T tile
constexpr int kCLD = 2 * kBNH + 8;  // LDS row stride of the output staging tile
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kBlocksPerXcd = 32;   // one block per CU (LDS-bound)

template <int BM>
struct Geo {
    static constexpr int a_elems = BM * kALD;
    static constexpr int b_elems = 2 * kBNH * kLD;
    static constexpr int stage = a_elems + b_elems;
    static constexpr int c_elems = BM * kCLD;
    static constexpr int lds = (2 * stage) > c_elems ? (2 * stage) : c_elems;
    static constexpr int mi = BM / 32;     // 16-row MFMA tiles per wavefront
    static constexpr int arows = BM / 32;  // A rows loaded per thread
};

// LDS layouts (chosen from bank-conflict counter measurements on gfx950):
//  * A tile: 128-byte rows, 16-byte chunk XOR (row & 7). Both the row-wise
//    writes and the 16-row operand reads are conflict-free.
//  * B^T tile: 144-byte rows, chunk XOR (n >> 4) & 7. Operand reads are
//    conflict-free when an MFMA tile's 16 columns are 8 apart (n = 8j + q),
//    which is how wavefronts map their columns below.
__device__ __forceinline__ int aswz(int r, int chunk) { return r * kALD + 8 * (chunk ^ (r & 7)); }
__device__ __forceinline__ int bswz(int n, int chunk) { return n * kLD + 8 * (chunk ^ ((n >> 4) & 7)); }
// B^T row (column of the half) read by lane-column j of MFMA tile ni of
// wavefront column wc: columns 8 apart.
__device__ __forceinline__ int bcol(int wc, int ni, int j) { return 8 * j + 4 * wc + ni; }

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

// Map this workgroup to (row tile, column tile) of the work order; false for
// surplus workgroups. Work order: for each group, for each band of gn column
// tiles, the group's row tiles x the band's column tiles (column fastest).
// XCD x (workgroup id mod 8) takes the contiguous run [x*per, (x+1)*per).
__device__ __forceinline__ bool pick_tile(const GemmProblem &p, int nN, int bm, int &mt, int &nt) {
    const int n_tiles = p.tiles ? *p.n_tiles : (p.M + bm - 1) / bm;
    const int n_work = n_tiles * nN;
    const int per = (n_work + kXcds - 1) / kXcds;
    const int slot = blockIdx.x / kXcds;
    if (slot >= per) return false;
    const int id = (blockIdx.x % kXcds) * per + slot;
    if (id >= n_work) return false;
    if (!p.tiles || !p.group_tile_start) {
        mt = id % n_tiles;
        nt = id / n_tiles;
        return true;
    }
    // group holding id: largest g with starts[g] * nN <= id (binary search)
    int lo = 0, hi = p.n_groups;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.group_tile_start[mid] * nN <= id) lo = mid;
        else hi = mid;
    }
    const int t0 = p.group_tile_start[lo];
    const int cnt = p.group_tile_start[lo + 1] - t0;  // > 0: id lies in this group
    int gn = (kBlocksPerXcd + cnt - 1) / cnt;
    if (gn > nN) gn = nN;
    const int j = id - t0 * nN;
    const int band = j / (cnt * gn);
    const int q = j - band * cnt * gn;
    const int width = min(gn, nN - band * gn);
    nt = band * gn + q % width;
    mt = t0 + q / width;
    return true;
}

template <int WT, bool SWIGLU, int BM>
__global__ __launch_bounds__(kThreads, 1) void tiled_gemm_kernel(GemmProblem p, int nN) {
    typedef Geo<BM> G;
    __shared__ __attribute__((aligned(16))) uint16_t lds[G::lds];

    int mt, nt;
    if (!pick_tile(p, nN, BM, mt, nt)) return;
    int g, row0, row_end;
    if (p.tiles) {
        g = p.tiles[4 * mt];
        row0 = p.tiles[4 * mt + 1];
        row_end = p.tiles[4 * mt + 2];
    } else {
        g = 0;
        row0 = mt * BM;
        row_end = min(row0 + BM, p.M);
    }
    const int n0 = SWIGLU ? nt * kBNH : nt * 2 * kBNH;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, wr = w >> 1, wc = w & 1;

    // ---- A loader: BM/32 rows x one 8-element K chunk per thread ----
    const int a_kc = tid & 7;
    const uint16_t *a_src[G::arows];
    bool a_ok[G::arows];
    const bool extra = g == p.extra_group;
#pragma unroll
    for (int q = 0; q < G::arows; ++q) {
        const int r = row0 + (tid >> 3) + 32 * q;
        a_ok[q] = r < row_end;
        long long src = 0;
        if (a_ok[q]) {
            if (extra && p.row_src) src = r - p.extra_row0;
            else src = p.row_src ? (long long)(p.row_src[r] / p.gk) : (long long)r;
        }
        a_src[q] = reinterpret_cast<const uint16_t *>(p.A) + src * p.lda + 8 * a_kc;
    }

    // ---- B loader: 8 K rows x 8 columns per thread ----
    const int b_cg = tid & 31, b_kg = tid >> 5;
    const int b_half = b_cg >> 4;
    const int b_col = (SWIGLU ? n0 : n0 + b_half * kBNH) + 8 * (b_cg & 15);
    const bool b_ok = b_col < p.N;
    typedef typename std::conditional<WT == W_FP8, uint8_t, uint16_t>::type E;
    const void *bsrc = extra ? ((SWIGLU && b_half) ? p.Bx1 : p.Bx0) : ((SWIGLU && b_half) ? p.B1 : p.B0);
    const E *b_base = reinterpret_cast<const E *>(bsrc) + (extra ? 0 : (long long)g * p.b_stride) + b_col;
    const float *b_scale = extra ? ((SWIGLU && b_half) ? p.Sx1 : p.Sx0) : ((SWIGLU && b_half) ? p.S1 : p.S0);
    const long long b_sidx = (extra ? 0 : (long long)g * p.s_stride) + (b_col >> 7);

    u32x4 a_reg[G::arows];
    u32x4 b_reg[8];   // bf16: 8 columns per K row
    u32x2 q_reg[8];   // fp8: 8 codes per K row (decoded when staged)
    float q_scale = 0.0f;

    auto load_tile = [&](int k0) {
#pragma unroll
        for (int q = 0; q < G::arows; ++q) {
            const bool ok = a_ok[q] && (k0 + 8 * a_kc < p.K);
            a_reg[q] = ok ? *reinterpret_cast<const u32x4 *>(a_src[q] + k0) : u32x4{};
        }
        const int kr0 = k0 + 8 * b_kg;
        if constexpr (WT == W_FP8) {
            q_scale = (b_ok && kr0 < p.K) ? b_scale[b_sidx + (long long)(kr0 >> 7) * (p.N >> 7)] : 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool ok = b_ok && (kr0 + i < p.K);
                q_reg[i] = ok ? *reinterpret_cast<const u32x2 *>(b_base + (long long)(kr0 + i) * p.N) : u32x2{};
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool ok = b_ok && (kr0 + i < p.K);
                b_reg[i] = ok ? *reinterpret_cast<const u32x4 *>(b_base + (long long)(kr0 + i) * p.N) : u32x4{};
            }
        }
    };

    auto store_tile = [&](int stage) {
        uint16_t *As = lds + stage * G::stage;
        uint16_t *Bs = As + G::a_elems;
        if constexpr (WT == W_FP8) {
#pragma unroll
            for (int i = 0; i < 8; ++i) b_reg[i] = fp8x8_scaled(q_reg[i], q_scale);
        }
#pragma unroll
        for (int q = 0; q < G::arows; ++q)
            *reinterpret_cast<u32x4 *>(As + aswz((tid >> 3) + 32 * q, a_kc)) = a_reg[q];
        // transpose 8 (K) x 8 (column) bf16 into 8 K-contiguous column vectors
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
            u32x4 v;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp)
                v[pp] = __builtin_amdgcn_perm(b_reg[2 * pp + 1][c >> 1], b_reg[2 * pp][c >> 1], sel);
            *reinterpret_cast<u32x4 *>(Bs + bswz(b_cg * 8 + c, b_kg)) = v;
        }
    };

    f32x4 acc[2][G::mi][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mi = 0; mi < G::mi; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) acc[h][mi][ni] = f32x4{};

    const int nk = (p.K + kBK - 1) / kBK;
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_tile((kt + 1) * kBK);
        const uint16_t *As = lds + cur * G::stage;
        const uint16_t *Bs = As + G::a_elems;
        // operand fragments of both 32-deep K steps; the second step's reads
        // are issued before the first step's MFMAs so LDS latency overlaps them
        bf16x8 af[2][G::mi], bfr[2][2][4];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int kc = ks * 4 + (lane >> 4);  // logical 8-wide K chunk
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    bfr[ks][h][ni] = *reinterpret_cast<const bf16x8 *>(
                        Bs + bswz(h * kBNH + bcol(wc, ni, lane & 15), kc));
#pragma unroll
            for (int mi = 0; mi < G::mi; ++mi)
                af[ks][mi] = *reinterpret_cast<const bf16x8 *>(As + aswz(wr * (BM / 2) + mi * 16 + (lane & 15), kc));
        }
        // keep all fragment reads ahead of the MFMAs (the scheduler would
        // otherwise sink each read next to its first use)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int mi = 0; mi < G::mi; ++mi)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        acc[h][mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks][mi], bfr[ks][h][ni],
                                                                                 acc[h][mi][ni], 0, 0, 0);
        // the other stage was last read before the previous barrier
        if (kt + 1 < nk) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: stage the bf16 tile in LDS, then 16-byte row stores ----
    uint16_t *Cs = lds;
    constexpr int W = SWIGLU ? kBNH : 2 * kBNH;  // output tile width
#pragma unroll
    for (int mi = 0; mi < G::mi; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wr * (BM / 2) + mi * 16 + 4 * (lane >> 4) + i;
                const int c = bcol(wc, ni, lane & 15);
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
    for (int idx = tid; idx < BM * chunks_per_row; idx += kThreads) {
        const int r = idx / chunks_per_row, cc = idx % chunks_per_row;
        const int row = row0 + r, col = n0 + 8 * cc;
        if (row < row_end && col < p.N)
            *reinterpret_cast<u32x4 *>(Cg + (long long)row * p.ldc + col) =
                *reinterpret_cast<const u32x4 *>(Cs + r * kCLD + 8 * cc);
    }
}

template <int WT, bool SWIGLU, int BM>
hipError_t launch_t(const GemmProblem &p, hipStream_t s) {
    const int W = SWIGLU ? kBNH : 2 * kBNH;
    const int nN = (p.N + W - 1) / W;
    const long long mt_cap = p.tiles ? p.max_tiles : (p.M + BM - 1) / BM;
    long long blocks = mt_cap * nN;
    blocks = (blocks + kXcds - 1) / kXcds * kXcds;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((tiled_gemm_kernel<WT, SWIGLU, BM>), dim3((unsigned)blocks), dim3(kThreads), 0, s, p, nN);
    return hipGetLastError();
}

template <int WT, int BM>
hipError_t launch_bm(const GemmProblem &p, bool swiglu, hipStream_t s) {
    return swiglu ? launch_t<WT, true, BM>(p, s) : launch_t<WT, false, BM>(p, s);
}

}  // namespace

int tiled_gemm_bm(long long rows, int groups) {
    // 256-row tiles once experts average >= 192 rows, else 128
    return (groups > 0 && rows >= 192LL * groups) ? 256 : 128;
}

bool tiled_gemm_supports(WType wt, int N, int K) {
    if (wt == W_F32) return false;
    if (N % 8 || K % 32) return false;
    if (wt == W_FP8 && (N % 128 || K % 128)) return false;
    return true;
}

hipError_t launch_tiled_gemm(const GemmProblem &p, WType wt, bool swiglu, bool out_bf16, int bm,
                             hipStream_t s) {
    // an extra group needs its own weights (and scales for fp8)
    if (p.extra_group >= 0 && (!p.Bx0 || (swiglu && !p.Bx1) || (wt == W_FP8 && (!p.Sx0 || (swiglu && !p.Sx1)))))
        return hipErrorInvalidValue;
    if (!out_bf16 || p.ksplit != 1 || !tiled_gemm_supports(wt, p.N, p.K)) return hipErrorInvalidValue;
    if (bm != 128 && bm != 256) return hipErrorInvalidValue;
    switch (wt) {
    case W_BF16:
        return bm == 256 ? launch_bm<W_BF16, 256>(p, swiglu, s) : launch_bm<W_BF16, 128>(p, swiglu, s);
    case W_FP8:
        return bm == 256 ? launch_bm<W_FP8, 256>(p, swiglu, s) : launch_bm<W_FP8, 128>(p, swiglu, s);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace moe
