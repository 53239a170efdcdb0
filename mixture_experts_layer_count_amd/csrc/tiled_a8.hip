// W8A8 grouped GEMM for many rows per expert: fp8 (OCP E4M3) weights with
// 128x128 block scales times fp8 activations with per-row 128-column scales.
// build-flags: -mllvm -amdgpu-mfma-vgpr-form
// (MFMA results in architectural VGPRs, where the per-block scaling adds
// them to the accumulators.)
//
// Pages: the grouped GEMM of "MoE-推理部署" (operator section) and
// "MOE推理流程解析" §二/§三 (one launch for every expert's rows, gather fused
// into the A load); §三 also names quantising activations before the expert
// GEMM, which is what feeds this kernel; "MoE-推理部署" (expert-quantisation
// section) gives the per-expert FP8 weight scales.
//
// Math: C[r, n] = sum over 128-deep K blocks b of
//   sa[r, b] * sw[b, n / 128] * sum_{k in b} qa[r, k] * qw[k, n]
// One v_mfma_f32_16x16x128_f8f6f4 computes exactly one block's inner sum for
// a 16x16 output tile (fresh accumulator), which is then added to the result
// times sa * sw: the scales never meet a partial sum of another block.
//
// Tile: 128 rows x 128 B-columns x 128 deep; 4 wavefronts in a 2 x 2 grid,
// each 64 rows x 64 B-columns (4 x 4 MFMA tiles).
//  * gate/up (SWIGLU): B-columns 0..63 are W1[:, n0:n0+64], 64..127 are
//    W3[:, n0:n0+64]; output columns n0..n0+63 (h, bf16).
//  * down (PLAIN): B-columns are W2[:, n0:n0+128].
// Pipeline as in the bf16 ring kernel (tiled_gemm_kernel.h): global -> LDS
// copies (global_load_lds) into a ring of S stages with a fixed count of
// copies in flight, one barrier per K step, the next step's fragments read
// between the MFMA groups of the current one.
//  * A tile: 128-byte rows (128 codes), 16-byte chunk c of row r stored at
//    c ^ (r & 7); an operand is 32 consecutive codes (two ds_read_b128).
//  * B tile: [K][N] layout, 128-byte rows, chunk c of row k stored at
//    c ^ ((k >> 1) & 3) ^ (((k >> 5) & 1) << 2), so the two 16-lane groups of
//    a ds_read_b64_tr_b8 touch distinct banks; an operand is four
//    transposing reads (8 K rows each) of the lane's column.
//  * the activation scales of the tile's rows ride along with each stage
//    (gathered through row_src like the rows); the weight block scales too.
#include "tiled_gemm_kernel.h"

namespace moe {
namespace tiled {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kA8Threads = 256;  // 2 x 2 wavefronts of 64 x 64
constexpr int kA8BM = 128;
constexpr int kA8BN = 128;   // B-columns per tile
constexpr int kA8BK = 128;   // K per step = one scale block
constexpr int kA8Budget = 144 * 1024;

struct RingA8 {
    static constexpr int a_bytes = kA8BM * kA8BK;   // 16 KB
    static constexpr int b_bytes = kA8BK * kA8BN;   // 16 KB
    static constexpr int sa_bytes = 2 * kA8BM * 4;  // row scales (+ a duplicate half)
    static constexpr int sw_bytes = 4 * 256;        // per-wavefront weight scales
    static constexpr int stage = a_bytes + b_bytes + sa_bytes + sw_bytes;
    static constexpr int S = (kA8Budget / stage) < 8 ? (kA8Budget / stage) : 8;
    static constexpr int nA = a_bytes / (kA8Threads * 16);  // 4
    static constexpr int nB = b_bytes / (kA8Threads * 16);  // 4
    static constexpr int per_tile = nA + nB + 2;
};

template <bool SWIGLU>
struct OutA8 {
    static constexpr int width = SWIGLU ? 64 : 128;
    static constexpr int ld = width + 8;
};

__device__ __forceinline__ int bswz_a8(int k) { return ((k >> 1) & 3) ^ (((k >> 5) & 1) << 2); }

template <bool SWIGLU>
__global__ __launch_bounds__(kA8Threads, 1) void tiled_a8_kernel(GemmProblem p, int nN) {
    typedef RingA8 R;
    constexpr int S = R::S;
    constexpr int LDS = (R::S * R::stage) > kA8BM * OutA8<SWIGLU>::ld * 2 ? R::S * R::stage
                                                                          : kA8BM * OutA8<SWIGLU>::ld * 2;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS];

    int mt, nt;
    if (!pick_tile(p, nN, kA8BM, mt, nt)) return;
    int g, row0, row_end;
    if (p.tiles) {
        g = p.tiles[4 * mt];
        row0 = p.tiles[4 * mt + 1];
        row_end = p.tiles[4 * mt + 2];
    } else {
        g = 0;
        row0 = mt * kA8BM;
        row_end = min(row0 + kA8BM, p.M);
    }
    const int n0 = nt * OutA8<SWIGLU>::width;
    const bool extra = g == p.extra_group;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, wr = w >> 1, wc = w & 1;

    auto src_row = [&](int r) -> long long {
        if (r >= row_end) r = row0;  // padding rows read a valid row (never stored)
        if (extra && p.row_src) return r - p.extra_row0;
        return p.row_src ? (long long)(p.row_src[r] / p.gk) : (long long)r;
    };

    // ---- copy sources ----
    // A: copy q of wavefront w fills rows 8 (4w + q) .. +7; lane -> row lane/8,
    // physical chunk lane%8, i.e. logical chunk (lane%8) ^ (row & 7)
    const uint8_t *a_src[R::nA];
#pragma unroll
    for (int q = 0; q < R::nA; ++q) {
        const long long src = src_row(row0 + 8 * (w * R::nA + q) + (lane >> 3));
        a_src[q] = reinterpret_cast<const uint8_t *>(p.A) + src * p.lda + 16 * ((lane & 7) ^ ((lane >> 3) & 7));
    }
    // A scales: wavefronts 0/1 copy rows 0..63 / 64..127, 2/3 the same rows
    // into the duplicate half (unused), so every wavefront issues one copy
    const float *sa_src = p.As + src_row(row0 + 64 * (w & 1) + lane) * p.as_ld;
    // B: copy q of wavefront w fills K rows 8 (4w + q) .. +7; lane -> row
    // lane/8, physical chunk lane%8 holding data chunk (lane%8) ^ swizzle
    const uint8_t *b_src[R::nB];
    const void *B0 = extra ? p.Bx0 : p.B0;
    const void *B1 = extra ? p.Bx1 : p.B1;
    const long long gofs = extra ? 0 : (long long)g * p.b_stride;
#pragma unroll
    for (int q = 0; q < R::nB; ++q) {
        const int k = 8 * (w * R::nB + q) + (lane >> 3);
        const int c = (lane & 7) ^ bswz_a8(k);
        const void *base;
        int col;
        if (SWIGLU) { base = (c >> 2) ? B1 : B0; col = n0 + 16 * (c & 3); }
        else { base = B0; col = n0 + 16 * c; }
        if (col > p.N - 16) col = p.N - 16;
        b_src[q] = reinterpret_cast<const uint8_t *>(base) + gofs + (long long)k * p.N + col;
    }
    // weight block scales of this wavefront's columns: W1 / W3 of block
    // n0 / 128 (gate/up) or the W2 block of n0 + 64 wc (down)
    const float *sw_src;
    {
        const float *S0 = extra ? p.Sx0 : p.S0;
        const float *S1 = extra ? p.Sx1 : p.S1;
        const long long sofs = extra ? 0 : (long long)g * p.s_stride;
        if (SWIGLU) sw_src = ((lane & 1) ? S1 : S0) + sofs + (n0 >> 7);
        else sw_src = S0 + sofs + min((n0 + 64 * wc) >> 7, (p.N >> 7) - 1);
    }

    constexpr int NC = R::per_tile;
    auto copy = [&](int q, int kt, int stage) {
        uint8_t *st = lds + stage * R::stage;
        const int k0 = kt * kA8BK;
        if (q < R::nA) {
            copy16(a_src[q] + k0, st + (w * R::nA + q) * 1024);
        } else if (q < R::nA + R::nB) {
            const int qb = q - R::nA;
            copy16(b_src[qb] + (long long)k0 * p.N, st + R::a_bytes + (w * R::nB + qb) * 1024);
        } else if (q == R::nA + R::nB) {
            copy4(sa_src + kt, st + R::a_bytes + R::b_bytes + (w >> 1) * kA8BM * 4 + 64 * 4 * (w & 1));
        } else {
            copy4(sw_src + (long long)kt * (p.N >> 7), st + R::a_bytes + R::b_bytes + R::sa_bytes + w * 256);
        }
    };

    // ---- fragment reads: B blocks (4 transposing reads each), then A row
    // blocks (two 16-byte reads each), then the weight scales ----
    struct Frag {
        i32x8 a[4];
        i32x8 b[4];
        float s0, s1;
    };
    u32x2 raw[4][4];  // transposed reads of the set being loaded
    constexpr int NR = 16 + 4 + 1;
    const int i16 = lane & 15, gq = lane >> 4;
    const int a_row = wr * 64 + i16;  // + 16 m
    auto read = [&](Frag &f, int r, int stage) {
        const uint8_t *st = lds + stage * R::stage;
        if (r < 16) {
            const int j = r >> 2, t = r & 3;
            const int nb = SWIGLU ? 64 * (j >> 1) + 32 * wc + 16 * (j & 1) : 64 * wc + 16 * j;
            const int k = 32 * gq + 8 * t + (i16 >> 1);
            raw[j][t] = ds_tr8(lds_addr(st + R::a_bytes) + k * 128 + 16 * ((nb >> 4) ^ bswz_a8(k)) + 8 * (i16 & 1));
        } else if (r < 20) {
            const int m = r - 16;
            const int row = a_row + 16 * m;
            const uint8_t *base = st + row * 128;
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(base + 16 * ((2 * gq) ^ (row & 7)));
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(base + 16 * ((2 * gq + 1) ^ (row & 7)));
            f.a[m] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        } else {
            const float *sc = reinterpret_cast<const float *>(st + R::a_bytes + R::b_bytes + R::sa_bytes + w * 256);
            f.s0 = sc[0];
            f.s1 = sc[1];
        }
    };
    auto land = [&](Frag &f) {
        wait_lds();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int t = 0; t < 4; ++t) fence(raw[j][t]);
            f.b[j] = i32x8{(int)raw[j][0][0], (int)raw[j][0][1], (int)raw[j][1][0], (int)raw[j][1][1],
                           (int)raw[j][2][0], (int)raw[j][2][1], (int)raw[j][3][0], (int)raw[j][3][1]};
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[m][j] = f32x4{};

    // row block m of the current step: 4 MFMAs (one 128-deep block each),
    // added with scale sa[row] * sw[half]
    auto mma_rows = [&](const Frag &f, const f32x4 &sa, int m) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.a[m], f.b[j], f32x4{0, 0, 0, 0},
                                                                            0, 0, 0, 0, 0, 0);
            const float sw = (SWIGLU && j >= 2) ? f.s1 : f.s0;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m][j][i] = fmaf(t[i], sa[i] * sw, acc[m][j][i]);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // this lane's four row scales (rows 4 (lane/16) + i of row block m)
    auto read_sa = [&](f32x4 (&sa)[4], int stage) {
        const float *sc = reinterpret_cast<const float *>(lds + stage * R::stage + R::a_bytes + R::b_bytes);
#pragma unroll
        for (int m = 0; m < 4; ++m) sa[m] = *reinterpret_cast<const f32x4 *>(sc + wr * 64 + 16 * m + 4 * gq);
    };

    const int nk = p.K / kA8BK;
    Frag fa, fb;
#pragma unroll
    for (int t = 0; t < S; ++t)
#pragma unroll
        for (int q = 0; q < NC; ++q) copy(q, min(t, nk - 1), t);
    wait_vm<(S - 1) * R::per_tile>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < NR; ++r) read(fa, r, 0);
    land(fa);
    int stage = 0;
    for (int kt = 0; kt < nk; ++kt) {
        const int nstage = stage + 1 == S ? 0 : stage + 1;
        const int src = min(kt + S, nk - 1);
        // the row scales of tile kt, before the barrier lets its stage refill
        f32x4 sa[4];
        read_sa(sa, stage);
        mma_rows(fa, sa[0], 0);
        wait_vm<(S - 2) * R::per_tile>();
        wait_lds();  // the scale reads are done before anyone refills the stage
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int c = 0; c < 3; ++c) {
#pragma unroll
            for (int q = c * NC / 3; q < (c + 1) * NC / 3; ++q) copy(q, src, stage);
#pragma unroll
            for (int r = c * NR / 3; r < (c + 1) * NR / 3; ++r) read(fb, r, nstage);
            mma_rows(fa, sa[c + 1], c + 1);
        }
        land(fb);
        fa = fb;
        stage = nstage;
    }

    // ---- epilogue: bf16 tile through LDS, 16-byte row stores ----
    constexpr int LD = OutA8<SWIGLU>::ld;
    __syncthreads();
    uint16_t *Cs = reinterpret_cast<uint16_t *>(lds);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wr * 64 + m * 16 + 4 * gq + i;
            if (SWIGLU) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float v = silu_f32(acc[m][j][i]) * acc[m][j + 2][i];
                    Cs[r * LD + 32 * wc + 16 * j + i16] = __builtin_bit_cast(uint16_t, (__bf16)v);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    Cs[r * LD + 64 * wc + 16 * j + i16] = __builtin_bit_cast(uint16_t, (__bf16)acc[m][j][i]);
            }
        }
    __syncthreads();
    constexpr int W = OutA8<SWIGLU>::width;
    constexpr int chunks_per_row = W / 8;
    uint16_t *Cg = reinterpret_cast<uint16_t *>(p.C);
    for (int idx = tid; idx < kA8BM * chunks_per_row; idx += kA8Threads) {
        const int r = idx / chunks_per_row, cc = idx % chunks_per_row;
        const int row = row0 + r, col = n0 + 8 * cc;
        if (row < row_end && col < p.N)
            *reinterpret_cast<u32x4 *>(Cg + (long long)row * p.ldc + col) =
                *reinterpret_cast<const u32x4 *>(Cs + r * LD + 8 * cc);
    }
}

template <bool SWIGLU>
hipError_t launch_a8(const GemmProblem &p, hipStream_t s) {
    const int W = OutA8<SWIGLU>::width;
    const int nN = (p.N + W - 1) / W;
    const long long mt_cap = p.tiles ? p.max_tiles : (p.M + kA8BM - 1) / kA8BM;
    long long blocks = mt_cap * nN;
    blocks = (blocks + kXcds - 1) / kXcds * kXcds;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((tiled_a8_kernel<SWIGLU>), dim3((unsigned)blocks), dim3(kA8Threads), 0, s, p, nN);
    return hipGetLastError();
}

}  // namespace
}  // namespace tiled

bool tiled_a8_supports(int N, int K) { return N >= 128 && N % 128 == 0 && K >= 128 && K % 128 == 0; }

hipError_t launch_tiled_a8(const GemmProblem &p, bool swiglu, hipStream_t s) {
    if (p.extra_group >= 0 && (!p.Bx0 || !p.Sx0 || (swiglu && (!p.Bx1 || !p.Sx1)))) return hipErrorInvalidValue;
    if (!p.As || p.as_ld < p.K / 128 || p.ksplit != 1 || !tiled_a8_supports(p.N, p.K) || !p.S0 ||
        (swiglu && (!p.B1 || !p.S1)))
        return hipErrorInvalidValue;
    return swiglu ? tiled::launch_a8<true>(p, s) : tiled::launch_a8<false>(p, s);
}

}  // namespace moe
