// Row-streaming grouped GEMM for few rows per expert (decode).
//
// The decode case of the grouped expert computation (page "MoE-推理部署",
// operator section: with one or two tokens per expert the fused MoE kernel is
// in effect a batched GEMV and needs its own tile strategy; page
// "MOE推理流程解析" §二: grouped GEMM runs every expert's row block in one
// launch). Each wavefront owns one (expert row tile of 16 rows, 64-column
// (fp8: 128-column) slice of the weight) pair and streams that slice of the expert's weights
// from HBM exactly once, over its K range. Only experts that received rows
// produce tiles, so untouched experts' weights are never read.
//
// MI355X mapping:
//  * the weight matrices are stored [K][N] (N contiguous). A lane loads 4
//    (fp8: 8) consecutive columns from 8 consecutive K rows; v_perm packs them into
//    K-contiguous bf16 pairs, which is exactly the B operand layout of
//    v_mfma_f32_16x16x32_bf16 (no LDS round trip).
//  * the token rows (<= 16, zero-padded) are the A operand, read directly in
//    their natural K-contiguous layout, gathered through row_src.
//  * fp8 E4M3 weights are loaded 8 columns (8 bytes) a lane, decoded to bf16
//    in registers (v_cvt_scalef32_pk_bf16_fp8, scale 1: exact) and multiplied
//    on the bf16 MFMA. The fp32 block scale of the step's 128x128 block is
//    folded into the token fragment (x * s rounded once to bf16), so the
//    MFMAs accumulate in place; that frees the registers that let two
//    wavefronts share a SIMD (DeepSeek-shaped decode layer 1.75 -> 1.59 ms).
//  * every form but the all-fp32 one is built for two wavefronts per SIMD
//    (at most 256 registers a lane), so one wavefront's loads are in flight
//    while the other multiplies.
//  * f32 weights use v_mfma_f32_16x16x4_f32 with no transpose.
//  * a ring of register stages keeps the weight, token and scale loads of
//    the next K steps in flight while the current step is multiplied.
#include "common.h"

namespace moe {

MOE_BOUNDS_FILE(stream)
namespace {

constexpr int kWaves = 4;   // wavefronts per block (at most)
constexpr int kBM = 16;     // rows per tile
// weight columns per lane: 8 for fp8 (8-byte loads, the same bytes per load
// instruction as bf16), else 4; a wavefront slice is 16 lanes wide
template <int WT> constexpr int vec_of() { return WT == W_FP8 || WT == W_MXFP4 ? 8 : 4; }
template <int WT> constexpr int slice_of() { return 16 * vec_of<WT>(); }

template <int WT> struct WTraits;
template <> struct WTraits<W_BF16> {
    typedef uint16_t elem;
    typedef u32x2 raw;  // 4 columns
    typedef uint16_t act;
};
template <> struct WTraits<W_FP8> {
    typedef uint8_t elem;
    typedef u32x2 raw;  // 8 columns
    typedef uint16_t act;
};
template <> struct WTraits<W_F32> {
    typedef float elem;
    typedef f32x4 raw;  // 4 columns
    typedef float act;
};
template <> struct WTraits<W_F32_XBF16> {
    typedef float elem;
    typedef f32x4 raw;  // 4 columns
    typedef uint16_t act;
};
template <> struct WTraits<W_MXFP4> {
    typedef uint8_t elem;
    typedef u32x2 raw;  // 8 columns of one K-pair row (8 K rows per lane: 4 raws)
    typedef uint16_t act;
};
// per-step scale operand of a lane: fp8's 128x128 block scale, or the E8M0
// bytes of MXFP4's 8 columns for the step's 32-deep block
template <int WT> struct ScaleOf { typedef float type; };
template <> struct ScaleOf<W_MXFP4> { typedef u32x2 type; };
// weight rows (raws) a lane loads per 32-deep step: 8 K rows, or 4 K-pair
// rows for MXFP4
template <int WT> constexpr int rows_of() { return WT == W_MXFP4 ? 4 : 8; }
// K values per stored weight row
template <int WT> constexpr int kpack_of() { return WT == W_MXFP4 ? 2 : 1; }

// Pack element `c` (0..3) of 8 consecutive K rows (each row: 4 bf16 columns
// in two dwords) into a K-contiguous bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8 column_frag(const u32x2 (&r)[8], int c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    u32x4 v;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t lo = (c < 2) ? r[2 * p].x : r[2 * p].y;
        const uint32_t hi = (c < 2) ? r[2 * p + 1].x : r[2 * p + 1].y;
        v[p] = __builtin_amdgcn_perm(hi, lo, sel);
    }
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t q) {
    u32x2 o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, 1.0f, false));
    o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, 1.0f, true));
    return o;
}

// Weight rows are read exactly once per launch: non-temporal loads (the nt
// cache policy) keep them from displacing reused lines in L2 and the Infinity
// Cache. Measured: Mixtral-shaped decode layer 0.487 -> 0.439 ms, Qwen3-shaped
// 0.211 -> 0.191 ms, DeepSeek-shaped 1.81 -> 1.74 ms.
template <int WT>
__device__ __forceinline__ void load_rows(typename WTraits<WT>::raw (&r)[rows_of<WT>()],
                                          const typename WTraits<WT>::elem *B, long long ldb,
                                          bool ok) {
    typedef typename WTraits<WT>::raw R;
#pragma unroll
    for (int i = 0; i < rows_of<WT>(); ++i) {
        if (ok) r[i] = __builtin_nontemporal_load(reinterpret_cast<const R *>(B + i * ldb));
        else r[i] = R{};
    }
}

// One K step (32 deep) of acc[c] += A * B[:, c] for the wave's column tiles
// (fp8: times the step's 128x128 block scale s).
template <int WT>
__device__ __forceinline__ void mma_step(f32x4 (&acc)[vec_of<WT>()],
                                         const typename WTraits<WT>::raw (&r)[rows_of<WT>()], const void *afrag,
                                         typename ScaleOf<WT>::type s);

template <>
__device__ __forceinline__ void mma_step<W_BF16>(f32x4 (&acc)[4], const u32x2 (&r)[8], const void *afrag,
                                                 float) {
    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(afrag);
#pragma unroll
    for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, column_frag(r, c), acc[c], 0, 0, 0);
}

// fp8: the step's block scale s multiplies the token fragment (x * s rounded
// once to bf16) and the exactly decoded codes multiply that, accumulating in
// place: no per-step products or per-block partial sums take registers
template <>
__device__ __forceinline__ void mma_step<W_FP8>(f32x4 (&acc)[8], const u32x2 (&q)[8], const void *afrag,
                                                float s) {
    const u32x4 av = *reinterpret_cast<const u32x4 *>(afrag);
    u32x4 sv;
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = pack_bf16x2(bf16_lo(av[i]) * s, bf16_hi(av[i]) * s);
    const bf16x8 a = __builtin_bit_cast(bf16x8, sv);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        u32x2 r[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = fp8x4_to_bf16x4(h ? q[i].y : q[i].x);
#pragma unroll
        for (int c = 0; c < 4; ++c)
            acc[4 * h + c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, column_frag(r, c), acc[4 * h + c], 0, 0, 0);
    }
}

template <>
__device__ __forceinline__ void mma_step<W_F32>(f32x4 (&acc)[4], const f32x4 (&r)[8], const void *afrag,
                                                float) {
    const float *a = reinterpret_cast<const float *>(afrag);
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], r[s][c], acc[c], 0, 0, 0);
}

// fp32 weights against bf16 token rows: the 8 token values widen exactly to
// fp32 (a bf16 value is the high half of its fp32 bit pattern) and take the
// fp32 matrix-core steps of the all-fp32 form
template <>
__device__ __forceinline__ void mma_step<W_F32_XBF16>(f32x4 (&acc)[4], const f32x4 (&r)[8], const void *afrag,
                                                      float) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(afrag);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const uint32_t w = v[s >> 1];
        const float a = __uint_as_float((s & 1) ? (w & 0xffff0000u) : (w << 16));
#pragma unroll
        for (int c = 0; c < 4; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, r[s][c], acc[c], 0, 0, 0);
    }
}

// MXFP4: byte c of K-pair row j holds K rows 2j, 2j + 1 of the lane's column
// c, so converting byte c of rows 0..3 (the conversion selects the byte) gives
// the column's 8 consecutive K values as four bf16 pairs, each times the
// column's E8M0 scale (the conversion takes only the scale's exponent: exact).
// s holds the 8 scale bytes of the lane's columns for this 32-deep block.
// Eight columns a lane make each row segment of a wavefront 128 contiguous
// bytes: whole lines.
template <int B>
__device__ __forceinline__ bf16x8 mxfp4_column(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3, float sc) {
    u32x4 v;
    v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r0, sc, B));
    v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r1, sc, B));
    v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r2, sc, B));
    v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r3, sc, B));
    return __builtin_bit_cast(bf16x8, v);
}

template <int C>
__device__ __forceinline__ void mxfp4_mma(f32x4 (&acc)[8], const u32x2 (&r)[4], const bf16x8 &a, u32x2 s) {
    constexpr int B = C & 3;
    const uint32_t sw = C < 4 ? s.x : s.y;
    const float sc = __uint_as_float(((sw >> (8 * B)) & 0xffu) << 23);
    const bf16x8 b = C < 4 ? mxfp4_column<B>(r[0].x, r[1].x, r[2].x, r[3].x, sc)
                           : mxfp4_column<B>(r[0].y, r[1].y, r[2].y, r[3].y, sc);
    acc[C] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[C], 0, 0, 0);
}

template <>
__device__ __forceinline__ void mma_step<W_MXFP4>(f32x4 (&acc)[8], const u32x2 (&r)[4], const void *afrag,
                                                  u32x2 s) {
    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(afrag);
    mxfp4_mma<0>(acc, r, a, s);
    mxfp4_mma<1>(acc, r, a, s);
    mxfp4_mma<2>(acc, r, a, s);
    mxfp4_mma<3>(acc, r, a, s);
    mxfp4_mma<4>(acc, r, a, s);
    mxfp4_mma<5>(acc, r, a, s);
    mxfp4_mma<6>(acc, r, a, s);
    mxfp4_mma<7>(acc, r, a, s);
}

// A fragment: 8 consecutive K values of the lane's row (bf16: 16 B, f32: 32 B).
template <int WT> struct AFrag;
template <> struct AFrag<W_BF16> { u32x4 v; };
template <> struct AFrag<W_FP8> { u32x4 v; };
template <> struct AFrag<W_F32> { f32x4 v[2]; };
template <> struct AFrag<W_F32_XBF16> { u32x4 v; };
template <> struct AFrag<W_MXFP4> { u32x4 v; };

template <int WT>
__device__ __forceinline__ void load_a(AFrag<WT> &f, const typename WTraits<WT>::act *p, bool ok) {
    if constexpr (WT == W_F32) {
        if (ok) {
            f.v[0] = *reinterpret_cast<const f32x4 *>(p);
            f.v[1] = *reinterpret_cast<const f32x4 *>(p + 4);
        } else {
            f.v[0] = f32x4{};
            f.v[1] = f32x4{};
        }
    } else {
        f.v = ok ? *reinterpret_cast<const u32x4 *>(p) : u32x4{};
    }
}

// K steps held in the register ring (kDepth - 1 in flight while one is
// multiplied), chosen by measurement: 3 for bf16 gate/up (two wavefronts per
// SIMD), 4 for the single-matrix bf16 down projection; fp8 steps are twice as
// wide (8 columns a lane), best at 2 for gate/up and 3 for down.
// MXFP4 steps carry half of fp8's weight bytes (8 columns, K in pairs): best at 4 and 6.
template <int WT, bool SWIGLU> constexpr int ring_depth() {
    return WT == W_MXFP4 ? (SWIGLU ? 4 : 6) : !SWIGLU ? (WT == W_FP8 ? 3 : 4) : (WT == W_FP8 ? 2 : 3);
}

// One K step's operands for one lane: weight rows of both matrices, the token
// fragment and (fp8) the block scales of the step's 128-deep K block.
template <int WT, bool SWIGLU>
struct Stage {
    typename WTraits<WT>::raw w0[rows_of<WT>()];
    typename WTraits<WT>::raw w1[SWIGLU ? rows_of<WT>() : 1];
    AFrag<WT> a;
    typename ScaleOf<WT>::type s0, s1;
};

template <int WT, bool SWIGLU, bool OUT_BF16>
__device__ __forceinline__ void stream_gemm_body(const GemmProblem &p, int n_slices) {
    typedef typename WTraits<WT>::elem E;
    typedef typename WTraits<WT>::act AT;
    constexpr int kDepth = ring_depth<WT, SWIGLU>();

    const int lane = threadIdx.x & 63;
    const long long wave = (long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int mt = (int)(wave / n_slices);
    const int ns = (int)(wave - (long long)mt * n_slices);
    const int split = blockIdx.y;

    int g, row0, row_end;
    if (p.tiles) {
        if (mt >= p.max_tiles || mt >= *p.n_tiles) return;
        g = p.tiles[4 * mt];
        row0 = p.tiles[4 * mt + 1];
        row_end = p.tiles[4 * mt + 2];
        if (MOE_BOUNDS_FAIL(g >= 0 && g < p.n_groups && row0 >= 0 && row0 < row_end && row_end <= p.M,
                            BOUNDS_TILE))
            return;
    } else {
        g = 0;
        row0 = mt * kBM;
        if (row0 >= p.M) return;
        row_end = min(row0 + kBM, p.M);
    }

    const int kg = lane >> 4;
    constexpr int KV = vec_of<WT>();
    const int col = ns * slice_of<WT>() + KV * (lane & 15);
    const bool colok = col < p.N;
    const int kbeg = split * p.kchunk;
    const int kend = min(p.K, kbeg + p.kchunk);
    const int nsteps = kend > kbeg ? (kend - kbeg) / 32 : 0;

    // this lane's activation row (MFMA A operand row = lane & 15)
    const int r = row0 + (lane & 15);
    const bool rok = r < row_end;
    const bool extra = g == p.extra_group;
    long long arow = 0;
    if (rok) {
        if (extra && p.row_src) arow = r - p.extra_row0;
        else arow = p.row_src ? (long long)(p.row_src[r] / p.gk) : (long long)r;
        if (MOE_BOUNDS_FAIL(arow >= 0 && (p.a_rows <= 0 || arow < p.a_rows), BOUNDS_A_ROW)) arow = 0;
    }
    const AT *Ap = reinterpret_cast<const AT *>(p.A) + arow * p.lda + 8 * kg + kbeg;

    const long long ldb = p.N;
    const long long goff = extra ? 0 : (long long)g * p.b_stride;
    constexpr int KP = kpack_of<WT>();  // K values per stored weight row
    const long long brow = (8 * kg + kbeg) / KP;
    const E *B0 = reinterpret_cast<const E *>(extra ? p.Bx0 : p.B0) + goff + col + brow * ldb;
    const E *B1 = SWIGLU ? reinterpret_cast<const E *>(extra ? p.Bx1 : p.B1) + goff + col + brow * ldb
                         : nullptr;
    const float *S0p = extra ? p.Sx0 : p.S0;
    const float *S1p = extra ? p.Sx1 : p.S1;
    const long long sbase = (extra ? 0 : (long long)g * p.s_stride) + (col >> 7);
    const int sstride = p.N >> 7;

    auto issue = [&](Stage<WT, SWIGLU> &st, int step) {
        load_rows<WT>(st.w0, B0 + (long long)step * (32 / KP) * ldb, ldb, colok);
        if constexpr (SWIGLU) load_rows<WT>(st.w1, B1 + (long long)step * (32 / KP) * ldb, ldb, colok);
        load_a<WT>(st.a, Ap + step * 32, rok);
        if constexpr (WT == W_FP8) {
            const long long si = sbase + (long long)((kbeg + step * 32) >> 7) * sstride;
            st.s0 = colok ? S0p[si] : 0.0f;
            st.s1 = (SWIGLU && colok) ? S1p[si] : 0.0f;
        }
        if constexpr (WT == W_MXFP4) {
            // the E8M0 bytes of the lane's 8 columns for this 32-deep block
            const long long si = (extra ? 0 : (long long)g * p.s_stride) + (long long)((kbeg + step * 32) >> 5) * p.N + col;
            const uint8_t *S0b = reinterpret_cast<const uint8_t *>(S0p);
            const uint8_t *S1b = reinterpret_cast<const uint8_t *>(S1p);
            st.s0 = colok ? *reinterpret_cast<const u32x2 *>(S0b + si) : u32x2{};
            st.s1 = (SWIGLU && colok) ? *reinterpret_cast<const u32x2 *>(S1b + si) : u32x2{};
        }
    };

    f32x4 acc0[KV], acc1[KV];
#pragma unroll
    for (int c = 0; c < KV; ++c) {
        acc0[c] = f32x4{};
        acc1[c] = f32x4{};
    }

    auto consume = [&](Stage<WT, SWIGLU> &st, int) {
        mma_step<WT>(acc0, st.w0, &st.a, st.s0);
        if constexpr (SWIGLU) mma_step<WT>(acc1, st.w1, &st.a, st.s1);
    };

    // ring of kDepth stages: step j lives in slot j % kDepth
    Stage<WT, SWIGLU> ring[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d)
        if (d < nsteps) issue(ring[d], d);
    for (int s0 = 0; s0 < nsteps; s0 += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const int step = s0 + d;
            const int ahead = step + kDepth - 1;
            if (ahead < nsteps) issue(ring[(d + kDepth - 1) % kDepth], ahead);
            if (step < nsteps) consume(ring[d], step);
        }
    }

    // epilogue: lane holds C[row0 + 4*(lane>>4) + i][col + c]
    if (!colok) return;
    if constexpr (SWIGLU) {
        if (p.ksplit > 1) {
            // split gate/up: fp32 partials of x W1 (columns [0, N)) and x W3
            // (columns [N, 2N)) of this K range; SwiGLU follows the sum
            float *Cf = reinterpret_cast<float *>(p.C) + (long long)split * p.c_split_stride;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = row0 + 4 * kg + i;
                if (row >= row_end) continue;
                float *dst = Cf + (long long)row * p.ldc + col;
#pragma unroll
                for (int h = 0; h < KV / 4; ++h) {
                    *reinterpret_cast<f32x4 *>(dst + 4 * h) =
                        f32x4{acc0[4 * h][i], acc0[4 * h + 1][i], acc0[4 * h + 2][i], acc0[4 * h + 3][i]};
                    *reinterpret_cast<f32x4 *>(dst + p.N + 4 * h) =
                        f32x4{acc1[4 * h][i], acc1[4 * h + 1][i], acc1[4 * h + 2][i], acc1[4 * h + 3][i]};
                }
            }
            return;
        }
    }
    char *Cb = reinterpret_cast<char *>(p.C);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = row0 + 4 * kg + i;
        if (row >= row_end) continue;
        float v[KV];
#pragma unroll
        for (int c = 0; c < KV; ++c)
            v[c] = SWIGLU ? silu_f32(acc0[c][i]) * acc1[c][i] : acc0[c][i];
        const long long off = (long long)split * p.c_split_stride + (long long)row * p.ldc + col;
#pragma unroll
        for (int h = 0; h < KV / 4; ++h) {
            if (OUT_BF16) {
                u32x2 o;
                o.x = pack_bf16x2(v[4 * h], v[4 * h + 1]);
                o.y = pack_bf16x2(v[4 * h + 2], v[4 * h + 3]);
                *reinterpret_cast<u32x2 *>(Cb + (off + 4 * h) * 2) = o;
            } else {
                *reinterpret_cast<f32x4 *>(Cb + (off + 4 * h) * 4) = f32x4{v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]};
            }
        }
    }
}

// two wavefronts per SIMD (<= 256 registers a lane)
template <int WT, bool SWIGLU, bool OUT_BF16>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void stream_gemm_kernel(
    GemmProblem p, int n_slices) {
    stream_gemm_body<WT, SWIGLU, OUT_BF16>(p, n_slices);
}
// the all-fp32 form (small layers) would spill at that budget
template <bool SWIGLU>
__global__ __launch_bounds__(kWaves * 64) void stream_gemm_f32_kernel(GemmProblem p, int n_slices) {
    stream_gemm_body<W_F32, SWIGLU, false>(p, n_slices);
}

template <int WT, bool SWIGLU, bool OUT_BF16>
hipError_t launch_t(const GemmProblem &p, hipStream_t s) {
    const int n_slices = (p.N + slice_of<WT>() - 1) / slice_of<WT>();
    const long long mtiles = p.tiles ? (long long)p.max_tiles : (long long)((p.M + kBM - 1) / kBM);
    const long long waves = mtiles * n_slices;
    // 2 wavefronts per block when there are few (balances the blocks over
    // the CUs; measured 7% faster on 112 experts x 12 slices), else 4
    const int wpb = waves < 2048 ? 2 : kWaves;
    const long long blocks = (waves + wpb - 1) / wpb;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    dim3 grid((unsigned)blocks, (unsigned)p.ksplit);
    if constexpr (WT == W_F32)
        hipLaunchKernelGGL((stream_gemm_f32_kernel<SWIGLU>), grid, dim3(wpb * 64), 0, s, p, n_slices);
    else
        hipLaunchKernelGGL((stream_gemm_kernel<WT, SWIGLU, OUT_BF16>), grid, dim3(wpb * 64), 0, s, p, n_slices);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_gemm(const GemmProblem &p, WType wt, bool swiglu, bool out_bf16,
                              hipStream_t s) {
    // an extra group needs its own weights (and scales for fp8)
    if (p.extra_group >= 0 && (!p.Bx0 || (swiglu && !p.Bx1) || (wt == W_FP8 && (!p.Sx0 || (swiglu && !p.Sx1)))))
        return hipErrorInvalidValue;
    if (p.K % 32 || p.N % 4 || p.kchunk % 32 || p.ksplit < 1) return hipErrorInvalidValue;
    if (wt == W_FP8 && (p.K % 128 || p.N % 128 || p.kchunk % 128)) return hipErrorInvalidValue;
    switch (wt) {
    case W_BF16:
        if (swiglu) return out_bf16 ? launch_t<W_BF16, true, true>(p, s) : launch_t<W_BF16, true, false>(p, s);
        return out_bf16 ? launch_t<W_BF16, false, true>(p, s) : launch_t<W_BF16, false, false>(p, s);
    case W_FP8:
        if (swiglu) return out_bf16 ? launch_t<W_FP8, true, true>(p, s) : launch_t<W_FP8, true, false>(p, s);
        return out_bf16 ? launch_t<W_FP8, false, true>(p, s) : launch_t<W_FP8, false, false>(p, s);
    case W_F32:
        if (out_bf16) return hipErrorInvalidValue;
        return swiglu ? launch_t<W_F32, true, false>(p, s) : launch_t<W_F32, false, false>(p, s);
    case W_F32_XBF16:
        if (swiglu || out_bf16) return hipErrorInvalidValue;
        return launch_t<W_F32_XBF16, false, false>(p, s);
    case W_MXFP4:
        if (p.K % 32 || p.kchunk % 32 || p.N % 8) return hipErrorInvalidValue;
        if (swiglu) return out_bf16 ? launch_t<W_MXFP4, true, true>(p, s) : launch_t<W_MXFP4, true, false>(p, s);
        return out_bf16 ? launch_t<W_MXFP4, false, true>(p, s) : launch_t<W_MXFP4, false, false>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace moe
