// E4M3 activation quantisation for the W8A8 expert GEMMs.
//
// Page "MOE推理流程解析" §三: activations may be quantised before dispatch
// (fewer bytes moved) or dispatched in higher precision and quantised before
// the expert GEMM. Scales here are per row and 128-column group, so quantising
// the token rows once before the gather gives the same codes as quantising
// the gathered rows.
//
// One 16-lane group per (row, 128-column group); each lane owns 8 consecutive
// bf16 values (one 16-byte load). amax is reduced across the 16 lanes with
// xor shuffles; s = amax / 448 (correctly rounded fp32 division), and each
// value is divided by s, clamped to +-448 (the conversion gives NaN past
// 480 rather than saturating) and rounded to nearest even by
// v_cvt_pk_fp8_f32 (OCP E4M3 on gfx950).
//
// Scales go row-major (S[r][C/128], the public entry point) or transposed,
// S[g * s_ld + row], the layout the W8A8 GEMM reads: a tile's rows are then
// contiguous, so one 4-byte-per-lane copy of 64 rows' scales touches one or
// two cache lines instead of 64 (measured: 6 % of the DeepSeek-shaped gate/up).
// For the token rows of a layer the transposed scales are written at the rows
// the permutation gives each token's assignments (scatter[t*sk + j], j < sk,
// the inverse map) and, with a shared expert, at extra0 + t. That launch is
// ordered by group: a block takes 64 consecutive rows of one group, and the
// groups g with g % 8 == x go to XCD x (block index % 8), so the 4-byte
// scatter writes into group g's scale row all land in one XCD's L2 and merge
// there into whole lines (in row order, every XCD wrote partial lines of
// every scale row; the DeepSeek-shaped layer's quantisation went from 33.2
// to 31.1 us). Each 16-lane group quantises 4 of the block's rows, with the
// four 16-byte loads (and the rows' permuted positions) in flight together
// rather than one row and one load per group: 30.5 -> 26.5 us for the same
// layer's quantisation stage.
#include "common.h"

namespace moe {

MOE_BOUNDS_FILE(quant)
namespace {

// One (row, 128-column group): the 16 lanes of the group own 8 consecutive
// values each (raw: their 16-byte load); returns the scale, codes in w.
__device__ __forceinline__ float quant_group(const u32x4 &raw, uint32_t (&w)[2]) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_lo(raw[i]);
        v[2 * i + 1] = bf16_hi(raw[i]);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 16));
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = fminf(fmaxf(v[4 * h + i] / s, -448.0f), 448.0f);
        int p = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], p, true);
        w[h] = (uint32_t)p;
    }
    return s;
}

__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t *X, long long ldx, const int32_t *row_src,
                                                         int gk, int R, int C, uint8_t *Q, float *S, long long s_ld) {
    const int sub = threadIdx.x & 15;
    const int gpr = C >> 7;  // groups per row
    const long long gid = ((long long)blockIdx.x * 256 + threadIdx.x) >> 4;
    const bool ok = gid < (long long)R * gpr;
    const long long r = ok ? gid / gpr : 0;
    const int gc = ok ? (int)(gid - r * gpr) : 0;

    u32x4 raw = {0, 0, 0, 0};
    if (ok) {
        const long long xr = row_src ? (long long)(row_src[r] / gk) : r;
        raw = *reinterpret_cast<const u32x4 *>(X + xr * ldx + 128 * gc + 8 * sub);
    }
    uint32_t w[2];
    const float s = quant_group(raw, w);
    if (!ok) return;
    *reinterpret_cast<u32x2 *>(Q + r * C + 128 * gc + 8 * sub) = u32x2{w[0], w[1]};
    if (sub != 0) return;
    if (s_ld == 0) S[r * gpr + gc] = s;
    else S[gc * s_ld + r] = s;
}

// The token rows of a layer, scales scattered to the permuted rows. A block
// takes kScatterRows rows of one group: each 16-lane group kScatterRows / 16
// rows 16 apart, their loads issued together. XCD x = block % 8 takes groups
// x, x + 8, ...; its block s covers rows kScatterRows (s % chunks) .. + 63 of
// group x + 8 (s / chunks).
constexpr int kScatterRows = 64;
__global__ __launch_bounds__(256) void quant_scatter_kernel(const uint16_t *X, long long ldx, int R, int C,
                                                            uint8_t *Q, float *S, long long s_ld,
                                                            const int32_t *scatter, int sk, int extra0) {
    constexpr int RPT = kScatterRows / 16;  // rows per 16-lane group
    const int sub = threadIdx.x & 15;
    const int gpr = C >> 7;
    const int chunks = (R + kScatterRows - 1) / kScatterRows;
    const int x = blockIdx.x % 8, sblk = blockIdx.x / 8;
    const int gc = x + 8 * (sblk / chunks);
    if (gc >= gpr) return;  // the whole block: gc is uniform
    const int r0 = kScatterRows * (sblk % chunks) + (threadIdx.x >> 4);
    // the rows' values and (lane j < sk) the permuted row of assignment j,
    // all loads in flight together: unconditional loads, rows past the end
    // reading row R - 1 (their results are never stored)
    u32x4 raw[RPT];
    int dst0[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const long long rc = min(r0 + 16 * i, R - 1);
        raw[i] = *reinterpret_cast<const u32x4 *>(X + rc * ldx + 128 * gc + 8 * sub);
        dst0[i] = scatter[rc * sk + min(sub, sk - 1)];
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = r0 + 16 * i;
        uint32_t w[2];
        const float s = quant_group(raw[i], w);
        if (r >= R) continue;
        *reinterpret_cast<u32x2 *>(Q + (long long)r * C + 128 * gc + 8 * sub) = u32x2{w[0], w[1]};
        // lane j < sk writes the copy of assignment j, lane sk the shared row's
        for (int j = sub; j <= sk; j += 16) {
            long long dst;
            if (j < sk) dst = j == sub ? dst0[i] : scatter[(long long)r * sk + j];
            else if (extra0 >= 0) dst = extra0 + r;
            else continue;
            if (MOE_BOUNDS_FAIL(dst >= 0 && dst < s_ld, BOUNDS_QUANT_ROW)) continue;
            S[gc * s_ld + dst] = s;
        }
    }
}

}  // namespace

hipError_t launch_quant_rows(const void *X, long long ldx, const int32_t *row_src, int gk, int R, int C,
                             uint8_t *Q, float *S, hipStream_t s, const ScaleLayout *sl) {
    if (R < 0 || C < 128 || C % 128 || ldx < C || gk < 1) return hipErrorInvalidValue;
    if (sl && (sl->ld < 1 || (sl->scatter && sl->k < 1))) return hipErrorInvalidValue;
    if (R == 0) return hipSuccess;
    if (sl && sl->scatter) {
        if (row_src || gk != 1) return hipErrorInvalidValue;  // token rows in order
        // group-ordered launch: 8 XCDs x ceil(groups / 8) x row chunks
        const long long blocks = 8LL * ((C / 128 + 7) / 8) * ((R + kScatterRows - 1) / kScatterRows);
        if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
        hipLaunchKernelGGL(quant_scatter_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                           reinterpret_cast<const uint16_t *>(X), ldx, R, C, Q, S, sl->ld, sl->scatter, sl->k,
                           sl->extra0);
        return hipGetLastError();
    }
    const long long threads = (long long)R * (C / 128) * 16;
    const long long blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t *>(X), ldx, row_src, gk, R, C, Q, S, sl ? sl->ld : 0LL);
    return hipGetLastError();
}

}  // namespace moe
