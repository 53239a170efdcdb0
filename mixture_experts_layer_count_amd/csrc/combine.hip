// Combine / unpermute, and the fixed-order reduction of split-K partials.
//
// Page "MOE推理流程解析" §二: each token's expert contributions are multiplied
// by their routing weights and added; §三: the inverse map restores token
// order. §一: an always-on shared expert adds its output with weight 1.
//
// Y[t] = sum_{j<k} w[t,j] * (sum_s Yp_s[assign_row[t*k+j]]) (+ sum_s S_s[t]),
// accumulated in fp32 in ascending j (and ascending split s; the shared
// expert's partials may have their own split count), then rounded
// once to the output dtype. Each thread owns 16 consecutive columns of one
// token row for bf16 rows (two 16-byte loads per row; 128-thread blocks when
// a row needs no more), else 8 or, when H is not a multiple of 8, 4; the rows
// and weights of up to 8 contributions are fetched before their row loads are
// issued together. bf16 rows are widened only when used (86 registers a lane
// instead of 168 for 16 columns, so five wavefronts a SIMD instead of three);
// split partials (nsplit > 1) come as fp32 only.
#include "common.h"

namespace moe {

MOE_BOUNDS_FILE(combine)
namespace {

template <typename InT>
__device__ __forceinline__ f32x4 load4(const InT *p);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
}
template <>
__device__ __forceinline__ f32x4 load4<uint16_t>(const uint16_t *p) {
    const u32x2 v = *reinterpret_cast<const u32x2 *>(p);
    return f32x4{bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
}

template <typename OutT>
__device__ __forceinline__ void store4(OutT *p, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float *p, f32x4 v) {
    *reinterpret_cast<f32x4 *>(p) = v;
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t *p, f32x4 v) {
    u32x2 o;
    o.x = pack_bf16x2(v[0], v[1]);
    o.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<u32x2 *>(p) = o;
}

// V = 4, 8 or 16 consecutive columns per thread (4-column quarters). bf16
// rows of 8 or 16 columns stay packed until they are used: half the
// registers of widened values, so more rows are in flight per SIMD.
template <typename InT, int V>
struct Vec {
    static constexpr bool packed = (V == 8 || V == 16) && sizeof(InT) == 2;
    u32x4 raw[packed ? V / 8 : 1];
    f32x4 h[packed ? 1 : V / 4];
    __device__ __forceinline__ f32x4 quarter(int i) const {
        if constexpr (packed) {
            const u32x4 &v = raw[i >> 1];
            return (i & 1) ? f32x4{bf16_lo(v[2]), bf16_hi(v[2]), bf16_lo(v[3]), bf16_hi(v[3])}
                           : f32x4{bf16_lo(v[0]), bf16_hi(v[0]), bf16_lo(v[1]), bf16_hi(v[1])};
        } else {
            return h[i];
        }
    }
};
template <typename InT, int V>
__device__ __forceinline__ Vec<InT, V> loadv(const InT *p) {
    Vec<InT, V> r;
    if constexpr (Vec<InT, V>::packed) {
#pragma unroll
        for (int q = 0; q < V / 8; ++q) r.raw[q] = *reinterpret_cast<const u32x4 *>(p + 8 * q);
    } else {
#pragma unroll
        for (int i = 0; i < V / 4; ++i) r.h[i] = load4<InT>(p + 4 * i);
    }
    return r;
}

template <typename InT, typename OutT, int V>
__global__ __launch_bounds__(512) void combine_kernel(const InT *Yp, const InT *S,
                                                      long long split_stride, int nsplit, int nsplit_s,
                                                      const int32_t *assign_row, const float *w,
                                                      int T, int k, int H, OutT *Y, long long yp_rows) {
    const int t = blockIdx.y;
    const int col = (blockIdx.x * blockDim.x + threadIdx.x) * V;
    if (t >= T || col >= H) return;
    f32x4 acc[V / 4];
#pragma unroll
    for (int i = 0; i < V / 4; ++i) acc[i] = f32x4{};
    // up to 8 contributions at a time: their rows and weights first, then all
    // their loads, so the latencies overlap; then the weighted sum in j order
    for (int j0 = 0; j0 < k; j0 += 8) {
        long long row[8];
        float wj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (j0 + u < k) {
                const long long a = (long long)t * k + j0 + u;
                row[u] = assign_row[a];
                if (MOE_BOUNDS_FAIL(row[u] >= 0 && (yp_rows <= 0 || row[u] < yp_rows), BOUNDS_COMBINE_ROW))
                    row[u] = 0;
                wj[u] = w[a];
            }
        }
        Vec<InT, V> y[8];
        f32x4 ys[8][Vec<InT, V>::packed ? 1 : V / 4];  // split sums (fp32 partials only)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (j0 + u < k) {
                y[u] = loadv<InT, V>(Yp + row[u] * H + col);
                if constexpr (!Vec<InT, V>::packed) {
#pragma unroll
                    for (int i = 0; i < V / 4; ++i) ys[u][i] = y[u].h[i];
                    for (int s = 1; s < nsplit; ++s) {
                        const Vec<InT, V> z = loadv<InT, V>(Yp + s * split_stride + row[u] * H + col);
#pragma unroll
                        for (int i = 0; i < V / 4; ++i) ys[u][i] += z.h[i];
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (j0 + u < k) {
#pragma unroll
                for (int i = 0; i < V / 4; ++i) {
                    f32x4 v;
                    if constexpr (Vec<InT, V>::packed) v = y[u].quarter(i);
                    else v = ys[u][i];
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[i][c] = fmaf(wj[u], v[c], acc[i][c]);
                }
            }
        }
    }
    if (S) {
        const Vec<InT, V> y = loadv<InT, V>(S + (long long)t * H + col);
#pragma unroll
        for (int i = 0; i < V / 4; ++i) {
            f32x4 v = y.quarter(i);
            if constexpr (!Vec<InT, V>::packed)
                for (int s = 1; s < nsplit_s; ++s) v += load4<InT>(S + s * split_stride + (long long)t * H + col + 4 * i);
            acc[i] += v;
        }
    }
#pragma unroll
    for (int i = 0; i < V / 4; ++i) store4<OutT>(Y + (long long)t * H + col + 4 * i, acc[i]);
}

template <typename OutT>
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float *part, long long split_stride,
                                                            int nsplit, long long n4, OutT *out) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    f32x4 v = *reinterpret_cast<const f32x4 *>(part + 4 * i);
    for (int s = 1; s < nsplit; ++s) v += *reinterpret_cast<const f32x4 *>(part + s * split_stride + 4 * i);
    store4<OutT>(out + 4 * i, v);
}

// h[r, c] = silu(sum_s G_s[r, c]) * sum_s U_s[r, c], sums in ascending s;
// part holds per split s the rows [M][2N] with G in columns [0, N) and U in
// [N, 2N)
template <typename OutT>
__global__ __launch_bounds__(256) void swiglu_splits_kernel(const float *part, long long split_stride, int nsplit,
                                                            int M, int N, OutT *out) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;  // 4-column group
    const int n4 = N / 4;
    if (i >= (long long)M * n4) return;
    const long long r = i / n4;
    const int c = 4 * (int)(i - r * n4);
    const float *p0 = part + r * 2 * N + c;
    f32x4 g = *reinterpret_cast<const f32x4 *>(p0);
    f32x4 u = *reinterpret_cast<const f32x4 *>(p0 + N);
    for (int s = 1; s < nsplit; ++s) {
        g += *reinterpret_cast<const f32x4 *>(p0 + s * split_stride);
        u += *reinterpret_cast<const f32x4 *>(p0 + s * split_stride + N);
    }
    store4<OutT>(out + r * N + c, f32x4{silu_f32(g[0]) * u[0], silu_f32(g[1]) * u[1], silu_f32(g[2]) * u[2],
                                        silu_f32(g[3]) * u[3]});
}

}  // namespace

hipError_t launch_swiglu_splits(const float *part, long long split_stride, int nsplit, int M, int N,
                                moe_dtype out_dt, void *out, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if (N % 4 || nsplit < 1) return hipErrorInvalidValue;
    const long long n = (long long)M * (N / 4);
    const dim3 grid((unsigned)((n + 255) / 256)), block(256);
    if (out_dt == MOE_F32)
        hipLaunchKernelGGL(swiglu_splits_kernel<float>, grid, block, 0, s, part, split_stride, nsplit, M, N,
                           (float *)out);
    else if (out_dt == MOE_BF16)
        hipLaunchKernelGGL(swiglu_splits_kernel<uint16_t>, grid, block, 0, s, part, split_stride, nsplit, M, N,
                           (uint16_t *)out);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_combine(const void *Yp, const void *S, long long split_stride, int nsplit, int nsplit_s,
                          moe_dtype in_dt, const int32_t *assign_row, const float *w, int T,
                          int k, int H, moe_dtype out_dt, void *Y, hipStream_t s, long long yp_rows) {
    if (T <= 0) return hipSuccess;
    if (H % 4 || nsplit < 1 || nsplit_s < 1 || T > 65535) return hipErrorInvalidValue;
    // split partials are fp32 (bf16 rows come whole from the tiled kernels)
    if (in_dt == MOE_BF16 && (nsplit != 1 || nsplit_s != 1)) return hipErrorInvalidValue;
    // 16 bf16 columns a thread (two 16-byte loads per row) when H allows
    const bool v16 = H % 16 == 0 && in_dt == MOE_BF16;
    const bool v8 = H % 8 == 0;
    const int vw = v16 ? 16 : v8 ? 8 : 4;
    const int nthr = H / vw;
    // one block per token row when the row's threads make whole wavefronts
    // (up to 512: the DeepSeek-shaped prefill's 448), else blocks of 128/256
    // (one block per token instead of two of 256 threads: DeepSeek-shaped
    // prefill combine 117 -> 110 us)
    const int bs = (nthr % 64 == 0 && nthr <= 512) ? nthr : (nthr <= 128 ? 128 : 256);
    const dim3 grid((nthr + bs - 1) / bs, T), block(bs);
#define MOE_COMBINE(IT, OT)                                                                               \
    do {                                                                                                  \
        if (v16)                                                                                          \
            hipLaunchKernelGGL((combine_kernel<IT, OT, 16>), grid, block, 0, s, (const IT *)Yp,            \
                               (const IT *)S, split_stride, nsplit, nsplit_s, assign_row, w, T, k, H, (OT *)Y, yp_rows); \
        else if (v8)                                                                                      \
            hipLaunchKernelGGL((combine_kernel<IT, OT, 8>), grid, block, 0, s, (const IT *)Yp,             \
                               (const IT *)S, split_stride, nsplit, nsplit_s, assign_row, w, T, k, H, (OT *)Y, yp_rows);    \
        else                                                                                              \
            hipLaunchKernelGGL((combine_kernel<IT, OT, 4>), grid, block, 0, s, (const IT *)Yp,             \
                               (const IT *)S, split_stride, nsplit, nsplit_s, assign_row, w, T, k, H, (OT *)Y, yp_rows);    \
    } while (0)
    if (in_dt == MOE_F32 && out_dt == MOE_F32) MOE_COMBINE(float, float);
    else if (in_dt == MOE_F32 && out_dt == MOE_BF16) MOE_COMBINE(float, uint16_t);
    else if (in_dt == MOE_BF16 && out_dt == MOE_BF16) MOE_COMBINE(uint16_t, uint16_t);
    else if (in_dt == MOE_BF16 && out_dt == MOE_F32) MOE_COMBINE(uint16_t, float);
    else return hipErrorInvalidValue;
#undef MOE_COMBINE
    return hipGetLastError();
}

hipError_t launch_reduce_splits(const float *part, long long split_stride, int nsplit, int M, int N,
                                moe_dtype out_dt, void *out, hipStream_t s) {
    const long long n = (long long)M * N;
    if (n <= 0) return hipSuccess;
    if (n % 4) return hipErrorInvalidValue;
    const long long n4 = n / 4;
    const dim3 grid((unsigned)((n4 + 255) / 256)), block(256);
    if (out_dt == MOE_F32)
        hipLaunchKernelGGL(reduce_splits_kernel<float>, grid, block, 0, s, part, split_stride, nsplit, n4,
                           (float *)out);
    else if (out_dt == MOE_BF16)
        hipLaunchKernelGGL(reduce_splits_kernel<uint16_t>, grid, block, 0, s, part, split_stride, nsplit,
                           n4, (uint16_t *)out);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace moe
