// Combine / unpermute, and the fixed-order reduction of split-K partials.
//
// Page "MOE推理流程解析" §二: each token's expert contributions are multiplied
// by their routing weights and added; §三: the inverse map restores token
// order. §一: an always-on shared expert adds its output with weight 1.
//
// Y[t] = sum_{j<k} w[t,j] * (sum_s Yp_s[assign_row[t*k+j]]) (+ sum_s S_s[t]),
// accumulated in fp32 in ascending j (and ascending split s), then rounded
// once to the output dtype. Each thread owns 4 consecutive columns of one
// token row; rows are read with 8-byte (bf16) or 16-byte (f32) vectors.
#include "common.h"

namespace moe {
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

template <typename InT, typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(const InT *Yp, const InT *S,
                                                      long long split_stride, int nsplit,
                                                      const int32_t *assign_row, const float *w,
                                                      int T, int k, int H, OutT *Y) {
    const int t = blockIdx.y;
    const int col = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (t >= T || col >= H) return;
    f32x4 acc = f32x4{};
    for (int j = 0; j < k; ++j) {
        const long long a = (long long)t * k + j;
        const long long row = assign_row[a];
        const float wj = w[a];
        f32x4 y = load4<InT>(Yp + row * H + col);
        for (int s = 1; s < nsplit; ++s) y += load4<InT>(Yp + s * split_stride + row * H + col);
        acc[0] = fmaf(wj, y[0], acc[0]);
        acc[1] = fmaf(wj, y[1], acc[1]);
        acc[2] = fmaf(wj, y[2], acc[2]);
        acc[3] = fmaf(wj, y[3], acc[3]);
    }
    if (S) {
        f32x4 y = load4<InT>(S + (long long)t * H + col);
        for (int s = 1; s < nsplit; ++s) y += load4<InT>(S + s * split_stride + (long long)t * H + col);
        acc += y;
    }
    store4<OutT>(Y + (long long)t * H + col, acc);
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

}  // namespace

hipError_t launch_combine(const void *Yp, const void *S, long long split_stride, int nsplit,
                          moe_dtype in_dt, const int32_t *assign_row, const float *w, int T,
                          int k, int H, moe_dtype out_dt, void *Y, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (H % 4 || nsplit < 1 || T > 65535) return hipErrorInvalidValue;
    const dim3 grid((H / 4 + 255) / 256, T), block(256);
#define MOE_COMBINE(IT, OT)                                                                         \
    hipLaunchKernelGGL((combine_kernel<IT, OT>), grid, block, 0, s, (const IT *)Yp, (const IT *)S, \
                       split_stride, nsplit, assign_row, w, T, k, H, (OT *)Y)
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
