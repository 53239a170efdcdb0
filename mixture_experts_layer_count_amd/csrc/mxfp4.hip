// MXFP4 weights decoded to bf16 for the tiled (matrix-core) kernels.
//
// The OCP microscaling format MXFP4: E2M1 element codes, two K-consecutive
// values a byte (row 2i in the low nibble, 2i + 1 in the high nibble of byte
// (i, n)), and one E8M0 scale 2^(e - 127) per 32 consecutive K rows of a
// column. Pages: "MoE-推理部署", expert-quantisation section (MXFP4 beside FP8
// for single-GPU serving); the element and scale encodings are those of the
// OCP microscaling specification. The tiled kernels stream bf16 tiles into
// LDS; at prefill sizes the layer is matrix-bound, so one HBM-bound pass that
// writes the experts as bf16 costs a fraction of the GEMMs it feeds. Every
// E2M1 value times a power of two within bf16's range is exact in bf16.
#include "common.h"

namespace moe {
namespace {

// the two bf16 values of byte B of `codes` (low half: row 2i, high half:
// row 2i + 1), times the E8M0 scale in byte B of `scales`
template <int B>
__device__ __forceinline__ uint32_t pair_of(uint32_t codes, uint32_t scales) {
    const float sc = __uint_as_float(((scales >> (8 * B)) & 0xffu) << 23);
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, B));
}

// 4 columns (one code word) -> row 2i in lo.x, lo.y and row 2i + 1 in hi.x, hi.y
__device__ __forceinline__ void four_columns(uint32_t w, uint32_t s, uint32_t &lo0, uint32_t &lo1, uint32_t &hi0,
                                             uint32_t &hi1) {
    const uint32_t p0 = pair_of<0>(w, s), p1 = pair_of<1>(w, s);
    const uint32_t p2 = pair_of<2>(w, s), p3 = pair_of<3>(w, s);
    lo0 = __builtin_amdgcn_perm(p1, p0, 0x05040100u);
    lo1 = __builtin_amdgcn_perm(p3, p2, 0x05040100u);
    hi0 = __builtin_amdgcn_perm(p1, p0, 0x07060302u);
    hi1 = __builtin_amdgcn_perm(p3, p2, 0x07060302u);
}

// one thread: 8 columns of one K-pair row -> 2 bf16 rows of 8 columns (16 B each)
__global__ __launch_bounds__(256) void mxfp4_to_bf16_kernel(const uint8_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ scales, long long kp_rows,
                                                            int N, uint16_t *__restrict__ out) {
    // kp_rows = G * K / 2 (K-pair rows over all groups); K % 32 == 0, so the
    // scale row of pair row i is i / 16 over all groups too
    const int no = N >> 3;
    const long long total = kp_rows * no;
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        const long long i = t / no;
        const int c = (int)(t - i * no) * 8;
        const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(codes + i * N + c));
        const u32x2 s = *reinterpret_cast<const u32x2 *>(scales + (i >> 4) * N + c);
        uint32_t a0, a1, a2, a3, b0, b1, b2, b3;
        four_columns(w.x, s.x, a0, a1, b0, b1);
        four_columns(w.y, s.y, a2, a3, b2, b3);
        *reinterpret_cast<u32x4 *>(out + (2 * i) * N + c) = u32x4{a0, a1, a2, a3};
        *reinterpret_cast<u32x4 *>(out + (2 * i + 1) * N + c) = u32x4{b0, b1, b2, b3};
    }
}

}  // namespace

hipError_t launch_mxfp4_to_bf16(const void *codes, const void *scales, int G, int K, int N, void *out,
                                hipStream_t s) {
    if (G < 1 || K < 32 || N < 8 || K % 32 || N % 8 || !codes || !scales || !out) return hipErrorInvalidValue;
    const long long kp_rows = (long long)G * (K / 2);
    const long long total = kp_rows * (N / 8);
    const long long want = (total + 255) / 256;
    const int blocks = (int)(want < 8192 ? want : 8192);
    hipLaunchKernelGGL(mxfp4_to_bf16_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const uint8_t *>(codes),
                       static_cast<const uint8_t *>(scales), kp_rows, N, static_cast<uint16_t *>(out));
    return hipGetLastError();
}

}  // namespace moe
