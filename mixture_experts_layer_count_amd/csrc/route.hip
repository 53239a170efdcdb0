// Router selection: softmax, top-k, renormalised weights.
//
// Page "MoE serving production quirks" (memory-paradox section): the gate
// applies a linear projection and a softmax over all experts. Page
// "MOE推理流程解析" §三: top-k keeps the chosen expert indices and weights;
// §九: the kept weights are renormalised. The logits themselves come from the
// grouped GEMM (one group, fp32 accumulation).
//
// One wavefront per token. Each lane holds E/64 logits in registers; k rounds
// of a 64-lane butterfly argmax (ties to the lower expert index) pick the
// experts best first. The renormalised weight of the j-th pick equals the
// softmax over the k kept logits, exp(l_j - l_0) / sum_j' exp(l_j' - l_0),
// because the full softmax's denominator cancels.
#include <math.h>

#include "common.h"

namespace moe {
namespace {

constexpr int kWaves = 4;

// true if (va, ia) ranks before (vb, ib): larger value, then lower index
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

template <int NPER>
__global__ __launch_bounds__(kWaves * 64) void topk_kernel(const float *part, int nsplit,
                                                           long long split_stride, const float *bias,
                                                           int T, int E, int k, float *logits,
                                                           int32_t *idx, float *w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (t >= T) return;
    const float *prow = part + (long long)t * E;
    float *row = logits + (long long)t * E;

    float v[NPER];   // logit used for ranking (NaN -> -inf)
    float raw[NPER]; // logit as stored
    bool taken[NPER];
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
        const int e = lane + 64 * i;
        float x = -INFINITY;
        if (e < E) {
            // fixed-order sum of the split-K partials; loads issued in
            // batches of 8 so their latencies overlap
            x = 0.0f;
            for (int s0 = 0; s0 < nsplit; s0 += 8) {
                float v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    v[u] = (s0 + u < nsplit) ? prow[(long long)(s0 + u) * split_stride + e] : 0.0f;
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (s0 + u < nsplit) x = (s0 + u == 0) ? v[u] : x + v[u];
            }
            if (bias) x += bias[e];
            row[e] = x;
        }
        raw[i] = x;
        v[i] = (x != x) ? -INFINITY : x;
        taken[i] = e >= E;
    }

    float sel_val = 0.0f;  // lane j < k keeps the j-th pick
    int sel_idx = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        float braw = 0.0f;
#pragma unroll
        for (int i = 0; i < NPER; ++i) {
            const int e = lane + 64 * i;
            if (!taken[i] && better(v[i], e, bv, bi)) {
                bv = v[i];
                bi = e;
                braw = raw[i];
            }
        }
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float ov = __shfl_xor(bv, d, 64);
            const int oi = __shfl_xor(bi, d, 64);
            const float oraw = __shfl_xor(braw, d, 64);
            if (better(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
                braw = oraw;
            }
        }
        // every lane now agrees on (bv, bi); its owner marks it taken
#pragma unroll
        for (int i = 0; i < NPER; ++i)
            if (lane + 64 * i == bi) taken[i] = true;
        if (lane == j) {
            sel_val = braw;
            sel_idx = bi;
        }
    }

    const float top = __shfl(sel_val, 0, 64);
    float ex = (lane < k) ? expf(sel_val - top) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) sum += __shfl_xor(sum, d, 64);
    if (lane < k) {
        idx[(long long)t * k + lane] = sel_idx;
        w[(long long)t * k + lane] = ex / sum;
    }
}

}  // namespace

hipError_t launch_topk(const float *part, int nsplit, long long split_stride, const float *bias,
                       int T, int E, int k, float *logits, int32_t *idx, float *w, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (E < 1 || E > 1024 || k < 1 || k > E || k > 64) return hipErrorInvalidValue;
    const dim3 grid((T + kWaves - 1) / kWaves), block(kWaves * 64);
    const int nper = (E + 63) / 64;
#define MOE_TOPK(N)                                                                                 \
    hipLaunchKernelGGL(topk_kernel<N>, grid, block, 0, s, part, nsplit, split_stride, bias, T, E, k, \
                       logits, idx, w)
    if (nper <= 1) MOE_TOPK(1);
    else if (nper <= 2) MOE_TOPK(2);
    else if (nper <= 4) MOE_TOPK(4);
    else if (nper <= 8) MOE_TOPK(8);
    else MOE_TOPK(16);
#undef MOE_TOPK
    return hipGetLastError();
}

}  // namespace moe
