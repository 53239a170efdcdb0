// Router selection: softmax, top-k, renormalised weights.
//
// Page "MoE serving production quirks" (memory-paradox section): the gate
// applies a linear projection and a softmax over all experts. Page
// "MOE推理流程解析" §三: top-k keeps the chosen expert indices and weights;
// §九: the kept weights are renormalised. The logits themselves come from the
// grouped GEMM (one group, fp32 accumulation).
//
// One wavefront per token. Each lane holds E/64 logits in registers; k rounds
// of a 64-lane argmax pick the experts best first: the largest 32-bit ranking
// key by DPP row steps and row broadcasts, then the lowest expert index
// holding it by ballot (ties go to the lower index). The renormalised weight of the j-th pick equals the
// softmax over the k kept logits, exp(l_j - l_0) / sum_j' exp(l_j' - l_0),
// because the full softmax's denominator cancels.
#include <math.h>

#include "common.h"

namespace moe {
namespace {

constexpr int kWaves = 4;

// Ranking key of a logit: its bits made monotonic as an unsigned integer, so
// a larger key means a larger logit. Every real key is above 0 (-inf maps to
// 0x007fffff), and 0 marks taken entries. (NaN logits are ranked as -inf
// before they get here.) Equal keys go to the lower expert index, found by
// ballot after the maximum.
__device__ __forceinline__ uint32_t rank_key(float v) {
    const uint32_t b = __float_as_uint(v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
// DPP row steps: the key of another lane of the same 16-lane row, or (with a
// row mask) of the last lane of an earlier row for the enabled rows, the
// other rows keeping their own
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_key(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t bcast_key(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, ROW_MASK, 0xf, false);
}
// wavefront-wide maximum key, the same in every lane: quad permutations and
// row rotations give every lane its 16-lane row's maximum; row broadcasts
// (lane 15 into row 1 and row 3, then lane 31 into rows 2 and 3) leave the
// wavefront's maximum in lane 63, which is read out. All VALU (DPP) steps.
__device__ __forceinline__ uint32_t wave_max_key(uint32_t x) {
    x = max(x, dpp_key<0xB1>(x));   // quad_perm [1,0,3,2]
    x = max(x, dpp_key<0x4E>(x));   // quad_perm [2,3,0,1]
    x = max(x, dpp_key<0x124>(x));  // row_ror:4
    x = max(x, dpp_key<0x128>(x));  // row_ror:8
    x = max(x, bcast_key<0x142, 0xa>(x));  // row_bcast:15 into rows 1, 3
    x = max(x, bcast_key<0x143, 0xc>(x));  // row_bcast:31 into rows 2, 3
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
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

    float raw[NPER];              // logit as stored
    uint32_t key[NPER];           // ranking key (0 once taken or past E)
    // fixed-order sum (ascending split) of the split-K partials: the loads of
    // up to 4 of the lane's experts x 16 splits, and their biases, are issued
    // together so that their latencies overlap
    constexpr int IG = NPER < 4 ? NPER : 4;
#pragma unroll
    for (int i0 = 0; i0 < NPER; i0 += IG) {
        float x[IG], b[IG];
#pragma unroll
        for (int i = 0; i < IG; ++i) {
            const int e = lane + 64 * (i0 + i);
            x[i] = 0.0f;
            b[i] = (bias && e < E) ? bias[e] : 0.0f;
        }
        for (int s0 = 0; s0 < nsplit; s0 += 16) {
            float v[IG][16];
#pragma unroll
            for (int i = 0; i < IG; ++i) {
                const int e = lane + 64 * (i0 + i);
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    v[i][u] = (e < E && s0 + u < nsplit) ? prow[(long long)(s0 + u) * split_stride + e] : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < IG; ++i)
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    if (s0 + u < nsplit) x[i] = (s0 + u == 0) ? v[i][u] : x[i] + v[i][u];
        }
#pragma unroll
        for (int i = 0; i < IG; ++i) {
            const int e = lane + 64 * (i0 + i);
            float xe = -INFINITY;
            if (e < E) {
                xe = bias ? x[i] + b[i] : x[i];
                row[e] = xe;
            }
            raw[i0 + i] = xe;
            key[i0 + i] = e < E ? rank_key((xe != xe) ? -INFINITY : xe) : 0u;
        }
    }

    float sel_val = 0.0f;  // lane j < k keeps the j-th pick
    int sel_idx = 0;
    for (int j = 0; j < k; ++j) {
        uint32_t best = 0;
#pragma unroll
        for (int i = 0; i < NPER; ++i) best = max(best, key[i]);
        best = wave_max_key(best);
        // the lowest expert index holding the best key: expert e = lane + 64 i,
        // so the first group i with a match, then its lowest matching lane
        int bi = 0;
#pragma unroll
        for (int i = NPER - 1; i >= 0; --i) {
            const unsigned long long m = __ballot(key[i] == best);
            if (m) bi = 64 * i + __builtin_ctzll(m);
        }
        bi = __builtin_amdgcn_readfirstlane(bi);
        // its owner marks it taken
        float r = raw[0];
#pragma unroll
        for (int i = 0; i < NPER; ++i) {
            if (lane + 64 * i == bi) key[i] = 0u;
            if (i == (bi >> 6)) r = raw[i];
        }
        const float braw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), bi & 63));
        if (lane == j) {
            sel_val = braw;
            sel_idx = bi;
        }
    }

    const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel_val), 0));
    const float ex = (lane < k) ? expf(sel_val - top) : 0.0f;
    // the normaliser, summed over the picks in slot order (the same value in
    // every lane)
    float sum = 0.0f;
    for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
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
