// LDS-tiled grouped GEMM (prefill): tile-height choice, shape support and
// the launcher. The kernel is in tiled_gemm_kernel.h.
#include "tiled_gemm_kernel.h"

namespace moe {

int tiled_gemm_bm(WType wt, long long rows, int groups) {
    // fp8 keeps a second accumulator set for the open scale block: 128 rows
    if (wt == W_FP8) return 128;
    // 256-row tiles once experts average >= 192 rows, else 128
    return (groups > 0 && rows >= 192LL * groups) ? 256 : 128;
}

static_assert(tiled::kTailSlots == tiled_tail_counters, "one counter per tail slot");
// one partial tile (bm rows x 256 B-columns, fp32) per tail slot
size_t tiled_tail_bytes(int bm) { return sizeof(float) * (size_t)tiled::kTailSlots * bm * 256; }

// down projections with more K steps than this keep the tail split
constexpr int kPersistMaxSplitSteps = 128;

bool tiled_gemm_supports(WType wt, int N, int K) {
    if (wt == W_F32 || wt == W_F32_XBF16) return false;
    if (N % 8 || K % tiled::kBK || N < 16 || K < tiled::kBK) return false;
    if (wt == W_MXFP4 && N % 16) return false;  // 16-column byte chunks
    if (wt == W_FP8 && (N % 128 || K % 128)) return false;
    return true;
}

hipError_t launch_tiled_gemm(const GemmProblem &p, WType wt, bool swiglu, bool out_bf16, int bm,
                             hipStream_t s) {
    // an extra group needs its own weights (and scales for fp8 and MXFP4)
    const bool sc = wt == W_FP8 || wt == W_MXFP4;
    if (p.extra_group >= 0 && (!p.Bx0 || (swiglu && !p.Bx1) || (sc && (!p.Sx0 || (swiglu && !p.Sx1)))))
        return hipErrorInvalidValue;
    if (sc && (!p.S0 || (swiglu && !p.S1))) return hipErrorInvalidValue;
    if (!out_bf16 || p.ksplit != 1 || !tiled_gemm_supports(wt, p.N, p.K)) return hipErrorInvalidValue;
    if (!(bm == 128 || (bm == 256 && (wt == W_BF16 || wt == W_MXFP4)))) return hipErrorInvalidValue;
    // the tail split: plain GEMMs with bf16 or MXFP4 weights
    if (p.tail_part && (wt == W_FP8 || swiglu || !p.tail_cnt || !p.tiles)) return hipErrorInvalidValue;
    // the persistent form where it fits, unless a down projection's long K
    // makes the tail split (one item per workgroup) the better end of the
    // launch
    if (tiled_persist_fits(p, wt, swiglu, bm) && (!p.tail_part || p.K / tiled::kBK <= kPersistMaxSplitSteps))
        return launch_tiled_persist(p, swiglu, s);
    return bm == 256 ? launch_tiled_bm256(p, wt, swiglu, s) : launch_tiled_bm128(p, wt, swiglu, s);
}

}  // namespace moe
