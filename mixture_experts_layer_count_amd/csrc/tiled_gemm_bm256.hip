// 256-row tiles of the LDS-tiled grouped GEMM (bf16 weights). The 256
// accumulators per lane live in the AGPRs (the default register form).
#include "tiled_gemm_kernel.h"

namespace moe {

hipError_t launch_tiled_bm256(const GemmProblem &p, WType wt, bool swiglu, hipStream_t s) {
    if (wt != W_BF16) return hipErrorInvalidValue;
    return tiled::launch_bm<W_BF16, 256>(p, swiglu, s);
}

}  // namespace moe
