// 128-row tiles of the LDS-tiled grouped GEMM (bf16, fp8 and MXFP4 weights).
// build-flags: -mllvm -amdgpu-mfma-vgpr-form
// (MFMA accumulators in the architectural VGPRs: at 128 rows per tile they
// fit, and the register allocator then keeps every accumulator in place
// across the K loop instead of rotating it through the AGPRs.)
#include "tiled_gemm_kernel.h"

namespace moe {

MOE_BOUNDS_FILE(tiled128)

hipError_t launch_tiled_bm128(const GemmProblem &p, WType wt, bool swiglu, hipStream_t s) {
    switch (wt) {
    case W_BF16: return tiled::launch_bm<W_BF16, 128>(p, swiglu, s);
    case W_FP8: return tiled::launch_bm<W_FP8, 128>(p, swiglu, s);
    case W_MXFP4: return tiled::launch_bm<W_MXFP4, 128>(p, swiglu, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
