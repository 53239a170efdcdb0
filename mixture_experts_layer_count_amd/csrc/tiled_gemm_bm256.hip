// 256-row tiles of the LDS-tiled grouped GEMM (bf16 and MXFP4 weights), 8 wavefronts:
// a 4 x 2 grid of 64-row x 128-column wavefront tiles, two wavefronts per
// SIMD, so that one wavefront's copy and LDS-read issue overlaps the other's
// matrix-core work (5-7% faster than one 128 x 128 wavefront per SIMD).
// build-flags: -mllvm -amdgpu-mfma-vgpr-form
// (the 128 accumulators per lane fit the architectural VGPRs of a wavefront
// that shares its SIMD.)
#include "tiled_gemm_kernel.h"

namespace moe {

hipError_t launch_tiled_bm256(const GemmProblem &p, WType wt, bool swiglu, hipStream_t s) {
    if (wt == W_BF16) return tiled::launch_bm<W_BF16, 256, 4>(p, swiglu, s);
    if (wt == W_MXFP4) return tiled::launch_bm<W_MXFP4, 256, 4>(p, swiglu, s);
    return hipErrorInvalidValue;
}

}  // namespace moe
