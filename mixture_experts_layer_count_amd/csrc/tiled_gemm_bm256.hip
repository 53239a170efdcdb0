// 256-row tiles of the LDS-tiled grouped GEMM (bf16 and MXFP4 weights), 8 wavefronts,
// two per SIMD, so that one wavefront's copy and LDS-read issue overlaps the
// other's matrix-core work (5-7% faster than one 128 x 128 wavefront per
// SIMD): bf16 in a 2 x 4 grid of 128-row x 64-column wavefront tiles (fewer
// transposing B reads), MXFP4 in a 4 x 2 grid of 64 x 128 (its paired
// transposing reads cover 8 column blocks).
// build-flags: -mllvm -amdgpu-mfma-vgpr-form
// (the 128 accumulators per lane fit the architectural VGPRs of a wavefront
// that shares its SIMD.)
#include "tiled_gemm_kernel.h"

namespace moe {

MOE_BOUNDS_FILE(tiled256)

hipError_t launch_tiled_bm256(const GemmProblem &p, WType wt, bool swiglu, hipStream_t s) {
    if (wt == W_BF16) return tiled::launch_bm<W_BF16, 256, 2, 4>(p, swiglu, s);
    if (wt == W_MXFP4) return tiled::launch_bm<W_MXFP4, 256, 4>(p, swiglu, s);
    return hipErrorInvalidValue;
}

}  // namespace moe
