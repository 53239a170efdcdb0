// Router logits on the LDS-tiled GEMM: 128-row tiles, fp32 output and
// split-K partials (summed in fixed order by the top-k kernel).
// build-flags: -mllvm -amdgpu-mfma-vgpr-form
//
// Page "MoE serving production quirks" (memory-paradox section): the gate is
// a linear projection over all experts. For many tokens the row-streaming
// GEMV re-reads the gate matrix once per 16 rows; one 128 x 256 tile reads it
// once per 128 rows and multiplies on the matrix cores.
#include "tiled_gemm_kernel.h"

namespace moe {

MOE_BOUNDS_FILE(tiledf32)

bool tiled_f32_supports(int M, int N, int K, int ksplit, int kchunk) {
    return M > 0 && N >= 16 && N % 8 == 0 && K % tiled::kBK == 0 && ksplit >= 1 && kchunk % tiled::kBK == 0 &&
           kchunk > 0 && (long long)(ksplit - 1) * kchunk < K;
}

hipError_t launch_tiled_f32(const GemmProblem &p, hipStream_t s) {
    if (p.tiles || p.row_src || p.extra_group >= 0 || !tiled_f32_supports(p.M, p.N, p.K, p.ksplit, p.kchunk))
        return hipErrorInvalidValue;
    return tiled::launch_t<W_BF16, false, 128, 2, true>(p, s);
}

}  // namespace moe
