// LDS-tiled grouped GEMM for many rows per expert (prefill). Not built yet:
// every shape reports unsupported, so planning falls back to the
// row-streaming kernel.
#include "common.h"

namespace moe {

int tiled_gemm_bm() { return 128; }

bool tiled_gemm_supports(WType, int, int) { return false; }

hipError_t launch_tiled_gemm(const GemmProblem &, WType, bool, bool, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace moe
