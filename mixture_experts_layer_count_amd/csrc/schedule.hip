// Device-side tile list for the grouped GEMMs.
//
// Page "MOE推理流程解析" §二: one launch runs every expert's matrix even though
// their row counts differ. The row counts live on the device (they come out
// of the permutation), so the list of (expert, first row) tiles is built on
// the device too: no device-to-host copy, and the whole layer stays capturable
// in a HIP graph. The GEMM grids are sized for the worst case
// (ceil(M / bm) + G tiles) and surplus workgroups exit at once.
#include "common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t *offsets, int G, int extra_rows,
                                                           int bm, int32_t *tiles, int32_t *n_tiles,
                                                           int32_t *group_tile_start, int32_t *zero,
                                                           int n_zero) {
    __shared__ int scan_lds[16];
    for (int i = threadIdx.x; i < n_zero; i += 1024) zero[i] = 0;
    const int NG = G + (extra_rows > 0 ? 1 : 0);
    int carry = 0;
    // groups in rounds of 1024; each thread emits its group's tiles
    for (int g0 = 0; g0 < NG; g0 += 1024) {
        const int g = g0 + threadIdx.x;
        int lo = 0, hi = 0, n = 0;
        if (g < NG) {
            lo = offsets[g];
            hi = g < G ? offsets[g + 1] : lo + extra_rows;
            n = (hi - lo + bm - 1) / bm;
            if (n < 0) n = 0;
        }
        int total = 0;
        const int first = block_exclusive_scan(n, scan_lds, &total) + carry;
        if (g < NG && group_tile_start) group_tile_start[g] = first;
        for (int i = 0; i < n; ++i) {
            int *t = tiles + 4 * (first + i);
            t[0] = g;
            t[1] = lo + i * bm;
            t[2] = min(lo + (i + 1) * bm, hi);
            t[3] = 0;
        }
        carry += total;
    }
    if (threadIdx.x == 0) {
        *n_tiles = carry;
        if (group_tile_start) group_tile_start[NG] = carry;
    }
}

}  // namespace

hipError_t launch_build_tiles(const int32_t *offsets, int G, int extra_rows, int bm, int32_t *tiles,
                              int32_t *n_tiles, int32_t *group_tile_start, hipStream_t s, int32_t *zero,
                              int n_zero) {
    if (G < 1 || bm < 1 || extra_rows < 0 || n_zero < 0 || (n_zero > 0 && !zero)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, G, extra_rows, bm, tiles,
                       n_tiles, group_tile_start, zero, n_zero);
    return hipGetLastError();
}

}  // namespace moe
