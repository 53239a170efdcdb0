// Dispatch on one GPU: per-expert counts, offsets and a stable permutation.
//
// Page "MOE推理流程解析" §二: the T*k assignments are grouped by expert into
// contiguous matrices and each row keeps its token id; §三: the permutation
// writes rows in expert order and records an inverse map for combine.
//
// Rows of an expert block are in ascending assignment order. The order is
// decided without atomics, so the result is bit-identical run to run:
//  1. rank: one 1024-thread block per chunk of 1024 assignments. Inside a
//     wavefront, lanes holding the same expert are found with log2(E)
//     ballots; a lane's rank among them is a popcount of the lower lanes.
//     Per-wave counts go to LDS and are prefix-summed across the 16 waves.
//     The block writes its per-expert totals and each assignment's rank
//     within the chunk.
//  2. scan (one block): per expert, an exclusive sum over chunks, then an
//     exclusive scan over experts gives offsets; chunk bases are offset by it.
//  3. scatter: row = chunk base + rank; row_src[row] = a, assign_row[a] = row.
// When all assignments fit one chunk, the three steps run in one block. The
// block that forms the offsets (that one, or the scan block) also writes the
// grouped GEMMs' tile list (the work of build_tiles_kernel), saving a launch.
#include "common.h"

namespace moe {

MOE_BOUNDS_FILE(permute)
namespace {

constexpr int kChunk = 1024;

__device__ __forceinline__ int ceil_log2(int E) {
    int b = 0;
    while ((1 << b) < E) ++b;
    return b;
}

// Tile list of the grouped GEMMs (the records of build_tiles_kernel), written
// by a block that has just formed the offsets: thread g < E holds group g's
// rows [lo, hi), thread E the extra group's (when tr.extra_rows > 0); the host
// guarantees E + 1 <= 1024 groups. Called by the whole block.
__device__ __forceinline__ void emit_tiles(const TileRequest &tr, int E, int lo, int hi, int *scan_lds) {
    const int tid = threadIdx.x;
    for (int i = tid; i < tr.n_zero; i += blockDim.x) tr.zero[i] = 0;
    const int NG = E + (tr.extra_rows > 0 ? 1 : 0);
    const int n = tid < NG ? (hi - lo + tr.bm - 1) / tr.bm : 0;
    int nt = 0;
    const int first = block_exclusive_scan(n, scan_lds, &nt);
    if (tid < NG) {
        if (tr.group_tile_start) tr.group_tile_start[tid] = first;
        for (int i = 0; i < n; ++i) {
            int32_t *t = tr.tiles + 4 * (first + i);
            t[0] = tid;
            t[1] = lo + i * tr.bm;
            t[2] = min(lo + (i + 1) * tr.bm, hi);
            t[3] = 0;
        }
    }
    if (tid == 0) {
        *tr.n_tiles = nt;
        if (tr.group_tile_start) tr.group_tile_start[NG] = nt;
    }
}

template <bool SINGLE>
__global__ __launch_bounds__(kChunk) void permute_rank_kernel(
    const int32_t *idx, int A, int E, int32_t *chunk_counts, int32_t *rank, int32_t *counts,
    int32_t *offsets, int32_t *row_src, int32_t *assign_row, TileRequest tr) {
    // [16][E] per-wave counts, then per-wave prefixes (<= 1024: 16 bits)
    extern __shared__ unsigned short lds[];
    __shared__ int scan_lds[16];
    __shared__ int off_lds[SINGLE ? 1024 : 1];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int a = blockIdx.x * kChunk + tid;

    int e = (a < A) ? idx[a] : -1;
    if (e < 0 || e >= E) e = -1;

    for (int i = tid; i < 16 * E; i += kChunk) lds[i] = 0;
    __syncthreads();

    const unsigned long long valid = __ballot(e >= 0);
    unsigned long long same = valid;
    const int nbits = ceil_log2(E);
    for (int b = 0; b < nbits; ++b) {
        const int bit = (e >> b) & 1;
        const unsigned long long bal = __ballot(bit);
        same &= bit ? bal : ~bal;
    }
    const unsigned long long below = (1ull << lane) - 1ull;
    const int r_in_wave = __popcll(same & below);
    if (e >= 0 && r_in_wave == 0) lds[wid * E + e] = (unsigned short)__popcll(same);
    __syncthreads();

    // exclusive prefix over the 16 waves, per expert (one thread per expert)
    int total = 0;
    if (tid < E) {
        for (int w = 0; w < 16; ++w) {
            const int c = lds[w * E + tid];
            lds[w * E + tid] = (unsigned short)total;
            total += c;
        }
    }
    __syncthreads();
    const int r_in_chunk = (e >= 0) ? lds[wid * E + e] + r_in_wave : 0;

    if constexpr (!SINGLE) {
        if (tid < E) chunk_counts[(long long)blockIdx.x * E + tid] = total;
        if (e >= 0) rank[a] = r_in_chunk;
    } else {
        int all = 0;
        const int off = block_exclusive_scan(tid < E ? total : 0, scan_lds, &all);
        if (tid < E) {
            counts[tid] = total;
            offsets[tid] = off;
            off_lds[tid] = off;
        }
        if (tid == 0) offsets[E] = all;
        __syncthreads();
        if (e >= 0) {
            const int row = off_lds[e] + r_in_chunk;
            if (!MOE_BOUNDS_FAIL(row >= 0 && row < A, BOUNDS_PERM_ROW)) {
                row_src[row] = a;
                assign_row[a] = row;
            }
        }
        if (tr.tiles) {
            // the extra group's rows follow the routed ones
            const bool real = tid < E;
            emit_tiles(tr, E, real ? off : all, real ? off + total : all + tr.extra_rows, scan_lds);
        }
    }
}

// Per-chunk counts -> each chunk's first row in its expert block. The 1024
// threads split into P = min(1024 / E, chunks) groups; thread (group s,
// expert e) owns a contiguous run of chunks of expert e. Pass 1 sums the run
// (loads in batches of 16, so their latencies overlap), the runs and the
// experts are scanned in LDS, and pass 2 rewrites the run's counts as
// exclusive prefixes (from the registers of pass 1 when the run is one batch).
__global__ __launch_bounds__(1024) void permute_scan_kernel(int32_t *chunk_counts, int nchunks,
                                                            int E, int32_t *counts,
                                                            int32_t *offsets, TileRequest tr) {
    __shared__ int run_sum[1024];
    __shared__ int expert_off[1024];
    __shared__ int scan_lds[16];
    const int tid = threadIdx.x;
    const int P = min(1024 / E, nchunks);
    const int e = tid % E, sg = tid / E;
    const bool act = sg < P;
    const int per = (nchunks + P - 1) / P;
    const int c0 = act ? min(nchunks, sg * per) : 0;
    const int c1 = act ? min(nchunks, c0 + per) : 0;

    int sum = 0;
    int v0[16] = {};  // the first batch of the run
    for (int c = c0; c < c1; c += 16) {
        int v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = c + u < c1 ? chunk_counts[(long long)(c + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) sum += v[u];
        if (c == c0) {
#pragma unroll
            for (int u = 0; u < 16; ++u) v0[u] = v[u];
        }
    }
    run_sum[tid] = sum;
    __syncthreads();
    int before = 0, total = 0;
    if (act) {
        for (int g = 0; g < P; ++g) {
            const int v = run_sum[g * E + e];
            if (g < sg) before += v;
            total += v;
        }
    }
    int all = 0;
    const int off = block_exclusive_scan(act && sg == 0 ? total : 0, scan_lds, &all);
    if (act && sg == 0) expert_off[e] = off;
    __syncthreads();
    if (act) {
        int run = expert_off[e] + before;
        if (per <= 16) {
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (c0 + u < c1) chunk_counts[(long long)(c0 + u) * E + e] = run;
                run += v0[u];
            }
        } else {
            for (int c = c0; c < c1; c += 16) {
                int v[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) v[u] = c + u < c1 ? chunk_counts[(long long)(c + u) * E + e] : 0;
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    if (c + u < c1) chunk_counts[(long long)(c + u) * E + e] = run;
                    run += v[u];
                }
            }
        }
        if (sg == 0) {
            counts[e] = total;
            offsets[e] = off;
        }
    }
    if (tid == 0) offsets[E] = all;
    // the grouped GEMMs' tile list (thread e < E is (group 0, expert e): its
    // off and total are the expert's offset and count)
    if (tr.tiles) {
        const bool real = tid < E;
        emit_tiles(tr, E, real ? off : all, real ? off + total : all + tr.extra_rows, scan_lds);
    }
}

__global__ __launch_bounds__(256) void permute_scatter_kernel(const int32_t *idx, int A, int E,
                                                              const int32_t *chunk_base,
                                                              const int32_t *rank,
                                                              int32_t *row_src,
                                                              int32_t *assign_row) {
    const int a = blockIdx.x * 256 + threadIdx.x;
    if (a >= A) return;
    const int e = idx[a];
    if (e < 0 || e >= E) return;
    const int row = chunk_base[(long long)(a / kChunk) * E + e] + rank[a];
    if (MOE_BOUNDS_FAIL(row >= 0 && row < A, BOUNDS_PERM_ROW)) return;
    row_src[row] = a;
    assign_row[a] = row;
}

// Xp[r] = X[row_src[r] / gk] for the rows the permutation wrote (r <
// *n_rows when given: assignments of experts outside [0, E) get no row); one
// block per row, 16-byte vectors.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4 *X, int row_vecs,
                                                          const int32_t *row_src, int gk,
                                                          const int32_t *n_rows, long long x_rows,
                                                          uint4 *Xp) {
    const int r = blockIdx.x;
    if (n_rows && r >= *n_rows) return;
    long long src = row_src[r] / gk;
    if (MOE_BOUNDS_FAIL(src >= 0 && src < x_rows, BOUNDS_A_ROW)) src = 0;
    for (int i = threadIdx.x; i < row_vecs; i += 256)
        Xp[(long long)r * row_vecs + i] = X[src * row_vecs + i];
}

}  // namespace

// a block of 1024 threads can write the tile list of E (+1) groups
static bool tile_request_fits(const TileRequest *tr, int E) {
    return tr && tr->tiles && tr->n_tiles && tr->bm > 0 && tr->extra_rows >= 0 &&
           E + (tr->extra_rows > 0 ? 1 : 0) <= kChunk;
}

size_t permute_ws_bytes(int A, int E) {
    const long long nchunks = (A + kChunk - 1) / kChunk;
    if (nchunks <= 1) return 0;
    return (size_t)(nchunks * E + A) * sizeof(int32_t);
}

hipError_t launch_permute(const int32_t *idx, int A, int E, int32_t *counts, int32_t *offsets,
                          int32_t *row_src, int32_t *assign_row, void *ws, hipStream_t s,
                          const TileRequest *tr, bool *tiles_built) {
    if (A < 0 || E < 1 || E > 1024) return hipErrorInvalidValue;
    if (tiles_built) *tiles_built = false;
    const int nchunks = (A + kChunk - 1) / kChunk;
    const size_t lds = (size_t)16 * E * sizeof(unsigned short);
    if (nchunks <= 1) {
        TileRequest t{};
        if (tile_request_fits(tr, E)) {
            t = *tr;
            if (tiles_built) *tiles_built = true;
        }
        hipLaunchKernelGGL(permute_rank_kernel<true>, dim3(1), dim3(kChunk), lds, s, idx, A, E,
                           nullptr, nullptr, counts, offsets, row_src, assign_row, t);
        return hipGetLastError();
    }
    int32_t *chunk_counts = reinterpret_cast<int32_t *>(ws);
    int32_t *rank = chunk_counts + (size_t)nchunks * E;
    hipLaunchKernelGGL(permute_rank_kernel<false>, dim3(nchunks), dim3(kChunk), lds, s, idx, A, E,
                       chunk_counts, rank, nullptr, nullptr, nullptr, nullptr, TileRequest{});
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    TileRequest t{};
    if (tile_request_fits(tr, E)) {
        t = *tr;
        if (tiles_built) *tiles_built = true;
    }
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, s, chunk_counts, nchunks, E,
                       counts, offsets, t);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(permute_scatter_kernel, dim3((A + 255) / 256), dim3(256), 0, s, idx, A, E,
                       chunk_counts, rank, row_src, assign_row);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const void *X, int elem_bytes, int H, const int32_t *row_src,
                              int gk, int A, void *Xp, hipStream_t s, const int32_t *n_rows) {
    if (A <= 0) return hipSuccess;
    const long long row_bytes = (long long)H * elem_bytes;
    if (row_bytes % 16 || gk < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gather_rows_kernel, dim3(A), dim3(256), 0, s,
                       reinterpret_cast<const uint4 *>(X), (int)(row_bytes / 16), row_src, gk, n_rows,
                       (long long)((A + gk - 1) / gk), reinterpret_cast<uint4 *>(Xp));
    return hipGetLastError();
}

}  // namespace moe
