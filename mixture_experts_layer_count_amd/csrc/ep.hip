// Expert-parallel dispatch and combine, with the all-to-all done as a loopback
// between G ranks that share one device.
//
// Page "MOE推理流程解析" §五: experts live on different GPUs; an assignment
// whose expert is elsewhere travels as a record of the token vector plus its
// routing metadata (token id, target expert, source GPU, routing weight);
// each GPU groups what it holds by expert and runs one matrix per active
// local expert; the results travel back and the source GPU restores token
// order, applies the weights and sums. With more GPUs this is all-to-all
// traffic, and the expert weights never move.
//
// The steps either side of the one-GPU layer:
//  * dispatch (per source rank): the destination of an assignment is the
//    owner of its expert, rank e / (E/G). The assignments are bucketed by
//    destination with the single-GPU permutation (the same deterministic
//    ballot-ranked counting sort, keyed by owner instead of expert), so send
//    rows are ascending in assignment within a destination; then each send
//    row gets its token row and record (one pass, 16-byte vectors).
//  * exchange (all ranks at once): rank d's receive buffer is, for each
//    source s in ascending order, s's segment for d. Every (source,
//    destination) pair is one column of the grid; rows are copied in 16-byte
//    vectors. The return trip is the same exchange in the other direction,
//    gathering each expert rank's results straight from its permuted expert
//    output (through the inverse map of its local permutation), so results
//    arrive at the source in its send order.
//  * the receiver's local expert ids (record expert - rank * E/G) feed the
//    single-GPU permutation and grouped FFN unchanged; combine at the source
//    is the single-GPU combine with the send rows as its inverse map.
// On a multi-GPU node the exchange would be an RCCL all-to-all(v) over xGMI,
// whose split sizes are the count matrix this file's offsets come from.
#include "common.h"

namespace moe {

MOE_BOUNDS_FILE(ep)
namespace {

// key[a] = owner rank of the assignment's expert (-1: expert out of range,
// skipped by the permutation)
__global__ __launch_bounds__(256) void ep_owner_kernel(const int32_t *idx, int A, int E, int per_rank,
                                                       int32_t *key) {
    const int a = blockIdx.x * 256 + threadIdx.x;
    if (a >= A) return;
    const int e = idx[a];
    key[a] = (e >= 0 && e < E) ? e / per_rank : -1;
}

// Send row r: token row and record of assignment a = row_src[r]. One block
// per send row; the record is written by thread 0.
__global__ __launch_bounds__(256) void ep_pack_kernel(const uint4 *X, int row_vecs, const int32_t *row_src,
                                                      const int32_t *idx, const float *w, int k, int token0,
                                                      int rank, uint4 *rows, moe_ep_record *meta) {
    const int r = blockIdx.x;
    const int a = row_src[r];
    const long long t = a / k;
    for (int i = threadIdx.x; i < row_vecs; i += 256) rows[(long long)r * row_vecs + i] = X[t * row_vecs + i];
    if (threadIdx.x == 0) {
        moe_ep_record m;
        m.token = token0 + (int)t;
        m.expert = idx[a];
        m.src_rank = rank;
        m.weight = w[a];
        meta[r] = m;
    }
}

// recv[d][s] = sum over s' < s of the rows s' sends to d; recv[d][G] = total.
__global__ __launch_bounds__(1024) void ep_recv_offsets_kernel(const int32_t *send, int G, int32_t *recv) {
    for (int d = threadIdx.x; d < G; d += 1024) {
        int run = 0;
        for (int s = 0; s < G; ++s) {
            recv[(long long)d * (G + 1) + s] = run;
            run += send[(long long)s * (G + 1) + d + 1] - send[(long long)s * (G + 1) + d];
        }
        recv[(long long)d * (G + 1) + G] = run;
    }
}

// Grid: x = row chunk, y = (source s, destination d) pair. Row i of the pair:
//   out[d][out_off[d][s] + i] = in[s][g(in_off[s][d] + i)], g = gather[s] or identity.
__global__ __launch_bounds__(256) void ep_exchange_kernel(int G, const uint8_t *in, long long in_stride,
                                                          const int32_t *in_off, const int32_t *gather,
                                                          long long gather_stride, uint8_t *out,
                                                          long long out_stride, const int32_t *out_off,
                                                          int row_vecs, int rows_per_block) {
    const int s = blockIdx.y / G, d = blockIdx.y % G;
    const int lo = in_off[(long long)s * (G + 1) + d];
    const int n = in_off[(long long)s * (G + 1) + d + 1] - lo;
    const int r0 = blockIdx.x * rows_per_block;
    if (r0 >= n) return;
    const int nr = min(rows_per_block, n - r0);
    const int dst0 = out_off[(long long)d * (G + 1) + s] + r0;
    const uint4 *src_base = reinterpret_cast<const uint4 *>(in + s * in_stride);
    uint4 *dst_base = reinterpret_cast<uint4 *>(out + d * out_stride);
    const int32_t *gth = gather ? gather + s * gather_stride : nullptr;
    // rows a rank holds (the bounds-checked build's checks; 0: not known)
    const long long in_rows = in_stride / (16LL * row_vecs), out_rows = out_stride / (16LL * row_vecs);
    for (int v = threadIdx.x; v < nr * row_vecs; v += 256) {
        const int i = v / row_vecs, c = v - i * row_vecs;
        const long long j = lo + r0 + i;
        long long sr = gth ? gth[j] : j;
        if (MOE_BOUNDS_FAIL(sr >= 0 && (in_rows <= 0 || sr < in_rows), BOUNDS_EP_ROW)) sr = 0;
        if (MOE_BOUNDS_FAIL(out_rows <= 0 || dst0 + i < out_rows, BOUNDS_EP_ROW)) continue;
        dst_base[(long long)(dst0 + i) * row_vecs + c] = src_base[sr * row_vecs + c];
    }
}

__global__ __launch_bounds__(256) void ep_local_experts_kernel(const moe_ep_record *meta, int n, int lo, int per_rank,
                                                               int32_t *local) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int l = meta[i].expert - lo;
    local[i] = (l >= 0 && l < per_rank) ? l : -1;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_ep_dispatch_workspace_bytes(int T, int k, int G) {
    if (T < 0 || k < 1 || G < 1 || G > 1024 || (long long)T * k > 0x7fffffffLL) return 0;
    const int A = T * k;
    return align256(sizeof(int32_t) * (size_t)A) * 2 + align256(sizeof(int32_t) * (size_t)G) +
           align256(permute_ws_bytes(A, G));
}

moe_status moe_ep_dispatch(const int32_t *topk_idx, const float *topk_w, const void *X, moe_dtype x_dt, int T,
                           int k, int H, int E, int G, int rank, int token0, int32_t *send_offsets,
                           int32_t *send_slot, void *send_rows, moe_ep_record *send_meta, void *ws,
                           size_t ws_bytes, hipStream_t stream) {
    if (T < 0 || k < 1 || H < 1 || E < 1 || G < 1 || k > E || rank < 0 || rank >= G || token0 < 0)
        return MOE_ERR_INVALID_ARG;
    if (E % G) return MOE_ERR_INVALID_ARG;  // experts in contiguous blocks of E/G
    if (G > 1024 || E > 1024 || (long long)T * k > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
    if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    const size_t esz = x_dt == MOE_F32 ? 4 : 2;
    if (((size_t)H * esz) % 16) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!topk_idx || !topk_w || !X || !send_offsets || !send_slot || !send_rows || !send_meta)
        return MOE_ERR_INVALID_ARG;
    const size_t need = moe_ep_dispatch_workspace_bytes(T, k, G);
    if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
    const int A = T * k;
    char *p = static_cast<char *>(ws);
    int32_t *key = reinterpret_cast<int32_t *>(p);
    p += align256(sizeof(int32_t) * (size_t)A);
    int32_t *row_src = reinterpret_cast<int32_t *>(p);
    p += align256(sizeof(int32_t) * (size_t)A);
    int32_t *counts = reinterpret_cast<int32_t *>(p);
    p += align256(sizeof(int32_t) * (size_t)G);
    hipLaunchKernelGGL(ep_owner_kernel, dim3((A + 255) / 256), dim3(256), 0, stream, topk_idx, A, E, E / G, key);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    if (launch_permute(key, A, G, counts, send_offsets, row_src, send_slot, p, stream) != hipSuccess)
        return MOE_ERR_HIP;
    hipLaunchKernelGGL(ep_pack_kernel, dim3(A), dim3(256), 0, stream, static_cast<const uint4 *>(X),
                       (int)((size_t)H * esz / 16), row_src, topk_idx, topk_w, k, token0, rank,
                       static_cast<uint4 *>(send_rows), send_meta);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_ep_recv_offsets(const int32_t *send_offsets, int G, int32_t *recv_offsets, hipStream_t stream) {
    if (G < 1) return MOE_ERR_INVALID_ARG;
    if (G > 1024) return MOE_ERR_UNSUPPORTED;
    if (!send_offsets || !recv_offsets) return MOE_ERR_INVALID_ARG;
    hipLaunchKernelGGL(ep_recv_offsets_kernel, dim3(1), dim3(1024), 0, stream, send_offsets, G, recv_offsets);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_ep_exchange(int G, const void *in, long long in_rank_stride, const int32_t *in_offsets,
                           const int32_t *gather, long long gather_rank_stride, void *out,
                           long long out_rank_stride, const int32_t *out_offsets, int row_bytes, int max_rows,
                           hipStream_t stream) {
    if (G < 1 || row_bytes < 1 || max_rows < 0 || in_rank_stride < 0 || out_rank_stride < 0 ||
        gather_rank_stride < 0)
        return MOE_ERR_INVALID_ARG;
    if (G > 1024 || row_bytes % 16 || in_rank_stride % 16 || out_rank_stride % 16) return MOE_ERR_UNSUPPORTED;
    if ((uintptr_t)in % 16 || (uintptr_t)out % 16) return MOE_ERR_UNSUPPORTED;
    if (max_rows == 0) return MOE_OK;
    if (!in || !out || !in_offsets || !out_offsets) return MOE_ERR_INVALID_ARG;
    const int row_vecs = row_bytes / 16;
    // about 32 KB per block; at least one row
    int rpb = 32768 / row_bytes;
    rpb = rpb < 1 ? 1 : rpb > 256 ? 256 : rpb;
    const long long chunks = ((long long)max_rows + rpb - 1) / rpb;
    if ((long long)G * G > 65535 || chunks > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(ep_exchange_kernel, dim3((unsigned)chunks, (unsigned)(G * G)), dim3(256), 0, stream, G,
                       static_cast<const uint8_t *>(in), in_rank_stride, in_offsets, gather, gather_rank_stride,
                       static_cast<uint8_t *>(out), out_rank_stride, out_offsets, row_vecs, rpb);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_ep_local_experts(const moe_ep_record *recv_meta, int n, int E, int G, int rank, int32_t *local_idx,
                                hipStream_t stream) {
    if (n < 0 || E < 1 || G < 1 || rank < 0 || rank >= G || E % G) return MOE_ERR_INVALID_ARG;
    if (n == 0) return MOE_OK;
    if (!recv_meta || !local_idx) return MOE_ERR_INVALID_ARG;
    const int per = E / G;
    hipLaunchKernelGGL(ep_local_experts_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, recv_meta, n,
                       rank * per, per, local_idx);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
