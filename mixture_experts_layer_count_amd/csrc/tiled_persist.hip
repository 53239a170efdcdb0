// Persistent form of the LDS-tiled grouped GEMM for bf16 weights and 256-row
// tiles, for the plain GEMM without a row gather (the prefill down
// projections).
// build-flags: -mllvm -amdgpu-mfma-vgpr-form
//
// Pages: the grouped GEMM of "MoE-推理部署" (operator section) and
// "MOE推理流程解析" §二/§三 (every expert's rows in one launch), as in
// tiled_gemm_kernel.h, whose tile, ring, swizzles, fragment reads and MFMA
// grid (8 wavefronts in 2 x 4, 128 rows x 64 B-columns each) this kernel
// keeps.
//
// What differs: one workgroup per CU walks its share of the work order, so
// the copy ring never drains between work items. Cycle stamps of the
// one-item-per-workgroup kernel put the ring fill before the first MFMA at
// 20 % of a Qwen3-shaped down projection's workgroup time and the LDS-staged
// epilogue at 13 % (9 % and 7 % for gate/up). Here:
//  * XCD x takes the same contiguous run of the work order as before (so
//    an expert's weight tiles and its rows stay in that XCD's L2), and
//    its 32 workgroups take items slot, slot + 32, ... in order. Wavefront 0
//    decodes the workgroup's items into an LDS table once, at the start.
//  * the last S steps of an item issue the copies of the next item's first
//    S steps (its pointers are set between two copies of the K loop, so no
//    pointer changes inside one); the last step reads the next item's first
//    fragments.
//  * each finished tile is stored row block by row block through a small
//    LDS staging area per wavefront (8-byte writes, 16-byte row pieces read
//    back and stored), with no workgroup barrier, while the next item's
//    copies are in flight.
//  * every row block is multiplied, also past a short tile's end: copies of
//    the K loop that skip them (as the one-item kernel has) made this kernel
//    spill inside the loop. The same structure for gate/up (SwiGLU epilogue,
//    the next tile's gathered row indices copied to LDS ahead of the pointer
//    switch) measured neutral on the Mixtral shape and 4 % slower on the
//    Qwen3 shape, whose many short last tiles the one-item kernel skips, so
//    gate/up keeps the one-item kernel.
//  * register pressure: offsets of the rare paths (item switch, epilogue)
//    are recomputed from a re-read lane index, and Item holds only ints
//    (a bool member made the compiler keep item copies in LDS, behind a full
//    wait for the copy ring at every item).
#include "tiled_gemm_kernel.h"

namespace moe {

MOE_BOUNDS_FILE(persist)

namespace tiled {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kPersistItems = 64;  // work items per workgroup at most (LDS table)

struct Persist {
    typedef Ring<W_BF16, 256, 2, 4> R;
    static constexpr int cols = Out<false>::width / 4;  // output columns per wavefront
    static constexpr int sld = cols + 8;                 // staging row pitch (elements)
    static constexpr int stg_bytes = 16 * sld * 2;       // one 16-row block
    static constexpr int pieces = cols / 8;              // 16-byte pieces per staged row
    static constexpr int table = R::ring + 8 * stg_bytes;
    static constexpr int lds = table + kPersistItems * 16;
    static_assert(lds <= 160 * 1024, "LDS");
};

struct Item {
    int g, row0, row_end, n0;
    int extra;  // the extra group's item
};

__global__ __launch_bounds__(512, 1) void tiled_persist_kernel(GemmProblem p, int nN) {
    typedef Persist P;
    typedef typename P::R R;
    constexpr int S = R::S;
    constexpr int NB = R::nb;   // 4 column blocks a wavefront
    constexpr int MI = R::mi;   // 8 row blocks a wavefront
    constexpr int NC = R::per_tile;
    constexpr int NR = 2 * NB + MI;
    constexpr int W = Out<false>::width;
    static_assert(R::nA == 2 && R::nB == 2 && NB == 4 && MI == 8, "2 x 4 wavefronts of 128 x 64");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[P::lds];
    int *table = reinterpret_cast<int *>(lds + P::table);

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), wr = w / 4, wc = w % 4;
    const int i16 = lane & 15, gq = lane >> 4;
    const int nk = p.K / kBK;  // even, at least 2 S (the launcher checks)

    // ---- this workgroup's items ----
    const int n_tiles = p.tiles ? *p.n_tiles : (p.M + 255) / 256;
    const int n_work = n_tiles * nN;
    const int per = (n_work + kXcds - 1) / kXcds;
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int mine = min(per, n_work - xcd * per);  // items of this XCD
    if (slot >= mine) return;
    const int count = (mine - slot + kBlocksPerXcd - 1) / kBlocksPerXcd;
    if (MOE_BOUNDS_FAIL(count <= kPersistItems, BOUNDS_TILE)) return;
    if (w == 0 && lane < count) {
        int mt, nt;
        tile_of(p, nN, n_tiles, xcd * per + slot + kBlocksPerXcd * lane, mt, nt);
        int g, r0, r1;
        if (p.tiles) {
            const bool ok = mt < p.max_tiles;
            g = ok ? p.tiles[4 * mt] : 0;
            r0 = ok ? p.tiles[4 * mt + 1] : 0;
            r1 = ok ? p.tiles[4 * mt + 2] : 0;
            // an invalid record becomes one row of group 0 (computed, stored
            // nowhere past the problem): the debug build reports it
            if (MOE_BOUNDS_FAIL(ok && g >= 0 && g < p.n_groups && r0 >= 0 && r0 < r1 && r1 <= p.M, BOUNDS_TILE)) {
                g = 0;
                r0 = 0;
                r1 = 1;
            }
        } else {
            g = 0;
            r0 = mt * 256;
            r1 = min(r0 + 256, p.M);
        }
        *reinterpret_cast<i32x4 *>(table + 4 * lane) = i32x4{g, r0, r1, nt * W};
    }
    __syncthreads();
    auto item_at = [&](int j) {
        const i32x4 t = *reinterpret_cast<const i32x4 *>(table + 4 * j);
        Item it;
        it.g = __builtin_amdgcn_readfirstlane(t[0]);
        it.row0 = __builtin_amdgcn_readfirstlane(t[1]);
        it.row_end = __builtin_amdgcn_readfirstlane(t[2]);
        it.n0 = __builtin_amdgcn_readfirstlane(t[3]);
        it.extra = it.g == p.extra_group;
        return it;
    };

    // ---- copy sources of an item (tiled_gemm_kernel.h's layout; the A
    // rows are the item's own GEMM rows, the extra group's included) ----
    const uint16_t *a_src[2];
    const uint16_t *b_src[2];
    auto set_sources = [&](const Item &it) {
        // the lane index re-read here, so that the compiler does not keep
        // every lane-dependent offset of this rare path live through the K
        // loop (which spills)
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            int r = it.row0 + 16 * (w * 2 + q) + (ln >> 2);
            if (r >= it.row_end) r = it.row0;  // padding rows read a valid row (never stored)
            long long src = r;
            if (MOE_BOUNDS_FAIL(p.a_rows <= 0 || src < p.a_rows, BOUNDS_A_ROW)) src = 0;
            a_src[q] = reinterpret_cast<const uint16_t *>(p.A) + src * p.lda + 8 * aswz_chunk(ln);
        }
        const uint16_t *B0 = reinterpret_cast<const uint16_t *>(it.extra ? p.Bx0 : p.B0);
        const long long gofs = it.extra ? 0 : (long long)it.g * p.b_stride;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int k = 2 * (w * 2 + q) + (ln >> 5);
            const int c = (ln & 31) ^ bswz16(k);
            // N is a multiple of the tile width: no clamp
            b_src[q] = B0 + gofs + (long long)k * p.N + it.n0 + 8 * c;
        }
    };

    auto copy = [&](int q, int kt, int stage) {
        uint8_t *st = lds + stage * R::stage;
        const int k0 = kt * kBK;
        if (q < 2) copy16(a_src[q] + k0, st + (w * 2 + q) * 1024);
        else copy16(b_src[q - 2] + (long long)k0 * p.N, st + R::a_bytes + (w * 2 + (q - 2)) * 1024);
    };

    // ---- fragment reads (bf16 as in tiled_gemm_kernel.h) ----
    auto b_col = [&](int j) { return 64 * wc + 16 * j; };
    const int a_off = (wr * 128 + i16) * 64 + 16 * ((lane >> 4) ^ ((lane >> 2) & 3));
    auto read = [&](Frags<MI, NB, 2> &f, int r, int stage) {
        const uint8_t *st = lds + stage * R::stage;
        if (r < 2 * NB) {
            const int j = r >> 1, kh = r & 1;
            const int k = 8 * gq + 4 * kh + (i16 >> 2);
            const int n = b_col(j) + 4 * (i16 & 3);
            f.raw[j][kh] = ds_tr16(lds_addr(st + R::a_bytes) + k * 512 + 16 * ((n >> 3) ^ bswz16(k)) + 2 * (n & 7));
        } else {
            const int m = r - 2 * NB;
            f.a[m] = *reinterpret_cast<const bf16x8 *>(st + a_off + m * 16 * 64);
        }
    };
    auto land = [&](Frags<MI, NB, 2> &f) {
        wait_lds();
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            fence(f.raw[j][0]);
            fence(f.raw[j][1]);
            u32x4 v;
            v[0] = f.raw[j][0][0];
            v[1] = f.raw[j][0][1];
            v[2] = f.raw[j][1][0];
            v[3] = f.raw[j][1][1];
            f.b[j] = __builtin_bit_cast(bf16x8, v);
        }
    };

    f32x4 acc[MI][NB];
#pragma unroll
    for (int m = 0; m < MI; ++m)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[m][j] = f32x4{};
    // weights first: a lane's four results are one row, four adjacent columns
    auto mma_rows = [&](const Frags<MI, NB, 2> &f, int m) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NB; ++j)
            acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[j], f.a[m], acc[m][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- a finished tile, through the wavefront's staging area ----
    // LDS operations of one wavefront complete in order, so the write, read
    // back and next write need no barrier. The last item first lets the ring's
    // discarded copies land (the LDS must not be written once the workgroup
    // has ended). The accumulators are cleared for the next item.
    auto tile_out = [&](const Item &it, bool last) {
        uint16_t *stg = reinterpret_cast<uint16_t *>(lds + R::ring + w * P::stg_bytes);
        uint16_t *Cb = reinterpret_cast<uint16_t *>(p.C) + (long long)it.row0 * p.ldc + it.n0 + P::cols * wc;
        // the row stride, the tile's row count and the lane, re-read here so
        // that the compiler does not hoist the offsets out of the K loop
        // (they would live in registers through it, which spills)
        int ldc = p.ldc, rows = it.row_end - it.row0, ln = lane;
        asm volatile("" : "+v"(ldc), "+v"(rows), "+v"(ln));
        const int l16 = ln & 15, lq = ln >> 4;
        if (last) wait_vm<0>();
#pragma unroll
        for (int m = 0; m < MI; ++m) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NB; ++j)
                *reinterpret_cast<u32x2 *>(stg + l16 * P::sld + 16 * j + 4 * lq) =
                    u32x2{pack_bf16x2(acc[m][j][0], acc[m][j][1]), pack_bf16x2(acc[m][j][2], acc[m][j][3])};
#pragma unroll
            for (int c = 0; c < 16 * P::pieces / 64; ++c) {
                const int piece = ln + 64 * c;
                const int r = piece / P::pieces, pc = piece % P::pieces;
                const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + r * P::sld + 8 * pc);
                const int lrow = wr * 128 + 16 * m + r;  // row within the tile
                if (lrow < rows) *reinterpret_cast<u32x4 *>(Cb + (lrow * ldc + 8 * pc)) = v;
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[m][j] = f32x4{};
        }
    };

    // ---- the ring: fill with the first item's first S steps ----
    Item cur = item_at(0);
    set_sources(cur);
    Frags<MI, NB, 2> fa, fb;
#pragma unroll
    for (int t = 0; t < S; ++t)
#pragma unroll
        for (int q = 0; q < NC; ++q) copy(q, t, t);
    wait_vm<(S - 1) * NC>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < NR; ++r) read(fa, r, 0);
    land(fa);

    int stage = 0;
    for (int j = 0; j < count; ++j) {
        const bool has_next = j + 1 < count;
        Item nx = cur;
        if (has_next) nx = item_at(j + 1);
        // one K step: multiply step kt (f) while reading step kt + 1
        // into g (the item's last step: the next item's first) and
        // copying step src of the item whose sources are set
        auto step = [&](Frags<MI, NB, 2> &f, Frags<MI, NB, 2> &g, int src) {
            const int nstage = stage + 1 == S ? 0 : stage + 1;
#pragma unroll
            for (int m = 0; m < 2; ++m) mma_rows(f, m);
            wait_vm<(S - 2) * NC>();
            __builtin_amdgcn_s_barrier();
#pragma unroll
            for (int c = 0; c < MI - 2; ++c) {
#pragma unroll
                for (int q = c * NC / (MI - 2); q < (c + 1) * NC / (MI - 2); ++q) copy(q, src, stage);
#pragma unroll
                for (int r = c * NR / (MI - 2); r < (c + 1) * NR / (MI - 2); ++r) read(g, r, nstage);
                mma_rows(f, c + 2);
            }
            land(g);
            stage = nstage;
        };
        // steps [0, nk - S): copies of this item's steps S ..
        int kt = 0;
        for (; kt < nk - S; kt += 2) {
            step(fa, fb, kt + S);
            step(fb, fa, kt + 1 + S);
        }
        // steps [nk - S, nk): copies of the next item's first S steps, or
        // past the last item this item's last step again (into stages
        // nobody reads)
        if (has_next) set_sources(nx);
        for (; kt < nk; kt += 2) {
            step(fa, fb, has_next ? kt + S - nk : nk - 1);
            step(fb, fa, has_next ? kt + 1 + S - nk : nk - 1);
        }
        tile_out(cur, !has_next);
        cur = nx;
    }
}

}  // namespace
}  // namespace tiled

// the plain GEMM without a row gather, bf16 weights, 256-row tiles, whole
// column tiles, an even number of K steps and at least two ring depths of
// them, and at most kPersistItems work items per workgroup for the
// worst-case tile count
bool tiled_persist_fits(const GemmProblem &p, WType wt, bool swiglu, int bm) {
    typedef tiled::Ring<W_BF16, 256, 2, 4> R;
    const int W = 256;
    if (swiglu || p.row_src || wt != W_BF16 || bm != 256 || p.ksplit != 1 || p.N % W ||
        p.K % (2 * tiled::kBK) || p.K / tiled::kBK < 2 * R::S)
        return false;
    const long long mt_cap = p.tiles ? p.max_tiles : (p.M + 255) / 256;
    const long long per = (mt_cap * (p.N / W) + tiled::kXcds - 1) / tiled::kXcds;
    return (per + tiled::kBlocksPerXcd - 1) / tiled::kBlocksPerXcd <= tiled::kPersistItems;
}

hipError_t launch_tiled_persist(const GemmProblem &p, bool swiglu, hipStream_t s) {
    if (!tiled_persist_fits(p, W_BF16, swiglu, 256)) return hipErrorInvalidValue;
    if (p.M <= 0 || (p.tiles && p.max_tiles <= 0)) return hipSuccess;
    const dim3 grid(tiled::kXcds * tiled::kBlocksPerXcd), block(512);
    hipLaunchKernelGGL(tiled::tiled_persist_kernel, grid, block, 0, s, p, p.N / 256);
    return hipGetLastError();
}

}  // namespace moe
