// LDS-tiled grouped GEMM for many rows per expert (prefill): the kernel
// template, instantiated per tile height by tiled_gemm_bm128.hip and
// tiled_gemm_bm256.hip (separate files: each is compiled with the register
// form that keeps its accumulators in place), launched by tiled_gemm.hip.
//
// The grouped GEMM of the page "MoE-推理部署" (operator section) and the page
// "MOE推理流程解析" §二/§三: every expert's block of rows runs in one launch,
// with row counts that differ per expert; §三 also asks that fusion keep
// intermediates out of HBM, so the row gather (permutation) is fused into the
// A-tile load and SwiGLU into the gate/up epilogue.
//
// Tile: BM rows (256, or 128 when experts hold few rows, always 128 for fp8
// weights) x 256 B-columns x 32 deep. Wavefronts form a WR x WC grid, each
// owning BM/WR rows x 256/WC B-columns: 2 x 2 (4 wavefronts, one per SIMD)
// for 128-row tiles; for 256-row tiles 8 wavefronts, two per SIMD: 2 x 4
// (128 rows x 64 B-columns each) with bf16 weights, 4 x 2 with MXFP4.
// The B operands are read with transposing 8-byte reads, about half the LDS
// bandwidth of the A operands' 16-byte reads, so with bf16 the taller 2 x 4
// wavefront tiles (twice the A reads, half the B reads of 4 x 2) take less
// LDS time for the same MFMAs.
//  * gate/up (SWIGLU): B-columns 0..127 are W1[:, n0:n0+128] and 128..255 are
//    W3[:, n0:n0+128]; wavefront column wc holds the W1 and W3 accumulators of
//    output columns n0 + (128/WC) wc .. +128/WC-1, so h = silu(g) * u is
//    formed in registers.
//  * down (PLAIN): B-columns are W2[:, n0:n0+256]; wavefront column wc owns
//    n0 + (256/WC) wc .. +256/WC-1.
// MI355X mapping:
//  * operands go global -> LDS with global_load_lds_dwordx4 (no register
//    staging) into a ring of S stages (S = 4..8, as many as fit in 144 KB), so
//    S - 1 K tiles are in flight while one is multiplied. Each thread waits
//    only for its own copies of the next tile (s_waitcnt vmcnt(n), n = copies
//    issued after it), then one barrier per K tile publishes the tile and
//    frees the stage read before it. One loop with one MFMA site and a fixed
//    wait keeps the accumulators in place (no register shuffling).
//  * the A tile holds 64-byte token rows, 16 rows x 4 chunks per 1 KB copy,
//    read back as 16-byte MFMA A operands (v_mfma_f32_16x16x32_bf16); the
//    chunk order inside a row is XOR-swizzled by row / 4 (measured: without
//    it the operand reads conflict 2-way).
//  * the B tile keeps the weights' [K][N] layout; the MFMA B operand (8
//    K-consecutive values of one column) is read with ds_read_b64_tr_b16
//    (bf16) or ds_read_b64_tr_b8 (fp8). 16-byte chunks of a K row are
//    XOR-swizzled by the row index (the copies fetch the swizzled chunk, since
//    a copy's lanes land in consecutive LDS), so each half-wavefront of a
//    transposing read touches every bank once.
//  * fp8 E4M3 weights are decoded exactly to bf16 after the transposing read
//    (v_cvt_scalef32_pk_bf16_fp8, scale 1); every 128-deep K block is
//    accumulated separately and added to the result times its 128x128 block
//    scale, as the block-scaled format defines.
//  * A rows are gathered through row_src by the copies themselves (the
//    permuted token matrix is never written).
//  * the next K tile's fragments are read while the current tile's MFMAs run
//    (two fragment register sets); the copies and reads are spread between
//    the MFMA groups of the row blocks, so their issue never idles the matrix
//    cores (measured: issued all at once after the barrier, they took as long
//    as the MFMAs).
//  * tile order: the row tiles of one expert times a band of column tiles
//    are consecutive, and each XCD (own L2) takes a contiguous run of that
//    order, so an expert's weight tiles and its gathered rows are read from
//    beyond L2 about once. The real tile count is read on the device, so
//    surplus workgroups of the worst-case grid exit without unbalancing the
//    XCDs.
//  * the weight fragment is the MFMA's first operand, so a lane's four
//    results are four adjacent columns of one row: the epilogue stages the
//    bf16 tile in LDS with 8-byte writes and stores 16-byte row pieces (fp32
//    output: 16-byte stores straight from the accumulators).
#pragma once

#include <type_traits>

#include "common.h"

namespace moe {
namespace tiled {

#define AS1 __attribute__((address_space(1)))
#define AS3 __attribute__((address_space(3)))
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kBK = 32;            // K depth per tile: one MFMA step
constexpr int kXcds = 8;
constexpr int kBlocksPerXcd = 32;  // one workgroup per CU (LDS-bound)
constexpr int kRingBudget = 144 * 1024;

// WR x WC wavefronts: WR rows of BM/WR tile rows, WC columns of 256/WC
// B-columns (2 x 2: one wavefront per SIMD; 4 x 2 or 2 x 4: two per SIMD)
template <int WT, int BM, int WR = 2, int WC = 2>
struct Ring {
    static constexpr int threads = 64 * WR * WC;
    static constexpr int waves = WR * WC;
    static constexpr bool fp8 = WT == W_FP8;
    static constexpr bool mx = WT == W_MXFP4;
    static constexpr int a_bytes = BM * kBK * 2;        // 64-byte bf16 rows
    // one K row of 256 B-columns (bf16 512 B, fp8 256 B); MXFP4: one row of
    // bytes, each holding two K rows of its column (256 B)
    static constexpr int b_row = (fp8 || mx) ? 256 : 512;
    static constexpr int b_bytes = (mx ? kBK / 2 : kBK) * b_row;
    // fp8: per-wavefront block-scale copies; MXFP4: the step's E8M0 scale row
    // (one byte per B-column)
    static constexpr int s_bytes = fp8 ? waves * 256 : mx ? 256 : 0;
    static constexpr int stage = a_bytes + b_bytes + s_bytes;
    static constexpr int S = (kRingBudget / stage) < 8 ? (kRingBudget / stage) : 8;
    static constexpr int nA = a_bytes / (threads * 16);  // 16-byte copies per thread per tile
    // MXFP4: the B tile is four 1 KB copies; with 8 wavefronts, wavefronts
    // 0..3 copy it and 4..7 the scale row (one copy each); with 4, each
    // copies 1 KB of B and then the scale row
    static constexpr int nB = mx ? 1 : b_bytes / (threads * 16);
    static constexpr int per_tile = nA + nB + ((fp8 || (mx && waves < 8)) ? 1 : 0);  // vector-memory ops per tile
    static constexpr int mi = BM / (16 * WR);              // 16-row MFMA blocks per wavefront
    static constexpr int nb = 16 / WC;                     // 16-column B blocks per wavefront
    static constexpr int ring = S * stage;
    // fp8 block scales and the MXFP4 read pairing assume two wavefront columns
    static_assert(WC == 2 || (!fp8 && !mx), "wavefront grid");
};

template <bool SWIGLU>
struct Out {
    static constexpr int width = SWIGLU ? 128 : 256;  // output columns per tile
    static constexpr int ld = width + 8;              // LDS staging row stride (elements)
};

template <int WT, bool SWIGLU, int BM, int WR, int WC>
constexpr int lds_bytes() {
    return Ring<WT, BM, WR, WC>::ring > BM * Out<SWIGLU>::ld * 2 ? Ring<WT, BM, WR, WC>::ring
                                                                  : BM * Out<SWIGLU>::ld * 2;
}

// A tile: 64-byte rows, 16-byte chunk c of row r stored at c ^ ((r >> 2) & 3),
// so the 8 rows an 8-lane group of a ds_read_b128 touches cover all banks.
// A copy's lane l lands in row l/4 (of its 16), physical chunk l%4, and
// therefore fetches logical chunk (l%4) ^ ((l/16) % 4).
__device__ __forceinline__ int aswz_chunk(int lane) { return (lane & 3) ^ ((lane >> 4) & 3); }
// chunk swizzles of the B tile (16-byte chunks of one K row)
__device__ __forceinline__ int bswz16(int k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }
__device__ __forceinline__ int bswz8(int k) { return k & 15; }
// MXFP4 B tile (16 byte rows of 256 B per step): chunk swizzle by byte row.
// A transposing read pairs two column chunks whose indices differ by 8
// (gate/up: W1 and W3 halves) or by 4 (down); the swizzle keeps the 8 rows
// read by each 32-lane half of a wavefront in distinct 16-byte bank groups
// for that pairing (down: byte-row bits 2 and 3 swapped, so no two rows of a
// half differ by 4 in the swizzle).
template <bool SWIGLU>
__device__ __forceinline__ int mxswz(int kb) {
    if constexpr (SWIGLU) return kb & 15;
    else return (kb & 3) | ((kb & 4) << 1) | ((kb & 8) >> 1);
}

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
template <int PER, int MAXT>
__device__ __forceinline__ void wait_tiles(int t) {
    // wait until at most t tiles (t <= MAXT) of PER copies each are in flight
    static_assert(MAXT <= 7, "ring depth");
    switch (t) {
    case 0: wait_vm<0>(); break;
    case 1: if constexpr (MAXT >= 1) wait_vm<PER>(); break;
    case 2: if constexpr (MAXT >= 2) wait_vm<2 * PER>(); break;
    case 3: if constexpr (MAXT >= 3) wait_vm<3 * PER>(); break;
    case 4: if constexpr (MAXT >= 4) wait_vm<4 * PER>(); break;
    case 5: if constexpr (MAXT >= 5) wait_vm<5 * PER>(); break;
    case 6: if constexpr (MAXT >= 6) wait_vm<6 * PER>(); break;
    default: if constexpr (MAXT >= 7) wait_vm<7 * PER>(); break;
    }
}
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14)); }

__device__ __forceinline__ void copy16(const void *g, uint8_t *l) {
    __builtin_amdgcn_global_load_lds((AS1 void *)g, (AS3 void *)l, 16, 0, 0);
}
__device__ __forceinline__ void copy4(const void *g, uint8_t *l) {
    __builtin_amdgcn_global_load_lds((AS1 void *)g, (AS3 void *)l, 4, 0, 0);
}
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) {
    return (uint32_t)(uintptr_t)(const AS3 uint8_t *)p;
}
// Transposing LDS reads, issued as plain instructions: the builtins carry no
// memory operand, which makes the compiler drain every outstanding global->LDS
// copy before them. The results are only valid after wait_lds(); fence()
// then hands them to the compiler as fresh values.
__device__ __forceinline__ u32x2 ds_tr16(uint32_t addr) {
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
    return r;
}
__device__ __forceinline__ u32x2 ds_tr8(uint32_t addr) {
    u32x2 r;
    asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(r) : "v"(addr));
    return r;
}
// the same with a constant byte offset in the instruction's offset field
template <int OFF>
__device__ __forceinline__ u32x2 ds_tr8_at(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    u32x2 r;
    asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
__device__ __forceinline__ void fence(u32x2 &v) { asm volatile("" : "+v"(v)); }

// Map this workgroup to (row tile, column tile) of the work order; false for
// surplus workgroups. Work order: for each group, for each band of gn column
// tiles, the group's row tiles x the band's column tiles (column fastest).
// XCD x (workgroup id mod 8) takes the contiguous run [x*per, (x+1)*per).
__device__ __forceinline__ void tile_of(const GemmProblem &p, int nN, int n_tiles, int id, int &mt, int &nt);
__device__ __forceinline__ bool pick_tile(const GemmProblem &p, int nN, int bm, int &mt, int &nt) {
    const int n_tiles = p.tiles ? *p.n_tiles : (p.M + bm - 1) / bm;
    const int n_work = n_tiles * nN;
    const int per = (n_work + kXcds - 1) / kXcds;
    const int slot = blockIdx.x / kXcds;
    if (slot >= per) return false;
    const int id = (blockIdx.x % kXcds) * per + slot;
    if (id >= n_work) return false;
    tile_of(p, nN, n_tiles, id, mt, nt);
    return true;
}

// Tail split. An XCD runs its n items on kBlocksPerXcd CUs; when n is not a
// multiple of that, the last round holds only tail = n % 32 items and most of
// the XCD idles through it (the Mixtral-shaped down projection has 2.25
// rounds: a third of its time at a quarter of the chip). The tail items are
// then split over K into parts = min(kTailSplit, 32 / tail) parts, one
// workgroup each, dispatched after the XCD's full rounds (only when the
// fullest XCDs' last round is at most half full). Part q of item i
// is workgroup slot full + i parts + q; tail_slot = (XCD, i) names its
// counter, part_slot = (XCD, i parts + q) its partial buffer.
constexpr int kTailSplit = 4;
constexpr int kTailSlots = kXcds * kBlocksPerXcd;  // partial buffers (and counters)
struct Unit {
    int mt, nt;
    int part = 0, parts = 1;
    int tail_slot = 0, part_slot = 0;
};
__device__ __forceinline__ bool pick_unit(const GemmProblem &p, int nN, int bm, int nk, Unit &u) {
    const int n_tiles = p.tiles ? *p.n_tiles : (p.M + bm - 1) / bm;
    const int n_work = n_tiles * nN;
    const int per = (n_work + kXcds - 1) / kXcds;
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int first = xcd * per;
    const int n = min(per, n_work - first);  // this XCD's items
    if (n <= 0) return false;
    const int tail = n % kBlocksPerXcd;
    const int full = n - tail;
    // the launch ends with the XCDs that hold `per` items: split only when
    // their last round is at most half full (else splitting any XCD's tail
    // only adds partial traffic), and never past one round of parts
    const int tail_max = per % kBlocksPerXcd;
    const int split = tail_max == 0 ? 1 : min(kTailSplit, kBlocksPerXcd / tail_max);
    int item = slot;
    if (slot >= full) {
        if (tail == 0) return false;
        const int parts = split < 2 ? 1 : min(min(split, kBlocksPerXcd / tail), nk);
        const int v = slot - full;
        if (v >= tail * parts) return false;
        item = full + v / parts;
        u.part = v % parts;
        u.parts = parts;
        u.tail_slot = xcd * kBlocksPerXcd + v / parts;
        u.part_slot = xcd * kBlocksPerXcd + v;
    }
    tile_of(p, nN, n_tiles, first + item, u.mt, u.nt);
    return true;
}

__device__ __forceinline__ void tile_of(const GemmProblem &p, int nN, int n_tiles, int id, int &mt, int &nt) {
    if (!p.tiles || !p.group_tile_start) {
        mt = id % n_tiles;
        nt = id / n_tiles;
        return;
    }
    // group holding id: a group's items are [start * nN, next start * nN), so
    // tile id / nN belongs to it, and the tile's record names the group (two
    // dependent loads instead of a search over the group starts)
    const int grp = p.tiles[4 * (id / nN)];
    const int t0 = p.group_tile_start[grp];
    const int cnt = p.group_tile_start[grp + 1] - t0;  // > 0: id lies in this group
    int gn = (kBlocksPerXcd + cnt - 1) / cnt;
    if (gn > nN) gn = nN;
    const int j = id - t0 * nN;
    const int band = j / (cnt * gn);
    const int q = j - band * cnt * gn;
    const int width = min(gn, nN - band * gn);
    nt = band * gn + q % width;
    mt = t0 + q / width;
}

// One fragment set: the A operands of the wavefront's MI row blocks, the B
// operands of its NB column blocks and (fp8) its two block scales.
// RW: transposed reads per block (bf16: 2 x 4 values; fp8: 8 values; MXFP4:
// raw[p] holds 8 K values of blocks p and p + 4, raw[4] the 8 blocks' scales)
template <int MI, int NB, int RW>
struct Frags {
    bf16x8 a[MI];
    bf16x8 b[NB];               // B operands, formed by land()
    u32x2 raw[NB][RW];
    float s0, s1;
};

// F32OUT (plain GEMM only): fp32 output straight from the accumulators, and
// split-K: blockIdx.y = split s multiplies K range [s kchunk, (s+1) kchunk)
// into C + s c_split_stride (every split must be non-empty).
template <int WT, bool SWIGLU, int BM, int WR, bool F32OUT = false, int WC = 2>
__global__ __launch_bounds__(64 * WR * WC, 1) void tiled_gemm_kernel(GemmProblem p, int nN) {
    static_assert(!(F32OUT && SWIGLU), "fp32 output is for the plain GEMM");
    typedef Ring<WT, BM, WR, WC> R;
    constexpr int NB = R::nb;
    constexpr int kT = R::threads;
    constexpr bool FP8 = R::fp8;
    constexpr bool MX = R::mx;
    static_assert(!(F32OUT && MX), "fp32 output takes bf16 weights");
    constexpr int RW = (FP8 || MX) ? 1 : 2;
    constexpr int S = R::S;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[lds_bytes<WT, SWIGLU, BM, WR, WC>()];

    // K steps of the problem (F32OUT: of this split)
    const int split = F32OUT ? (int)blockIdx.y : 0;
    const int nk_all = F32OUT ? (min(p.K, split * p.kchunk + p.kchunk) - split * p.kchunk) / kBK : p.K / kBK;
    // the tail split: down projections with bf16 or MXFP4 weights (fp8
    // weights close 128-deep scale blocks every 4 steps; the gate/up shapes
    // measured end their launches with well-filled rounds, and carrying the
    // split code cost them 2-3 %)
    constexpr bool TAIL = !F32OUT && !FP8 && !SWIGLU;
    Unit u;
    if (TAIL && p.tail_part) {
        if (!pick_unit(p, nN, BM, nk_all, u)) return;
    } else if (!pick_tile(p, nN, BM, u.mt, u.nt)) {
        return;
    }
    const int mt = u.mt, nt = u.nt;
    // this workgroup's K steps: [k_first, k_first + nk) (a tail part: its share)
    const int k_first = nk_all * u.part / u.parts;
    const int nk = nk_all * (u.part + 1) / u.parts - k_first;
    const int kbase = (F32OUT ? split * p.kchunk : 0) + k_first * kBK;  // first K of this workgroup
    int g, row0, row_end;
    if (p.tiles) {
        if (MOE_BOUNDS_FAIL(mt < p.max_tiles, BOUNDS_TILE)) return;
        g = p.tiles[4 * mt];
        row0 = p.tiles[4 * mt + 1];
        row_end = p.tiles[4 * mt + 2];
        if (MOE_BOUNDS_FAIL(g >= 0 && g < p.n_groups && row0 >= 0 && row0 < row_end && row_end <= p.M,
                            BOUNDS_TILE))
            return;
    } else {
        g = 0;
        row0 = mt * BM;
        row_end = min(row0 + BM, p.M);
    }
    const int n0 = nt * Out<SWIGLU>::width;
    const bool extra = g == p.extra_group;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), wr = w / WC, wc = w % WC;
    // 16-row blocks of this wavefront that hold rows of the group; a
    // wavefront with none (in a short last tile of an expert) skips its MFMAs
    // (its accumulators stay zero and are never stored)
    const int nblk = min(max((row_end - row0 - wr * (BM / WR) + 15) >> 4, 0), R::mi);

    // ---- copy sources (fixed over K; advanced by k0 per tile) ----
    // A: copy q of wavefront w fills rows 16 (w nA + q) .. +15, lane -> row
    // lane/4, 16-byte chunk lane%4. Rows past the tile's end copy a valid row
    // (their results are never stored).
    const uint16_t *a_src[R::nA];
#pragma unroll
    for (int q = 0; q < R::nA; ++q) {
        int r = row0 + 16 * (w * R::nA + q) + (lane >> 2);
        if (r >= row_end) r = row0;
        long long src;
        if (extra && p.row_src) src = r - p.extra_row0;
        else src = p.row_src ? (long long)(p.row_src[r] / p.gk) : (long long)r;
        if (MOE_BOUNDS_FAIL(src >= 0 && (p.a_rows <= 0 || src < p.a_rows), BOUNDS_A_ROW)) src = 0;
        a_src[q] = reinterpret_cast<const uint16_t *>(p.A) + src * p.lda + 8 * aswz_chunk(lane);
    }
    // B: copy q of wavefront w fills K rows of the B tile; each lane fetches
    // the chunk that the swizzle places at its LDS position. Columns past N
    // copy a valid chunk (their results are never stored).
    typedef typename std::conditional<FP8 || MX, uint8_t, uint16_t>::type WE;
    const WE *b_src[R::nB];
    const void *B0 = extra ? p.Bx0 : p.B0;
    const void *B1 = extra ? p.Bx1 : p.B1;
    const long long gofs = extra ? 0 : (long long)g * p.b_stride;
    // MXFP4 scale row copy: lane -> 4 bytes at 4 lane of the 256-byte row
    // (16-column chunk lane / 4), unswizzled
    const uint8_t *mx_s_src = nullptr;
    if constexpr (MX) {
        const uint8_t *S0 = reinterpret_cast<const uint8_t *>(extra ? p.Sx0 : p.S0);
        const uint8_t *S1 = reinterpret_cast<const uint8_t *>(extra ? p.Sx1 : p.S1);
        const long long sofs = extra ? 0 : (long long)g * p.s_stride;
        const int c = lane >> 2;
        const uint8_t *sb;
        int col;
        if (SWIGLU) { sb = (c >> 3) ? S1 : S0; col = n0 + 16 * (c & 7); }
        else { sb = S0; col = n0 + 16 * c; }
        if (col > p.N - 16) col = p.N - 16;
        mx_s_src = sb + sofs + col + 4 * (lane & 3);
    }
#pragma unroll
    for (int q = 0; q < R::nB; ++q) {
        int k, col;
        const void *base;
        if constexpr (MX) {
            // byte rows 4 (w % 4) .. +3 of the step: lane -> row lane / 16,
            // physical chunk lane % 16 holding the chunk the swizzle puts there
            k = 4 * (w & 3) + (lane >> 4);
            const int c = (lane & 15) ^ mxswz<SWIGLU>(k);
            if (SWIGLU) { base = (c >> 3) ? B1 : B0; col = n0 + 16 * (c & 7); }
            else { base = B0; col = n0 + 16 * c; }
            if (col > p.N - 16) col = p.N - 16;
        } else if constexpr (FP8) {
            k = 4 * (w * R::nB + q) + (lane >> 4);
            const int c = (lane & 15) ^ bswz8(k);  // 16 columns per chunk
            if (SWIGLU) { base = (c >> 3) ? B1 : B0; col = n0 + 16 * (c & 7); }
            else { base = B0; col = n0 + 16 * c; }
            if (col > p.N - 16) col = p.N - 16;
        } else {
            k = 2 * (w * R::nB + q) + (lane >> 5);
            const int c = (lane & 31) ^ bswz16(k);  // 8 columns per chunk
            if (SWIGLU) { base = (c >> 4) ? B1 : B0; col = n0 + 8 * (c & 15); }
            else { base = B0; col = n0 + 8 * c; }
            if (col > p.N - 8) col = p.N - 8;
        }
        b_src[q] = reinterpret_cast<const WE *>(base) + gofs + (long long)k * p.N + col;
    }
    // fp8 block scales: wavefront w copies its two scales (W1/W3 halves, or
    // its W2 column block twice) for every tile; lanes 0/1 pick them
    const float *s_src = nullptr;
    if constexpr (FP8) {
        const float *S0 = extra ? p.Sx0 : p.S0;
        const float *S1 = extra ? p.Sx1 : p.S1;
        const long long sofs = extra ? 0 : (long long)g * p.s_stride;
        int nb;
        const float *sb;
        if (SWIGLU) { nb = n0 >> 7; sb = (lane & 1) ? S1 : S0; }
        else { nb = min((n0 >> 7) + wc, (p.N >> 7) - 1); sb = S0; }
        s_src = sb + sofs + nb;
    }

    // ---- global -> LDS copies of one K tile: item q of NC ----
    constexpr int NC = R::per_tile;
    auto copy = [&](int q, int kt, int stage) {
        uint8_t *st = lds + stage * R::stage;
        const int k0 = kbase + kt * kBK;
        if (q < R::nA) {
            copy16(a_src[q] + k0, st + (w * R::nA + q) * 1024);
        } else if (q < R::nA + R::nB) {
            const int qb = q - R::nA;
            if constexpr (MX) {
                // a step is 16 byte rows of B and one row of scales
                if (R::waves >= 8 && w >= 4) copy4(mx_s_src + (long long)(k0 >> 5) * p.N, st + R::a_bytes + R::b_bytes);
                else copy16(b_src[0] + (long long)(k0 >> 1) * p.N, st + R::a_bytes + (w & 3) * 1024);
            } else {
                copy16(b_src[qb] + (long long)k0 * p.N, st + R::a_bytes + (w * R::nB + qb) * 1024);
            }
        } else if constexpr (FP8) {
            copy4(s_src + (long long)(k0 >> 7) * (p.N >> 7), st + R::a_bytes + R::b_bytes + w * 256);
        } else if constexpr (MX) {
            copy4(mx_s_src + (long long)(k0 >> 5) * p.N, st + R::a_bytes + R::b_bytes);
        }
    };

    // ---- fragment reads of one K tile: item r of NR (B blocks, then A row
    // blocks, then the fp8 scales); LDS byte offsets are fixed per lane ----
    constexpr int NBR = MX ? 5 : FP8 ? NB : 2 * NB;
    // B-column of the wavefront's column block j: gate/up, blocks 0..NB/2-1
    // of W1 and the same columns of W3; down, 256/WC consecutive columns
    auto b_col = [&](int j) {
        return SWIGLU ? 128 * (j / (NB / 2)) + (128 / WC) * wc + 16 * (j % (NB / 2)) : (256 / WC) * wc + 16 * j;
    };
    constexpr int NR = NBR + R::mi + (FP8 ? 1 : 0);
    const int a_off = (wr * (BM / WR) + (lane & 15)) * 64 + 16 * ((lane >> 4) ^ ((lane >> 2) & 3));
    const int i16 = lane & 15, gq = lane >> 4;
    // MXFP4: chunk of the wavefront's column block j in the 256-byte rows
    auto mx_chunk = [&](int j) { return SWIGLU ? 8 * (j >> 2) + 4 * wc + (j & 3) : 8 * wc + j; };
    auto read = [&](Frags<R::mi, NB, RW> &f, int r, int stage) {
        const uint8_t *st = lds + stage * R::stage;
        if (r < NBR) {
            const uint32_t bs = lds_addr(st + R::a_bytes);
            if constexpr (MX) {
                // r < 4: rows 0..3 of the transposed 8 x 16-byte block are byte
                // rows 4 gq .. +3 of block r's chunk, rows 4..7 the same byte
                // rows of block r + 4; lane l of a 16-lane group then holds 8 K
                // values (K 8 gq .. +7) of column l of both blocks. r == 4: the
                // scale row, row j = block j's chunk: lane l gets the 8 blocks'
                // scales of its column
                const int row = i16 >> 1, h = i16 & 1;
                if (r < 4) {
                    const int kb = 4 * gq + (row & 3);
                    const int c = mx_chunk(row < 4 ? r : r + 4);
                    f.raw[r][0] = ds_tr8(bs + kb * 256 + 16 * (c ^ mxswz<SWIGLU>(kb)) + 8 * h);
                } else {
                    f.raw[4][0] = ds_tr8(bs + R::b_bytes + 16 * mx_chunk(row) + 8 * h);
                }
            } else if constexpr (FP8) {
                const int j = r;
                const int nb = b_col(j);
                const int k = 8 * gq + (i16 >> 1);
                f.raw[j][0] = ds_tr8(bs + k * 256 + 16 * ((nb >> 4) ^ bswz8(k)) + 8 * (i16 & 1));
            } else {
                const int j = r >> 1, kh = r & 1;
                const int nb = b_col(j);
                const int k = 8 * gq + 4 * kh + (i16 >> 2);
                const int n = nb + 4 * (i16 & 3);
                f.raw[j][kh] = ds_tr16(bs + k * 512 + 16 * ((n >> 3) ^ bswz16(k)) + 2 * (n & 7));
            }
        } else if (r < NBR + R::mi) {
            const int m = r - NBR;
            f.a[m] = *reinterpret_cast<const bf16x8 *>(st + a_off + m * 16 * 64);
        } else if constexpr (FP8) {
            const float *sc = reinterpret_cast<const float *>(st + R::a_bytes + R::b_bytes + w * 256);
            f.s0 = sc[0];
            f.s1 = sc[1];
        }
    };

    // completes this wavefront's reads of f, hands the transposed reads to
    // the compiler and forms the B operands (fp8: exact E4M3 -> bf16, scale
    // 1; K order kept, byte e of a read being K row e)
    auto land = [&](Frags<R::mi, NB, RW> &f) {
        wait_lds();
        if constexpr (MX) {
            // E2M1 pairs -> bf16 times the column's E8M0 scale (the conversion
            // takes the scale's exponent field: 2^(code - 127), exact)
#pragma unroll
            for (int q = 0; q < 5; ++q) fence(f.raw[q][0]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const uint32_t word = f.raw[q][0][hh];
                    const float s = __uint_as_float(((f.raw[4][0][hh] >> (8 * q)) & 0xffu) << 23);
                    u32x4 v;
                    v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 0));
                    v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 1));
                    v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 2));
                    v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 3));
                    f.b[q + 4 * hh] = __builtin_bit_cast(bf16x8, v);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
#pragma unroll
                for (int h = 0; h < RW; ++h) fence(f.raw[j][h]);
                u32x4 v;
                if constexpr (FP8) {
                    v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f.raw[j][0][0], 1.0f, false));
                    v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f.raw[j][0][0], 1.0f, true));
                    v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f.raw[j][0][1], 1.0f, false));
                    v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f.raw[j][0][1], 1.0f, true));
                } else {
                    v[0] = f.raw[j][0][0];
                    v[1] = f.raw[j][0][1];
                    v[2] = f.raw[j][RW - 1][0];
                    v[3] = f.raw[j][RW - 1][1];
                }
                f.b[j] = __builtin_bit_cast(bf16x8, v);
            }
        }
    };

    f32x4 acc[R::mi][NB];
    f32x4 part[FP8 ? R::mi : 1][NB];  // fp8: the current 128-deep K block
#pragma unroll
    for (int m = 0; m < R::mi; ++m)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            acc[m][j] = f32x4{};
            if constexpr (FP8) part[m][j] = f32x4{};
        }

    // the NB MFMAs of row block m, kept together as one scheduling group
    // (row blocks m >= ACT, past the group's end, issue none). The weights
    // are the first operand, so the MFMA forms the transposed 16 x 16 block:
    // a lane's four results are one row (16 m + lane % 16 of the wavefront's
    // rows) and four adjacent columns (4 (lane / 16) .. +3 of the block), which
    // the epilogue stores as one 8-byte (bf16) or 16-byte (fp32) vector
    auto mma_rows = [&](const Frags<R::mi, NB, RW> &f, int m, auto act) {
        constexpr int ACT = decltype(act)::value;
        __builtin_amdgcn_sched_barrier(0);
        if (m < ACT) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if constexpr (FP8) part[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[j], f.a[m], part[m][j], 0, 0, 0);
                else acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[j], f.a[m], acc[m][j], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // fp8: add the closed 128-deep K block, times its block scales
    auto promote = [&](const Frags<R::mi, NB, RW> &f) {
        if constexpr (FP8) {
#pragma unroll
            for (int m = 0; m < R::mi; ++m)
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const float s = (SWIGLU && j >= NB / 2) ? f.s1 : f.s0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[m][j][i] += part[m][j][i] * s;
                    part[m][j] = f32x4{};
                }
        }
    };

    // One K tile per step, with a fixed number of copies in flight. Step kt
    // multiplies tile kt (fragments already in registers) row block by row
    // block; after the first one or two blocks it waits for tile kt+1 (all but the S-2
    // newest tiles' copies), publishes it with the barrier (which also means
    // every wavefront has finished reading the stage tile kt came from), and
    // spreads over the remaining blocks the copies of tile kt+S into that
    // stage and the fragment reads of tile kt+1, so the matrix cores stay
    // busy while they issue. Past the last tile the copies repeat the last
    // tile into stages nobody reads, keeping the counts fixed; the read after
    // the last tile is discarded. Two steps a loop trip swap the roles of the
    // two fragment sets instead of copying one into the other (the copy took
    // 16 register moves a step: 3-5 % on the Mixtral-shaped gate/up).
    Frags<R::mi, NB, RW> fa, fb;
#pragma unroll
    for (int t = 0; t < S; ++t)
#pragma unroll
        for (int q = 0; q < NC; ++q) copy(q, min(t, nk - 1), t);
    wait_vm<(S - 1) * R::per_tile>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < NR; ++r) read(fa, r, 0);
    land(fa);
    // Two copies of the loop: all row blocks active, or none (a wavefront
    // whose rows all lie past the group's end). Neither copy branches; both
    // issue the same copies, reads, waits and barriers, and only the MFMAs
    // differ. (Copies for 1..3 active blocks made the compiler spill.)
    auto kloop = [&](auto act) {
        int stage = 0;  // kt % S
        // one K step: multiply tile kt (cur) while reading tile kt + 1 into
        // nxt; two steps a trip swap the roles of the fragment sets
        auto step = [&](Frags<R::mi, NB, RW> &cur, Frags<R::mi, NB, RW> &nxt, int kt) {
            const int nstage = stage + 1 == S ? 0 : stage + 1;
            const int src = min(kt + S, nk - 1);
            // PRE row blocks before the barrier: with 8 row blocks, two (more
            // matrix-core work to absorb the wavefronts' skew at the barrier:
            // 1 % on the Mixtral- and Qwen3-shaped prefill layers)
            constexpr int PRE = R::mi >= 8 ? 2 : 1;
            constexpr int SLOTS = R::mi - PRE;
#pragma unroll
            for (int m = 0; m < PRE; ++m) mma_rows(cur, m, act);
            wait_vm<(S - 2) * R::per_tile>();
            __builtin_amdgcn_s_barrier();
#pragma unroll
            for (int c = 0; c < SLOTS; ++c) {
#pragma unroll
                for (int q = c * NC / SLOTS; q < (c + 1) * NC / SLOTS; ++q) copy(q, src, stage);
#pragma unroll
                for (int r = c * NR / SLOTS; r < (c + 1) * NR / SLOTS; ++r) {
                    // the fragments of row blocks this wavefront does not
                    // multiply (past the group's end) are not read, nor,
                    // with none to multiply, the B fragments
                    constexpr int ACT = decltype(act)::value;
                    const bool a_rd = r >= NBR && r < NBR + R::mi;
                    if ((a_rd && r - NBR >= ACT) || (ACT == 0 && r < NBR)) continue;
                    read(nxt, r, nstage);
                }
                mma_rows(cur, c + PRE, act);
            }
            if constexpr (FP8)
                if ((kt & 3) == 3) promote(cur);
            land(nxt);
            stage = nstage;
        };
        int kt = 0;
        for (; kt + 1 < nk; kt += 2) {
            step(fa, fb, kt);
            step(fb, fa, kt + 1);
        }
        if (kt < nk) step(fa, fb, kt);
    };
    if (nblk == 0) kloop(std::integral_constant<int, 0>{});
    else if (R::mi >= 8 && nblk <= R::mi / 2) kloop(std::integral_constant<int, R::mi / 2>{});
    else kloop(std::integral_constant<int, R::mi>{});

    if constexpr (F32OUT) {
        wait_vm<0>();  // the last (discarded) copies land before the LDS is released
        // lane holds row lane % 16 of each 16-row block and columns
        // 4 (lane / 16) .. +3 of each 16-column block: 16-byte stores (N and
        // ldc are multiples of 8)
        float *Cf = reinterpret_cast<float *>(p.C) + (long long)split * p.c_split_stride;
#pragma unroll
        for (int m = 0; m < R::mi; ++m) {
            const int row = row0 + wr * (BM / WR) + m * 16 + i16;
            if (row >= row_end) continue;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int col = n0 + (256 / WC) * wc + 16 * j + 4 * gq;
                if (col < p.N) *reinterpret_cast<f32x4 *>(Cf + (long long)row * p.ldc + col) = acc[m][j];
            }
        }
        return;
    }
    if (TAIL && u.parts > 1) {
        // tail part: publish this part's fp32 sums ([accumulator][thread]
        // 16-byte vectors, coalesced); the last part to finish adds the
        // parts in part order, all read back from memory, so the sums are the
        // same whichever part is last, and stores the tile. Its counter is
        // left at zero.
        wait_vm<0>();  // the discarded copies land before the LDS is released
        if (MOE_BOUNDS_FAIL(u.part_slot < kTailSlots && u.tail_slot < kTailSlots && u.part_slot >= u.part,
                            BOUNDS_TAIL_SLOT))
            return;
        constexpr int NGR = R::mi * NB;
        f32x4 *buf = reinterpret_cast<f32x4 *>(p.tail_part);
        f32x4 *mine = buf + (long long)u.part_slot * NGR * kT;
#pragma unroll
        for (int m = 0; m < R::mi; ++m)
#pragma unroll
            for (int j = 0; j < NB; ++j) mine[(m * NB + j) * kT + tid] = acc[m][j];
        // Every wavefront's stores complete, then one thread makes them
        // visible beyond this XCD's L2 (an agent-scope release: an L2
        // writeback, so one per workgroup, not one per wavefront) and counts
        // the part; the last part's one acquire (L1 and L2 invalidate) serves
        // the whole workgroup, which shares the CU's L1, after the barrier.
        wait_vm<0>();
        __syncthreads();
        // the flag lives in the (now idle) ring: a separate __shared__
        // variable makes the compiler drain the copies before every LDS read
        // of the K loop
        int *tail_last = reinterpret_cast<int *>(lds);
        if (tid == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            const bool last = __hip_atomic_fetch_add(p.tail_cnt + u.tail_slot, 1, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT) == u.parts - 1;
            if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            *tail_last = last;
        }
        __syncthreads();
        if (!*tail_last) return;
        const f32x4 *part0 = buf + (long long)(u.part_slot - u.part) * NGR * kT;
        // P parts: the loads of GB accumulators' partials are issued together
        auto gather = [&](auto pc) {
            constexpr int P = decltype(pc)::value;
            constexpr int GB = 2;
#pragma unroll
            for (int g0 = 0; g0 < NGR; g0 += GB) {
                f32x4 v[P][GB];
#pragma unroll
                for (int q = 0; q < P; ++q)
#pragma unroll
                    for (int i = 0; i < GB; ++i) v[q][i] = part0[((long long)q * NGR + g0 + i) * kT + tid];
#pragma unroll
                for (int i = 0; i < GB; ++i) {
                    f32x4 sum = v[0][i];
#pragma unroll
                    for (int q = 1; q < P; ++q) sum += v[q][i];
                    acc[(g0 + i) / NB][(g0 + i) % NB] = sum;
                }
            }
        };
        static_assert(kTailSplit == 4, "part counts 2..4");
        if (u.parts == 2) gather(std::integral_constant<int, 2>{});
        else if (u.parts == 3) gather(std::integral_constant<int, 3>{});
        else gather(std::integral_constant<int, 4>{});
        if (tid == 0) __hip_atomic_store(p.tail_cnt + u.tail_slot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // ---- epilogue: stage the bf16 tile in LDS, then 16-byte row stores ----
    // A lane holds four adjacent columns of one row: one 8-byte LDS write
    // each (the 16 rows of a 16-lane group land 4 banks apart, conflict-free).
    // Stores of 8 bytes straight from the accumulators were slower (each
    // covers 16 row pieces of 32 bytes: 4x the L2 write requests per byte).
    constexpr int LD = Out<SWIGLU>::ld;
    __syncthreads();  // every wavefront is done with the ring
    uint16_t *Cs = reinterpret_cast<uint16_t *>(lds);
#pragma unroll
    for (int m = 0; m < R::mi; ++m) {
        const int r = wr * (BM / WR) + m * 16 + i16;
        if constexpr (SWIGLU) {
#pragma unroll
            for (int j = 0; j < NB / 2; ++j) {
                float h[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) h[i] = silu_f32(acc[m][j][i]) * acc[m][j + NB / 2][i];
                *reinterpret_cast<u32x2 *>(Cs + r * LD + (128 / WC) * wc + 16 * j + 4 * gq) =
                    u32x2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
            }
        } else {
#pragma unroll
            for (int j = 0; j < NB; ++j)
                *reinterpret_cast<u32x2 *>(Cs + r * LD + (256 / WC) * wc + 16 * j + 4 * gq) =
                    u32x2{pack_bf16x2(acc[m][j][0], acc[m][j][1]), pack_bf16x2(acc[m][j][2], acc[m][j][3])};
        }
    }
    __syncthreads();
    constexpr int W = Out<SWIGLU>::width;
    constexpr int chunks_per_row = W / 8;
    uint16_t *Cg = reinterpret_cast<uint16_t *>(p.C);
    for (int idx = tid; idx < BM * chunks_per_row; idx += kT) {
        const int r = idx / chunks_per_row, cc = idx % chunks_per_row;
        const int row = row0 + r, col = n0 + 8 * cc;
        if (row < row_end && col < p.N)
            *reinterpret_cast<u32x4 *>(Cg + (long long)row * p.ldc + col) =
                *reinterpret_cast<const u32x4 *>(Cs + r * LD + 8 * cc);
    }
}

template <int WT, bool SWIGLU, int BM, int WR = 2, bool F32OUT = false, int WC = 2>
inline hipError_t launch_t(const GemmProblem &p, hipStream_t s) {
    const int W = Out<SWIGLU>::width;
    const int nN = (p.N + W - 1) / W;
    const long long mt_cap = p.tiles ? p.max_tiles : (p.M + BM - 1) / BM;
    long long per = (mt_cap * nN + kXcds - 1) / kXcds;  // items per XCD, worst case
    if (per <= 0) return hipSuccess;
    if (!F32OUT && !SWIGLU && WT != W_FP8 && p.tail_part) {
        // tail parts: at most kBlocksPerXcd more workgroups per XCD
        if (!p.tail_cnt || !p.tiles) return hipErrorInvalidValue;
        per += kBlocksPerXcd;
    }
    const long long blocks = per * kXcds;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((tiled_gemm_kernel<WT, SWIGLU, BM, WR, F32OUT, WC>),
                       dim3((unsigned)blocks, F32OUT ? (unsigned)p.ksplit : 1u), dim3(64 * WR * WC), 0, s, p, nN);
    return hipGetLastError();
}

template <int WT, int BM, int WR = 2, int WC = 2>
inline hipError_t launch_bm(const GemmProblem &p, bool swiglu, hipStream_t s) {
    return swiglu ? launch_t<WT, true, BM, WR, false, WC>(p, s) : launch_t<WT, false, BM, WR, false, WC>(p, s);
}

}  // namespace tiled

// per-height launchers (one translation unit each)
hipError_t launch_tiled_bm128(const GemmProblem &p, WType wt, bool swiglu, hipStream_t s);
hipError_t launch_tiled_bm256(const GemmProblem &p, WType wt, bool swiglu, hipStream_t s);

}  // namespace moe
