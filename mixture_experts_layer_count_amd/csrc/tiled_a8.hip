// W8A8 grouped GEMM for many rows per expert: fp8 (OCP E4M3) weights with
// 128x128 block scales times fp8 activations with per-row 128-column scales.
// build-flags: -mllvm -amdgpu-mfma-vgpr-form
// (MFMA results in architectural VGPRs, where the per-block scaling adds
// them to the accumulators.)
//
// Pages: the grouped GEMM of "MoE-推理部署" (operator section) and
// "MOE推理流程解析" §二/§三 (one launch for every expert's rows, gather fused
// into the A load); §三 also names quantising activations before the expert
// GEMM, which is what feeds this kernel; "MoE-推理部署" (expert-quantisation
// section) gives the per-expert FP8 weight scales.
//
// Math: C[r, n] = sum over 128-deep K blocks b of
//   sa[r, b] * sw[b, n / 128] * sum_{k in b} qa[r, k] * qw[k, n]
// One v_mfma_f32_16x16x128_f8f6f4 computes exactly one block's inner sum for
// a 16x16 output tile (fresh accumulator), which is then added to the result
// times sa * sw: the scales never meet a partial sum of another block.
//
// Tile: BM rows x BN B-columns x 128 deep, BN = 64 WC; 2 x WC wavefronts in
// a 2 x WC grid, each BM/2 rows x 64 B-columns. Used: WC = 4 (8 wavefronts,
// two per SIMD, BN = 256: half the activation re-reads of BN = 128, and one
// wavefront's copies overlap the other's matrix-core work) and BM = 160 (5 x 4
// MFMA tiles a wavefront: an expert with up to 160 rows is one tile, so its
// weights are read once).
//  * gate/up (SWIGLU): B-columns 0..BN/2-1 are W1[:, n0:n0+BN/2], the rest
//    W3[:, n0:n0+BN/2]; output columns n0..n0+BN/2-1: h as bf16, or as E4M3
//    codes with one scale per row (the BN/2 = 128 columns are one scale group).
//  * down (PLAIN): B-columns are W2[:, n0:n0+BN].
// Pipeline as in the bf16 ring kernel (tiled_gemm_kernel.h): global -> LDS
// copies (global_load_lds) into a ring of S stages with a fixed count of
// copies in flight, one barrier per K step, the next step's fragments read
// between the MFMA groups of the current one.
//  * A tile: 128-byte rows (128 codes), 16-byte chunk c of row r stored at
//    c ^ ((r >> 1) & 7), so the 16 rows one 16-lane pass of a ds_read_b128
//    reads hit 16 distinct 16-byte bank groups of the 64 banks (with r & 7,
//    rows r and r + 8 share one); an operand is 32 consecutive codes (two
//    ds_read_b128).
//  * B tile: [K][N] layout, BN-byte rows, 16-byte chunk c of row k stored at
//    c ^ swz(k), so that the 16 rows that two 16-lane groups of a
//    ds_read_b64_tr_b8 read land in distinct banks; an operand is four
//    transposing reads (8 K rows each) of the lane's column.
//  * the activation scales of the tile's rows ride along with each stage, and
//    so do the weight block scales: one 4-byte copy per wavefront and stage
//    (slots of 64 rows' scales, then one slot for the two weight scales that
//    every further wavefront fills with the same copy), which keeps every
//    wavefront's count of copies per stage equal. The activation scales are
//    stored transposed and by GEMM row (As[k block][row], written there by
//    the quantiser), so a slot's 64 rows are one or two cache lines.
#include "tiled_gemm_kernel.h"

namespace moe {

MOE_BOUNDS_FILE(a8)

namespace tiled {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 8 wavefronts (256 B-columns per tile): measured 27% faster than 4 on the
// DeepSeek-V3 prefill layer
constexpr int kA8WC = 4;

constexpr int kA8BK = 128;   // K per step = one scale block
constexpr int kA8Budget = 160 * 1024;

// BM rows (160 as launched: 2 wavefront rows of BM/2) x BN B-columns
template <int WC, int BM>
struct RingA8 {
    static constexpr int threads = 128 * WC;        // 2 x WC wavefronts
    static constexpr int BN = 64 * WC;              // B-columns per tile
    static constexpr int mi = BM / 32;              // 16-row blocks per wavefront
    static constexpr int a_bytes = BM * kA8BK;
    static constexpr int b_bytes = kA8BK * BN;
    static constexpr int nsa = (BM + 63) / 64;      // activation-scale slots (64 rows each)
    static constexpr int sc_bytes = (nsa + 1) * 256;  // + one slot for the weight scales
    static constexpr int stage = a_bytes + b_bytes + sc_bytes;
    static constexpr int S = (kA8Budget / stage) < 8 ? (kA8Budget / stage) : 8;
    static constexpr int a_chunks = a_bytes / 1024;  // 1 KB copies (8 rows each)
    static constexpr int nA = (a_chunks + 2 * WC - 1) / (2 * WC);
    static constexpr int nB = b_bytes / (threads * 16);
    static constexpr int per_tile = nA + nB + 1;
    static constexpr int lanes_per_row = BN / 16;   // 16-byte chunks per B row
    static_assert(BM % 32 == 0 && 2 * WC >= nsa + 1, "tile shape");
};

template <bool SWIGLU, int WC>
struct OutA8 {
    static constexpr int width = SWIGLU ? 32 * WC : 64 * WC;
    static constexpr int ld = width + 8;
};

// B chunk swizzle: the 8 rows of a transposing read's 16-lane group (k & 7
// or (k >> 1) & 3 with the row's half of a 256-byte bank line) and the two
// groups 32 rows apart map to distinct 16-byte bank groups
template <int WC>
__device__ __forceinline__ int bswz_a8(int k) {
    if constexpr (WC == 4) return (k & 7) | (((k >> 5) & 1) << 3);
    else return ((k >> 1) & 3) ^ (((k >> 5) & 1) << 2);
}

// MULTI (plain GEMM only): a workgroup multiplies up to `per_wg`
// consecutive column tiles of its row tile with one copy ring: the ring runs
// on across the tile boundary, so only the first tile waits for it to fill,
// and each finished tile is stored from the accumulators while the next
// tile's first stages are already in flight.
template <bool SWIGLU, int WC, int BM, bool MULTI>
__global__ __launch_bounds__(128 * WC, 1) void tiled_a8_kernel(GemmProblem p, int nG, int nN, int per_wg) {
    static_assert(!(MULTI && SWIGLU), "multi-tile workgroups are for the plain GEMM");
    typedef RingA8<WC, BM> R;
    typedef OutA8<SWIGLU, WC> O;
    constexpr int S = R::S;
    constexpr int MI = R::mi;
    constexpr int LDS = (R::S * R::stage) > BM * O::ld * 2 ? R::S * R::stage : BM * O::ld * 2;
    static_assert(LDS <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS];

    int mt, ng;
    if (!pick_tile(p, nG, BM, mt, ng)) return;
    // column tiles of this workgroup: ng * per_wg .. + ntiles - 1
    const int ntiles = MULTI ? min(per_wg, nN - ng * per_wg) : 1;
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
    const int n0 = (MULTI ? ng * per_wg : ng) * O::width;  // first tile's first column
    const bool extra = g == p.extra_group;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), wr = w / WC, wc = w % WC;

    auto src_row = [&](int r) -> long long {
        if (r >= row_end) r = row0;  // padding rows read a valid row (never stored)
        long long s;
        if (extra && p.row_src) s = r - p.extra_row0;
        else s = p.row_src ? (long long)(p.row_src[r] / p.gk) : (long long)r;
        if (MOE_BOUNDS_FAIL(s >= 0 && (p.a_rows <= 0 || s < p.a_rows), BOUNDS_A_ROW)) s = 0;
        return s;
    };

    // ---- copy sources ----
    // A: copy q of wavefront w fills chunk a_chunk(q) (rows 8 chunk .. +7);
    // lane -> row lane/8, physical chunk lane%8, i.e. logical chunk
    // (lane%8) ^ ((row >> 1) & 7). When the chunks do not divide evenly, the
    // surplus copies repeat the last chunk (same bytes to the same place), so
    // every wavefront issues the same number of copies.
    auto a_chunk = [&](int q) { return min(w + 2 * WC * q, R::a_chunks - 1); };
    const uint8_t *a_src[R::nA];
#pragma unroll
    for (int q = 0; q < R::nA; ++q) {
        const int trow = 8 * a_chunk(q) + (lane >> 3);  // row within the tile
        const long long src = src_row(row0 + trow);
        a_src[q] = reinterpret_cast<const uint8_t *>(p.A) + src * p.lda + 16 * ((lane & 7) ^ ((trow >> 1) & 7));
    }
    // B: copy q of wavefront w fills 1024 / BN K rows; lane -> row
    // lane / lanes_per_row, physical chunk lane % lanes_per_row holding data
    // chunk (physical ^ swizzle)
    const uint8_t *b_src[R::nB];  // MULTI: the row start; the column is added per copy
    int b_col[MULTI ? R::nB : 1];
    const void *B0 = extra ? p.Bx0 : p.B0;
    const void *B1 = extra ? p.Bx1 : p.B1;
    const long long gofs = extra ? 0 : (long long)g * p.b_stride;
#pragma unroll
    for (int q = 0; q < R::nB; ++q) {
        constexpr int LPR = R::lanes_per_row;
        const int k = (1024 / R::BN) * (w * R::nB + q) + lane / LPR;
        const int c = (lane % LPR) ^ bswz_a8<WC>(k);
        const void *base;
        int col;
        if (SWIGLU) { base = c >= LPR / 2 ? B1 : B0; col = n0 + 16 * (c % (LPR / 2)); }
        else { base = B0; col = n0 + 16 * c; }
        if constexpr (MULTI) {
            b_col[q] = col;
            b_src[q] = reinterpret_cast<const uint8_t *>(base) + gofs + (long long)k * p.N;
        } else {
            if (col > p.N - 16) col = p.N - 16;
            b_src[q] = reinterpret_cast<const uint8_t *>(base) + gofs + (long long)k * p.N + col;
        }
    }
    // scale copy of wavefront w (one 4-byte copy per lane and stage) into
    // slot min(w, nsa): w < nsa: the A scales of rows 64 w .. +63; w >= nsa:
    // the weight block scales (the same copy into the same slot), lanes 0 / 1
    // giving W1 / W3 of block n0 / 128 (gate/up) or W2 blocks n0 / 128 and
    // n0 / 128 + 1 (down)
    const float *sc_src;
    long long sc_step;  // elements per K block
    // MULTI: weight-scale block of column tile u: min(sc_off + sc_du u, sc_max)
    // (all zero for the activation-scale copies)
    int sc_off = 0, sc_du = 0, sc_max = 0;
    const int sc_slot = min(w, R::nsa);
    if (w < R::nsa) {
        // 64 consecutive GEMM rows of the transposed scales (rows past the
        // tile's end read row0's: never used)
        int r = row0 + 64 * w + lane;
        if (r >= row_end) r = row0;
        if (MOE_BOUNDS_FAIL(r >= 0 && r < p.as_ld, BOUNDS_SCALE_ROW)) r = 0;
        sc_src = p.As + r;
        sc_step = p.as_ld;
    } else {
        const float *S0 = extra ? p.Sx0 : p.S0;
        const float *S1 = extra ? p.Sx1 : p.S1;
        const long long sofs = extra ? 0 : (long long)g * p.s_stride;
        if (SWIGLU) sc_src = ((lane & 1) ? S1 : S0) + sofs + (n0 >> 7);
        else if (MULTI) {
            sc_src = S0 + sofs;
            sc_off = (n0 >> 7) + (lane & 1);
            sc_du = O::width >> 7;
            sc_max = (p.N >> 7) - 1;
        }
        else sc_src = S0 + sofs + min((n0 >> 7) + (lane & 1), (p.N >> 7) - 1);
        sc_step = p.N >> 7;
    }

    const int nk = p.K / kA8BK;
    constexpr int NC = R::per_tile;
    // the copies of global step gs: K step kt of column tile u
    auto copy = [&](int q, int gs, int stage) {
        uint8_t *st = lds + stage * R::stage;
        const int u = MULTI ? gs / nk : 0;
        const int kt = gs - u * nk;
        const int k0 = kt * kA8BK;
        if (q < R::nA) {
            copy16(a_src[q] + k0, st + a_chunk(q) * 1024);
        } else if (q < R::nA + R::nB) {
            const int qb = q - R::nA;
            if constexpr (MULTI) {
                const int col = min(b_col[qb] + u * O::width, p.N - 16);
                copy16(b_src[qb] + (long long)k0 * p.N + col, st + R::a_bytes + (w * R::nB + qb) * 1024);
            } else {
                copy16(b_src[qb] + (long long)k0 * p.N, st + R::a_bytes + (w * R::nB + qb) * 1024);
            }
        } else {
            const float *src = sc_src + (long long)kt * sc_step;
            if (MULTI) src += min(sc_off + sc_du * u, sc_max);
            copy4(src, st + R::a_bytes + R::b_bytes + sc_slot * 256);
        }
    };

    // ---- fragment reads: B blocks (4 transposing reads each), then A row
    // blocks (two 16-byte reads each), then the weight scales ----
    struct Frag {
        i32x8 a[MI];
        i32x8 b[4];
        float s0, s1;
    };
    u32x2 raw[4][4];  // transposed reads of the set being loaded
    constexpr int NR = 16 + MI + 1;
    const int i16 = lane & 15, gq = lane >> 4;
    const int a_row = wr * (BM / 2) + i16;  // + 16 m
    // B read addresses: K row k = 32 gq + 8 t + (lane % 16) / 2 of column
    // block j. Its chunk swizzle depends only on gq and lane % 16 (8 t adds
    // neither low bits nor a carry into bit 5), so t moves the address by
    // 8 t rows exactly: one lane base per column block, and t in the
    // instruction's offset field
    uint32_t b_base[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int nb = SWIGLU ? (R::BN / 2) * (j >> 1) + 32 * wc + 16 * (j & 1) : 64 * wc + 16 * j;
        const int k = 32 * gq + (i16 >> 1);
        b_base[j] = R::a_bytes + k * R::BN + 16 * ((nb >> 4) ^ bswz_a8<WC>(k)) + 8 * (i16 & 1);
    }
    auto read = [&](Frag &f, int r, int stage) {
        const uint8_t *st = lds + stage * R::stage;
        if (r < 16) {
            const int j = r >> 2, t = r & 3;
            const uint32_t addr = lds_addr(st) + b_base[j];
            switch (t) {
            case 0: raw[j][0] = ds_tr8_at<0>(addr); break;
            case 1: raw[j][1] = ds_tr8_at<8 * R::BN>(addr); break;
            case 2: raw[j][2] = ds_tr8_at<16 * R::BN>(addr); break;
            default: raw[j][3] = ds_tr8_at<24 * R::BN>(addr); break;
            }
        } else if (r < 16 + MI) {
            const int m = r - 16;
            const int row = a_row + 16 * m;
            const uint8_t *base = st + row * 128;
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(base + 16 * ((2 * gq) ^ ((row >> 1) & 7)));
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(base + 16 * ((2 * gq + 1) ^ ((row >> 1) & 7)));
            f.a[m] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        } else {
            const float *sc = reinterpret_cast<const float *>(st + R::a_bytes + R::b_bytes + R::nsa * 256);
            if (SWIGLU) {
                f.s0 = sc[0];
                f.s1 = sc[1];
            } else {
                f.s0 = f.s1 = sc[(64 * wc) >> 7];
            }
        }
    };
    auto land = [&](Frag &f) {
        wait_lds();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int t = 0; t < 4; ++t) fence(raw[j][t]);
            f.b[j] = i32x8{(int)raw[j][0][0], (int)raw[j][0][1], (int)raw[j][1][0], (int)raw[j][1][1],
                           (int)raw[j][2][0], (int)raw[j][2][1], (int)raw[j][3][0], (int)raw[j][3][1]};
        }
    };

    f32x4 acc[MI][4];
#pragma unroll
    for (int m = 0; m < MI; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[m][j] = f32x4{};

    // row block m of the current step: 4 MFMAs (one 128-deep block each),
    // added with scale sa[row] * sw[half]. The weights are the first operand,
    // so a lane's four results are one row (16 m + lane % 16 of the
    // wavefront's rows) and four adjacent columns (16 j + 4 (lane / 16) + i):
    // one row scale per lane, and 8-byte output writes
    auto mma_rows = [&](const Frag &f, float sa, int m) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (SWIGLU) {
            // gate/up: the four MFMAs first, then the 16 scaled adds, so each
            // result is read after the other MFMAs have issued (gate/up
            // 1.77 -> 1.74 ms on the DeepSeek-shaped layer; the down
            // projection measured 0.5 % slower this way and keeps the
            // interleaved order)
            f32x4 t[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                t[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.b[j], f.a[m], f32x4{0, 0, 0, 0}, 0, 0, 0,
                                                                       0, 0, 0);
            const float sc0 = sa * f.s0, sc1 = sa * f.s1;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[m][j][i] = fmaf(t[j][i], j >= 2 ? sc1 : sc0, acc[m][j][i]);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 18, 0);  // VALU
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.b[j], f.a[m], f32x4{0, 0, 0, 0},
                                                                                0, 0, 0, 0, 0, 0);
                const float sc = sa * f.s0;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[m][j][i] = fmaf(t[i], sc, acc[m][j][i]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // this lane's row scale in each row block
    auto read_sa = [&](float (&sa)[MI], int stage) {
        const float *sc = reinterpret_cast<const float *>(lds + stage * R::stage + R::a_bytes + R::b_bytes);
#pragma unroll
        for (int m = 0; m < MI; ++m) sa[m] = sc[wr * (BM / 2) + 16 * m + i16];
    };

    Frag fa, fb;
    const int total = ntiles * nk;  // global K steps of this workgroup
#pragma unroll
    for (int t = 0; t < S; ++t)
#pragma unroll
        for (int q = 0; q < NC; ++q) copy(q, min(t, total - 1), t);
    wait_vm<(S - 1) * R::per_tile>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < NR; ++r) read(fa, r, 0);
    land(fa);
    int stage = 0;
    // MULTI: column tile u's bf16 results straight from the accumulators: a
    // lane holds four adjacent columns of one row, so each store is 8 bytes
    // and one instruction covers 32 contiguous bytes of 16 rows (the four
    // stores of j fill the wavefront's 128-byte row segments)
    // Lanes l and l ^ 16 hold columns 4 (lane / 16) .. +3 of the same row.
    // For column blocks 2 jp and 2 jp + 1, the lane with even lane / 16 takes
    // its partner's four columns of the first block and the odd one its
    // partner's of the second (one 32-bit exchange per pair of values), so
    // each lane stores 8 adjacent columns (16 bytes) and one store covers 64
    // contiguous bytes of 16 rows: half the store instructions of 8-byte
    // stores, each with twice the bytes per row.
    auto tile_out = [&](int u) {
        uint16_t *Cg = reinterpret_cast<uint16_t *>(p.C);
        const bool odd = gq & 1;
        const int cbase = n0 + u * O::width + 64 * wc + 8 * (gq >> 1);
#pragma unroll
        for (int m = 0; m < MI; ++m) {
            const int row = row0 + wr * (BM / 2) + 16 * m + i16;
#pragma unroll
            for (int jp = 0; jp < 2; ++jp) {
                const f32x4 &x0 = acc[m][2 * jp], &x1 = acc[m][2 * jp + 1];
                const uint32_t a0 = pack_bf16x2(x0[0], x0[1]), a1 = pack_bf16x2(x0[2], x0[3]);
                const uint32_t b0 = pack_bf16x2(x1[0], x1[1]), b1 = pack_bf16x2(x1[2], x1[3]);
                const uint32_t r0 = __shfl_xor(odd ? a0 : b0, 16), r1 = __shfl_xor(odd ? a1 : b1, 16);
                const u32x4 v = odd ? u32x4{r0, r1, b0, b1} : u32x4{a0, a1, r0, r1};
                const int col = cbase + 16 * (2 * jp + (odd ? 1 : 0));
                if (row < row_end && col < p.N) *reinterpret_cast<u32x4 *>(Cg + (long long)row * p.ldc + col) = v;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[m][j] = f32x4{};
        }
    };
    // one K step: multiply step gs (in cur) while copying step gs + S and
    // reading step gs + 1 into nxt; two steps per loop trip swap the roles of
    // the fragment sets, so they are never copied
    // gs: the global K step; MULTI: the last K step of a column tile stores
    // the tile and clears the accumulators for the next one
    auto step = [&](Frag &cur, Frag &nxt, int gs) {
        const int nstage = stage + 1 == S ? 0 : stage + 1;
        const int src = min(gs + S, total - 1);
        // the row scales of step gs, before the barrier lets its stage refill
        float sa[MI];
        read_sa(sa, stage);
        mma_rows(cur, sa[0], 0);
        wait_vm<(S - 2) * R::per_tile>();
        wait_lds();  // the scale reads are done before anyone refills the stage
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int c = 0; c < MI - 1; ++c) {
#pragma unroll
            for (int q = c * NC / (MI - 1); q < (c + 1) * NC / (MI - 1); ++q) copy(q, src, stage);
#pragma unroll
            for (int r = c * NR / (MI - 1); r < (c + 1) * NR / (MI - 1); ++r) read(nxt, r, nstage);
            mma_rows(cur, sa[c + 1], c + 1);
        }
        land(nxt);
        if (MULTI && gs % nk == nk - 1) tile_out(gs / nk);
        stage = nstage;
    };
    if constexpr (MULTI) {
        // nk is even, so a column tile's last step is always the second of a pair
        for (int gs = 0; gs < total; gs += 2) {
            step(fa, fb, gs);
            step(fb, fa, gs + 1);
        }
        wait_vm<0>();  // the clamped copies of the last steps land before the workgroup ends
        return;
    }
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        step(fa, fb, kt);
        step(fb, fa, kt + 1);
    }
    if (kt < nk) step(fa, fb, kt);

    // ---- epilogue: bf16 tile through LDS, 16-byte row stores ----
    if constexpr (MULTI) return;
    constexpr int LD = O::ld;
    __syncthreads();
    uint16_t *Cs = reinterpret_cast<uint16_t *>(lds);
#pragma unroll
    for (int m = 0; m < MI; ++m) {
        const int r = wr * (BM / 2) + m * 16 + i16;
        if (SWIGLU) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = silu_f32(acc[m][j][i]) * acc[m][j + 2][i];
                *reinterpret_cast<u32x2 *>(Cs + r * LD + 32 * wc + 16 * j + 4 * gq) =
                    u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<u32x2 *>(Cs + r * LD + 64 * wc + 16 * j + 4 * gq) =
                    u32x2{pack_bf16x2(acc[m][j][0], acc[m][j][1]), pack_bf16x2(acc[m][j][2], acc[m][j][3])};
        }
    }
    __syncthreads();
    if constexpr (SWIGLU && O::width == 128) {
        if (p.Cq) {
            // E4M3 codes of h instead of h: the tile's 128 columns are exactly
            // one 128-column scale group, so each row's scale is complete here.
            // Same arithmetic as the stand-alone row quantiser (scale
            // amax / 448 of the bf16 values, clamp to +-448, round to nearest
            // even); 4 adjacent threads a row, 32 columns each
            const int part = tid & 3;
            for (int r = tid >> 2; r < BM; r += R::threads / 4) {
            float v[32];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x4 raw = *reinterpret_cast<const u32x4 *>(Cs + r * LD + 32 * part + 8 * c);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[8 * c + 2 * i] = bf16_lo(raw[i]);
                    v[8 * c + 2 * i + 1] = bf16_hi(raw[i]);
                }
            }
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
            amax = fmaxf(amax, __shfl_xor(amax, 1, 4));
            amax = fmaxf(amax, __shfl_xor(amax, 2, 4));
            const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
            uint32_t qw[8];
#pragma unroll
            for (int h = 0; h < 8; ++h) {
                float q[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) q[i] = fminf(fmaxf(v[4 * h + i] / sc, -448.0f), 448.0f);
                int pk = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
                pk = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], pk, true);
                qw[h] = (uint32_t)pk;
            }
            const int row = row0 + r;
            if (row < row_end) {
                uint8_t *dst = p.Cq + (long long)row * p.ldc + n0 + 32 * part;
                *reinterpret_cast<u32x4 *>(dst) = u32x4{qw[0], qw[1], qw[2], qw[3]};
                *reinterpret_cast<u32x4 *>(dst + 16) = u32x4{qw[4], qw[5], qw[6], qw[7]};
                if (part == 0) p.Cqs[(long long)(n0 >> 7) * p.cqs_ld + row] = sc;
            }
            }
            return;
        }
    }
    constexpr int W = O::width;
    constexpr int chunks_per_row = W / 8;
    uint16_t *Cg = reinterpret_cast<uint16_t *>(p.C);
    for (int idx = tid; idx < BM * chunks_per_row; idx += R::threads) {
        const int r = idx / chunks_per_row, cc = idx % chunks_per_row;
        const int row = row0 + r, col = n0 + 8 * cc;
        if (row < row_end && col < p.N)
            *reinterpret_cast<u32x4 *>(Cg + (long long)row * p.ldc + col) =
                *reinterpret_cast<const u32x4 *>(Cs + r * LD + 8 * cc);
    }
}

// column tiles per workgroup of the plain GEMM (when K / 128 is even)
constexpr int kA8TilesPerWg = 4;

template <bool SWIGLU, int WC, int BM>
hipError_t launch_a8(const GemmProblem &p, hipStream_t s) {
    const int W = OutA8<SWIGLU, WC>::width;
    const int nN = (p.N + W - 1) / W;
    const int nk = p.K / kA8BK;
    const bool multi = !SWIGLU && nk % 2 == 0 && kA8TilesPerWg > 1 && nN > 1;
    const int per_wg = multi ? kA8TilesPerWg : 1;
    const int nG = (nN + per_wg - 1) / per_wg;
    const long long mt_cap = p.tiles ? p.max_tiles : (p.M + BM - 1) / BM;
    long long blocks = mt_cap * nG;
    blocks = (blocks + kXcds - 1) / kXcds * kXcds;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if constexpr (!SWIGLU) {
        if (multi) {
            hipLaunchKernelGGL((tiled_a8_kernel<false, WC, BM, true>), dim3((unsigned)blocks), dim3(128 * WC), 0, s, p,
                               nG, nN, per_wg);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((tiled_a8_kernel<SWIGLU, WC, BM, false>), dim3((unsigned)blocks), dim3(128 * WC), 0, s, p, nG,
                       nN, 1);
    return hipGetLastError();
}

}  // namespace
}  // namespace tiled

bool tiled_a8_supports(int N, int K) { return N >= 128 && N % 128 == 0 && K >= 128 && K % 128 == 0; }

// 160-row tiles: with up to 160 rows per expert (the DeepSeek-shaped prefill
// has 93..161) every expert is one tile, so its weights are read once
int tiled_a8_bm(long long, int) { return 160; }

hipError_t launch_tiled_a8(const GemmProblem &p, bool swiglu, int bm, hipStream_t s) {
    // quantised h output: gate/up only, with whole 128-column scale groups
    if (p.Cq && (!swiglu || !p.Cqs || p.ldc % 128 || tiled::OutA8<true, tiled::kA8WC>::width != 128))
        return hipErrorInvalidValue;
    if (p.extra_group >= 0 && (!p.Bx0 || !p.Sx0 || (swiglu && (!p.Bx1 || !p.Sx1)))) return hipErrorInvalidValue;
    if (p.Cq && p.cqs_ld < p.M) return hipErrorInvalidValue;
    if (!p.As || p.as_ld < p.M || p.ksplit != 1 || !tiled_a8_supports(p.N, p.K) || !p.S0 ||
        (swiglu && (!p.B1 || !p.S1)))
        return hipErrorInvalidValue;
    if (bm != 160) return hipErrorInvalidValue;
    return swiglu ? tiled::launch_a8<true, tiled::kA8WC, 160>(p, s) : tiled::launch_a8<false, tiled::kA8WC, 160>(p, s);
}

}  // namespace moe
