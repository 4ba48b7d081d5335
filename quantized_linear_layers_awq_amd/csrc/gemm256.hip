// Prefill GEMM with fused dequantization on 256 x 256 output tiles, for W4
// and W8 weights whose groups are whole 128-row k-tiles (G a multiple of
// 128, or G == K).  TileFuse summary, Methodology section 1: each weight tile is
// unpacked and dequantized once, kept in core-local memory and reused by
// every row of the output tile.
//
// MI355X design.  A workgroup of 8 waves (two per SIMD) owns a 256 x 256
// output tile; the waves form a 2 x 4 grid of 128 x 64 sub-tiles, each
// 4 x 2 bf16 32x32x16 MFMA tiles (128 fp32 accumulators per lane, in arch
// VGPRs).  Compared with 256 x 128 tiles this halves the activation bytes
// each workgroup moves into LDS per flop, and each wave's fragment reads
// per MFMA fall by a quarter; measured on the bare pipeline (LDS-DMA of the
// activations, unpack stores, barriers) that is 1.2-1.35x the throughput of
// 256 x 128 tiles.
//
// K advances in stages of 64 rows:
//   - activations: a ring of two [256][64] bf16 stages filled by LDS-DMA one
//     stage ahead;
//   - codes: W4, one k-tile (16 blocks x 1 KiB) by LDS-DMA, a k-tile ahead;
//     each unpacking lane reads its 16-byte unit of both blocks it unpacks
//     one stage before the first use and keeps the second half in
//     registers, so the buffer is free for the next k-tile after one stage.
//     W8 (a k-tile is two 1 KiB halves per block, one per stage): the half
//     of stage s + 2, fetched during stage s into the slots of the wave that
//     unpacks it, once that wave has read stage s + 1's;
//   - records: the k-tile's record of each block (2 x 4 KiB ring), a k-tile
//     ahead.
// Every load a stage issues is waited for at its end, before the one barrier
// per stage, so no load is issued past the last stage.  Wave w unpacks blocks 2w and 2w + 1 of the tile into the next
// stage's B buffer ([8 k-octets][256 columns] of exact bf16 q - z) while the
// current stage multiplies.
//
// Scales: the accumulators hold their partial sum divided by the scale of
// their latest group (one chain).  At a group's first slice each 32 x 32
// tile is multiplied by s_prev / s_new just before its first MFMA of the
// group, so the rescale of one tile overlaps the MFMAs of the others.  A zero
// scale keeps the previous scale (its group's operands are zero).  The output
// is the chain times the last scale.
#include "tf_common.h"
#include "tf_gemm_common.h"
#include "tf_launch.h"
#include "tf_operands.h"

namespace tf {

namespace {

constexpr int kBM = 256, kBN = 256;
constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kTileBlocks = kBN / kBlockCols;  // 16 packed blocks per column tile
constexpr int kAStageB = kBM * kStage * 2;     // 32 KiB of activations per stage
constexpr int kBStageB = kBN * kStage * 2;     // 32 KiB of exact bf16 (q - z) per stage
constexpr int kBOct = kBN * 16;                // bytes per k-octet row of a B stage
constexpr int kCodeBufB = kTileBlocks * 1024;  // one W4 k-tile of the 16 blocks
constexpr int kRecBlockB = 256;                // record bytes staged per block (one dword per lane)
constexpr int kRecBufB = kTileBlocks * kRecBlockB;
constexpr int kOffB = 2 * kAStageB;
constexpr int kOffCodes = kOffB + 2 * kBStageB;
constexpr int kOffRec = kOffCodes + kCodeBufB;
constexpr int kLds = kOffRec + 2 * kRecBufB; // 152 KiB
static_assert(kLds <= 160 * 1024, "LDS of one CU");
constexpr int kAJ = kBM * kStage * 2 / 16 / kThreads; // activation DMAs per lane and stage (4)

} // namespace

// The grid covers `splits` ranges of split_tiles k-tiles and, per range,
// m_tiles row tiles x (gridDim.x / splits / m_tiles) column tiles of 256.
// kMode: kGOneTile (G == 128, or G == K == 128) or kGWhole (groups of whole
// k-tiles).  With one range the output is y (bf16); with several, each range
// writes fp32 partial sums to ws[range][M][N].
template <int BITS, int kMode, int ACT>
__global__ __launch_bounds__(kThreads, 1) void gemm256_kernel(const uint16_t *__restrict__ x,
                                                              const uint8_t *__restrict__ packed,
                                                              uint16_t *__restrict__ y, Layout lay, int64_t M,
                                                              int m_tiles, int splits, int split_tiles,
                                                              float *__restrict__ ws)
{
    static_assert(kMode == kGOneTile || kMode == kGWhole, "groups of whole k-tiles");
    constexpr int RB = record_bytes(BITS);
    constexpr bool F16 = ACT == kActF16; // fp16 x, scales and y (else bf16)
    constexpr bool one_tile = kMode == kGOneTile;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;    // 128-row and 64-column slot of the wave
    const int r = lane & 15, o = lane >> 4;     // unpack: column r of a block, k-octet o
    const int l32 = lane & 31, h32 = lane >> 5; // MFMA fragments: row / column l32, k-octet h32

    // ---- tile order: each XCD (workgroups bid % 8) takes a contiguous range
    //      of tiles, in bands of kBand row tiles (rows first within a band) ----
    const int nwg = gridDim.x, bid = blockIdx.x;
    const int xcd = bid & 7, local = bid >> 3, q8 = nwg >> 3, rem = nwg & 7;
    const int tile_all = xcd < rem ? xcd * (q8 + 1) + local : rem * (q8 + 1) + (xcd - rem) * q8 + local;
    const int per_split = nwg / splits;
    const int split = tile_all / per_split, tile = tile_all - split * per_split;
    const int n_tiles = per_split / m_tiles;
    const int band_rows = kBand < m_tiles ? kBand : m_tiles;
    const int band = tile / (band_rows * n_tiles), in_band = tile - band * band_rows * n_tiles;
    const int rows_here = m_tiles - band * band_rows < band_rows ? m_tiles - band * band_rows : band_rows;
    const int nt = in_band / rows_here, mt = band * band_rows + (in_band - nt * rows_here);
    const int64_t m0 = (int64_t)mt * kBM;
    const int64_t blk0 = (int64_t)nt * kTileBlocks;

    // ---- this split's k range as a layout of its own (records from its first
    //      group, codes from its first k-tile); ranges start on group
    //      boundaries, and with one group over all of K each range is a
    //      one-group layout ----
    const int64_t lda = lay.K;
    Layout L = lay;
    int64_t k_begin = 0, g_begin = 0;
    if (splits > 1) {
        const int64_t kt0 = (int64_t)split * split_tiles;
        const int64_t kt1 = kt0 + split_tiles < lay.ktiles ? kt0 + split_tiles : lay.ktiles;
        k_begin = kt0 * kTileRows;
        const int64_t k_end = kt1 * kTileRows < lay.K ? kt1 * kTileRows : lay.K;
        g_begin = lay.G == lay.K ? 0 : k_begin / lay.G;
        L.K = k_end - k_begin;
        L.ktiles = kt1 - kt0;
        L.steps = L.K / kStepRows;
        if (lay.G == lay.K) {
            L.G = L.K;
            L.ngroups = 1;
            L.tiles_per_group = L.ktiles;
        } else {
            L.ngroups = L.K / lay.G;
        }
        L.meta_bytes = lay.meta_bytes - g_begin * RB + kt0 * tile_bytes(BITS);
    }
    const uint8_t *const pk = packed + g_begin * RB;
    const int ktiles = (int)L.ktiles;
    const int nstages = 2 * ktiles;
    const int steps = (int)L.steps;
    const int64_t K = L.K;
    const int tpg = one_tile ? 1 : (int)L.tiles_per_group; // k-tiles per group

    uint8_t *const sA = lds;
    uint8_t *const sB = lds + kOffB;
    uint8_t *const sCodes = lds + kOffCodes;
    uint8_t *const sRec = lds + kOffRec;

    // ---- activations: wave w fills rows 32 w .. 32 w + 31 of a stage, 8 rows
    //      per instruction j; lane p takes row 8 j + p / 8 and the 16-byte unit
    //      the swizzle places at slot p % 8.  Rows past M read row M - 1
    //      (computed, never stored); a unit past the range's last column is
    //      clamped to the row's last 16 bytes (meets zero weights) ----
    const int a_slot = lane & 7;
    const int a_c[2] = {a_slot ^ ((lane >> 4) & 7), a_slot ^ ((4 + (lane >> 4)) & 7)};
    const int64_t a_row_base = m0 + 32 * wave < M ? m0 + 32 * wave : M - 1;
    const Rsrc a_rsrc = make_rsrc(reinterpret_cast<const uint8_t *>(x) + (a_row_base * lda + k_begin) * 2);
    uint32_t a_voff[kAJ];
#pragma unroll
    for (int j = 0; j < kAJ; ++j) {
        int64_t row = m0 + 32 * wave + 8 * j + (lane >> 3);
        row = row < M ? row : M - 1;
        a_voff[j] = (uint32_t)((row - a_row_base) * lda * 2);
    }
    const uint32_t a_c16[2] = {16u * (uint32_t)a_c[0], 16u * (uint32_t)a_c[1]};
    const uint32_t a_last = (uint32_t)(2 * K - 16);
    auto dma_a = [&](int s, int j0, int j1) {
        uint8_t *dst = sA + (s & 1) * kAStageB + 32 * wave * 128;
        const uint32_t ks = (uint32_t)s * kStage * 2;
#pragma unroll
        for (int j = j0; j < j1; ++j)
            dma16(a_rsrc, a_voff[j] + __builtin_elementwise_min(ks + a_c16[j & 1], a_last), 0, dst + j * 1024);
    };

    // ---- packed blocks: wave w fetches and unpacks blocks 2 w and 2 w + 1 of
    //      the column tile (a block past N: any valid block; its columns are
    //      never stored).  One buffer resource per block. ----
    Rsrc blk_rsrc[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
        const int64_t b = blk0 + 2 * wave + bb;
        blk_rsrc[bb] = make_rsrc(pk + (b < L.nblocks ? b : 0) * L.block_bytes);
    }
    // W4: k-tile t (1 KiB per block, both stages); W8: stage t, the half of
    // k-tile t / 2 that holds its 64 rows (1 KiB per block).  Each wave
    // fetches and reads only its own two blocks' slots.
    auto dma_codes = [&](int t) {
        const uint32_t off = BITS == 4 ? (uint32_t)t * 1024u : (uint32_t)(t >> 1) * 2048u + (uint32_t)(t & 1) * 1024u;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
            dma16(blk_rsrc[bb], 16 * lane, (uint32_t)L.meta_bytes + off, sCodes + (2 * wave + bb) * 1024);
    };
    // group of k-tile t (a multiply-high by a per-launch constant for
    // multi-tile groups: exact while t * tpg < 2^32, else a division)
    const uint32_t tpg_m = 0xFFFFFFFFu / (uint32_t)tpg + 1u;
    const bool tpg_fast = L.G == L.K || (uint64_t)L.ktiles * (uint64_t)tpg < (1ull << 32);
    auto group_of = [&](int t) -> int {
        if constexpr (one_tile)
            return t;
        else if (L.G == L.K || tpg == 1)
            return L.G == L.K ? 0 : t;
        else
            return tpg_fast ? (int)__umulhi((uint32_t)t, tpg_m) : (int)((uint32_t)t / (uint32_t)tpg);
    };
    // record of k-tile t's group, one dword per lane (lanes past the record
    // re-read its first dword), into record buffer t % 2
    const uint32_t rec_lane = 4u * (uint32_t)(lane < RB / 4 ? lane : 0);
    auto dma_rec = [&](int t_src, int t_buf) {
        const uint32_t g = (uint32_t)group_of(t_src);
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
            dma4(blk_rsrc[bb], g * RB + rec_lane, 0, sRec + (t_buf & 1) * kRecBufB + (2 * wave + bb) * kRecBlockB);
    };

    // ---- unpack: B stage sd (k-tile td, half hd) from the lane's code words
    //      (rows 32 u + 8 o .. + 7 of column r, word u of its 16-byte unit)
    //      as exact bf16 q - z, zero where the row is past K or the group's
    //      scale is 0.  Unit (k-octet 4 uu + o, column 32 w + 16 bb + r),
    //      u = 2 hd + uu. ----
    u32x4 cw[2]; // the lane's code units of its two blocks: the k-tile's (W4), the stage's (W8)
    uint8_t *const fill_lane = sB + o * kBOct + (32 * wave + r) * 16;
    auto rec_buf = [&](int t) { return sRec + (t & 1) * kRecBufB; };
    struct UnpackIn {
        uint32_t sb[2], zb[2]; // scale bits, zero byte per block
    };
    // (sd: the stage unpacked; its parity hd is a compile-time constant)
    auto unpack_load = [&](int td, UnpackIn &in) {
        const uint8_t *rb = rec_buf(td);
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            const uint8_t *rec = rb + (2 * wave + bb) * kRecBlockB;
            in.sb[bb] = *reinterpret_cast<const uint16_t *>(rec + 2 * r);
            in.zb[bb] = BITS == 4 ? rec[32 + (r >> 1)] : rec[32 + r];
        }
    };
    auto unpack_store = [&](auto hd_c, int td, const UnpackIn &in, int uu) {
        constexpr int hd = decltype(hd_c)::value;
        const int u = 2 * hd + uu;
        const int step = 4 * td + u;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            const float live = (step < steps && (in.sb[bb] & 0x7FFFu) != 0) ? 1.f : 0.f;
            const uint32_t z = BITS == 4 ? (in.zb[bb] >> (4 * (r & 1))) & 0xFu : in.zb[bb];
            const float nz = -(float)z * live;
            // W4: word u of the k-tile's unit; W8: words 2 uu, 2 uu + 1 of the stage's
            const u32x4 v = BITS == 4 ? unpack_w4<F16>(cw[bb][u], live, nz)
                                      : unpack_w8<F16>(cw[bb][2 * uu], cw[bb][2 * uu + 1], live, nz);
            *reinterpret_cast<u32x4 *>(fill_lane + hd * kBStageB + uu * 4 * kBOct + bb * 256) = v;
        }
    };
    auto read_codes = [&]() {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
            cw[bb] = *reinterpret_cast<const u32x4 *>(sCodes + (2 * wave + bb) * 1024 + 16 * lane);
    };

    // ---- scales of the lane's two accumulator columns: column l32 of the
    //      wave's 32-column tiles j, i.e. column l32 % 16 of block
    //      4 wn + 2 j + l32 / 16 ----
    auto fold_scale_bits = [&](int t, int j) -> uint32_t {
        return *reinterpret_cast<const uint16_t *>(rec_buf(t) + (4 * wn + 2 * j + (l32 >> 4)) * kRecBlockB +
                                                   2 * (l32 & 15));
    };
    float s_last[2], ratio[2] = {1.f, 1.f};

    // ---- the accumulator chain ----
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.f;

    // ---- fragment reads: A unit (row, 2 sl + h32) of the swizzled stage, B
    //      unit (2 sl + h32, column) of the k-octet major stage.  The row
    //      tiles i are 32 rows (4 KiB) apart and the swizzle depends only on
    //      the row's low bits, so one offset per slice serves all four; the
    //      stage buffer and the tiles' offsets are immediates. ----
    int a_rd[4];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
        a_rd[sl] = 16 * swz(128 * wm + l32, 2 * sl + h32);
    const int b_rd = kOffB + h32 * kBOct + (64 * wn + l32) * 16;
    auto read_frags = [&](auto h_c, auto live_c, int sl, u32x4 (&af)[4], u32x4 (&bf)[2]) {
        constexpr int hb = decltype(h_c)::value, LIVE = decltype(live_c)::value;
#pragma unroll
        for (int i = 0; i < LIVE; ++i)
            af[i] = *reinterpret_cast<const u32x4 *>(lds + hb * kAStageB + a_rd[sl] + 4096 * i);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            bf[j] = *reinterpret_cast<const u32x4 *>(lds + b_rd + hb * kBStageB + sl * 2 * kBOct + 512 * j);
    };

    // ---- prologue: k-tile 0's codes (W8: stage 0's) and records and stage
    //      0's activations, then stage 0 unpacked and the chain's first scale
    //      (W8: and stage 1's codes, fetched once this wave has read stage
    //      0's from its slots) ----
    dma_codes(0);
    dma_rec(0, 0);
    dma_a(0, 0, kAJ);
    wait_vmcnt<0>();
    lds_barrier();
    {
        read_codes();
        UnpackIn in;
        unpack_load(0, in);
        unpack_store(ic<0>{}, 0, in, 0);
        unpack_store(ic<0>{}, 0, in, 1);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float sv = half_bits_to_f32<F16>(fold_scale_bits(0, j));
            s_last[j] = sv != 0.f ? sv : 1.f;
        }
    }
    wait_lgkmcnt0();
    if constexpr (BITS == 8) {
        dma_codes(1);
        wait_vmcnt<0>();
    }
    lds_barrier();

    // Fold of group boundary t (between k-tiles t - 1 and t): ratios from
    // the scales of k-tile t's group (ratio exactly 1 where no group starts
    // at t), applied to the row tiles i0 .. i0 + 1 (both columns j).
    auto fold_ratios = [&](int t) {
        const bool starts = t > 0 && t < ktiles && (one_tile || group_of(t) != group_of(t - 1));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float sv = half_bits_to_f32<F16>(fold_scale_bits(t < ktiles ? t : ktiles - 1, j));
            const float se = starts && sv != 0.f ? sv : s_last[j];
            ratio[j] = starts ? s_last[j] * __builtin_amdgcn_rcpf(se) : 1.f;
            s_last[j] = se;
        }
    };
    auto fold_rows = [&](int i0, auto live_c) {
        constexpr int LIVE = decltype(live_c)::value;
#pragma unroll
        for (int i = i0; i < (i0 + 2 < LIVE ? i0 + 2 : LIVE); ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    acc[i][j][e] *= ratio[j];
    };

    // ---- one stage (k-tile t, half h): four 16-row slices.  Loads for later
    //      stages first (the activations of the next stage; at a k-tile's
    //      first stage the next k-tile's codes and records), all waited for
    //      at the stage's end.  The scale fold of the group boundary before
    //      k-tile t + 1 is split in two: row tiles 0 and 1 right after their
    //      last MFMAs of k-tile t (the last slice of its second stage), row
    //      tiles 2 and 3 in the first slice of k-tile t + 1, before their
    //      MFMAs.  Each half overlaps the other tiles' MFMAs.  The next stage
    //      is unpacked in slices 1 and 2 (its codes read in slice 0 when it
    //      starts a new k-tile); within a slice the compiler's own schedule
    //      spreads that VALU work between the MFMAs (measured faster than
    //      forcing an MFMA/VALU pattern).  No step depends on a branch: after
    //      the last stage the loads re-read in-bounds data (clamped) into
    //      buffers no one reads, and the unpack writes the idle B buffer. ----
    auto stage = [&](int t, auto h_c, auto live_c) {
        constexpr int h = decltype(h_c)::value, LIVE = decltype(live_c)::value;
        constexpr int hn = h ^ 1; // parity of the next stage
        const int s = 2 * t + h;
        const int tn = h == 0 ? t : (t + 1 < ktiles ? t + 1 : t); // k-tile of the next stage (clamped)
        const int tc = t + 1 < ktiles ? t + 1 : t;                 // next k-tile's loads (clamped)
        u32x4 af[2][4], bf[2][2];
        read_frags(h_c, live_c, 0, af[0], bf[0]);
        UnpackIn uin;
        static_for<0, 4>([&](auto sl_c) {
            constexpr int sl = decltype(sl_c)::value;
            constexpr int cur = sl & 1;
            if constexpr (sl == 0) {
                if constexpr (BITS == 8 || h == 1)
                    read_codes(); // W4: k-tile t + 1, for its two stages; W8: stage s + 1
                unpack_load(tn, uin);
            }
            if constexpr (sl + 1 < 4)
                read_frags(h_c, live_c, sl + 1, af[cur ^ 1], bf[cur ^ 1]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (sl == 0) {
                dma_a(s + 1, 0, kAJ / 2);
            } else if constexpr (sl == 1) {
                dma_a(s + 1, kAJ / 2, kAJ);
                if constexpr (h == 0) {
                    if constexpr (BITS == 4)
                        dma_codes(tc);
                    dma_rec(tc, t + 1);
                }
                unpack_store(ic<hn>{}, tn, uin, 0);
            } else if constexpr (sl == 2) {
                unpack_store(ic<hn>{}, tn, uin, 1);
                // W8: stage s + 2's codes into this wave's slots, which its
                // unpack above has finished reading (clamped past the end)
                if constexpr (BITS == 8)
                    dma_codes(s + 2 < 2 * ktiles ? s + 2 : 2 * ktiles - 1);
            }
            if constexpr (sl == 0 && h == 0)
                fold_rows(2, live_c); // second half of the fold before k-tile t
#pragma unroll
            for (int i = 0; i < LIVE; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = mfma32x32x16<F16>(af[cur][i], bf[cur][j], acc[i][j]);
            if constexpr (sl == 3 && h == 1) {
                fold_ratios(t + 1); // the boundary before k-tile t + 1
                fold_rows(0, live_c);
            }
        });
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        lds_barrier();
    };
    // Row tiles of the wave below M: a last row tile with fewer than 256
    // rows leaves some waves' 32-row MFMA tiles entirely past M.  Their
    // MFMAs, fragment reads and folds are skipped (their outputs are never
    // stored); the wave still does its share of the loads, unpacking and
    // barriers.  One copy of the k loop per count, chosen once.
    const int64_t wave_rows = M - m0 - 128 * wm;
    const int live = wave_rows >= 128 ? 4 : wave_rows <= 0 ? 0 : (int)((wave_rows + 31) / 32);
    auto k_loop = [&](auto live_c) {
        for (int t = 0; t < ktiles; ++t) {
            stage(t, ic<0>{}, live_c);
            stage(t, ic<1>{}, live_c);
        }
    };
    switch (__builtin_amdgcn_readfirstlane(live)) {
    case 4: k_loop(ic<4>{}); break;
    case 3: k_loop(ic<3>{}); break;
    case 2: k_loop(ic<2>{}); break;
    case 1: k_loop(ic<1>{}); break;
    default: k_loop(ic<0>{}); break;
    }

    // ---- epilogue: y = chain * s_last, fp32 -> bf16 (nearest even).
    //      Element e of a 32x32 accumulator is row 8 (e / 4) + 4 h32 + e % 4,
    //      column l32. ----
    const int64_t n0 = (int64_t)nt * kBN;
    if (splits == 1) {
        // The tile's outputs go through LDS (free after the k loop's last
        // barrier) as [256 rows][TC] 16-bit values, TC = 256 (128 with the
        // SiLU product), and leave in 16-byte units, consecutive lanes on
        // consecutive units of a row: 16 stores per lane instead of 128
        // two-byte ones.  Measured 1-2 % faster on K = 4096, N = 14336 at
        // M = 2048.
        constexpr bool kSilu = ACT == kActSiluMul;
        constexpr int TC = kSilu ? kBN / 2 : kBN;
        uint16_t *const st = reinterpret_cast<uint16_t *>(lds);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int ct = 64 * wn + 32 * j + l32; // column within the tile
            // [gate | up] layout: column c < 8 of a 16-column block is gate,
            // c + 8 (lane l32 ^ 8, same rows) its up column; output column
            // 8 (ct / 16) + c
            const int oc = kSilu ? ((ct >> 4) << 3) + (ct & 7) : ct;
            const bool writer = !kSilu || (ct & 8) == 0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float v = acc[i][j][e] * s_last[j];
                    if constexpr (kSilu) {
                        const float u = __shfl_xor(v, 8);
                        v = v / (1.f + expf(-v)) * u;
                    }
                    const int rt = 128 * wm + 32 * i + 8 * (e >> 2) + 4 * h32 + (e & 3);
                    if (writer)
                        st[rt * TC + oc] = f32_to_half_bits<F16>(v);
                }
        }
        lds_barrier();
        // 16-byte units where y and its rows are 16-byte aligned (every W4
        // layer: N % 8 == 0); otherwise (W8 allows any N) per element, up to
        // the row's last column
        const int64_t out_n = kSilu ? (L.N >> 1) : L.N;
        const int64_t oc0 = kSilu ? n0 / 2 : n0;
        constexpr int UPR = TC / 8; // 16-byte units per tile row
        const bool vec = (reinterpret_cast<uintptr_t>(y) & 15) == 0 && (out_n & 7) == 0;
#pragma unroll 4
        for (int u = tid; u < kBM * UPR; u += kThreads) {
            const int rt = u / UPR, cu = u - rt * UPR;
            const int64_t row = m0 + rt, col = oc0 + 8 * cu;
            if (row >= M || col >= out_n)
                continue;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(st + rt * TC + 8 * cu);
            uint16_t *const dst = y + row * out_n + col;
            if (vec) {
                *reinterpret_cast<u32x4 *>(dst) = v;
            } else {
#pragma unroll
                for (int h = 0; h < 8; ++h)
                    if (col + h < out_n)
                        dst[h] = (uint16_t)(v[h >> 1] >> (16 * (h & 1)));
            }
        }
        return;
    }
    // K split: this range's fp32 partial sums (every column; the SiLU
    // product, if any, is applied by the summing kernel), through a buffer
    // resource based at the wave's first row whose size ends at row M, so
    // rows past M are dropped by the hardware; the lane's column is a fixed
    // offset and each row adds a uniform one (the tile's 128 rows of a wave
    // span at most 128 N elements, below 2^32 bytes while N < 2^22, which the
    // launcher checks).
    const int64_t row0 = m0 + 128 * wm;                    // the wave's first row
    const int64_t rows_left = M - row0 > 0 ? M - row0 : 0; // rows of the wave below M
    uint8_t *const base = reinterpret_cast<uint8_t *>(ws + ((int64_t)split * M + row0) * L.N);
    const uint64_t span = (uint64_t)rows_left * (uint64_t)L.N * 4u;
    const Rsrc out_rsrc = __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)(span < 0xFFFFFFFFull ? span : 0xFFFFFFFFull),
                                                            0x00020000);
    const uint32_t row_bytes = (uint32_t)(L.N * 4);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + 64 * wn + 32 * j + l32;
        if (col >= L.N)
            continue;
        const uint32_t lane_off = (uint32_t)(4 * h32) * row_bytes + (uint32_t)(col * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t roff = (uint32_t)(32 * i + 8 * (e >> 2) + (e & 3)) * row_bytes;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][e] * s_last[j]), out_rsrc,
                                                      (int)(lane_off + roff), 0, 0);
            }
    }
}

template <int BITS, int kMode, int ACT>
static void launch_256(int64_t wgs, int m_tiles, const GemmPlan &plan, hipStream_t stream, const uint16_t *x,
                       const uint8_t *pk, uint16_t *y, const Layout &lay, int64_t M, float *ws)
{
    auto kern = &gemm256_kernel<BITS, kMode, ACT>;
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    (void)attr;
    kern<<<dim3((unsigned)wgs), kThreads, kLds, stream>>>(x, pk, y, lay, M, m_tiles, (int)plan.splits,
                                                         (int)plan.split_tiles, ws);
}

template <int BITS>
static void launch_256_bits(int64_t wgs, int mt, const GemmPlan &plan, hipStream_t stream, const uint16_t *x,
                            const uint8_t *pk, uint16_t *y, const Layout &lay, int64_t M, float *ws, int act)
{
    const bool one = lay.tiles_per_group == 1;
    if (act == kActSiluMul) {
        if (one)
            launch_256<BITS, kGOneTile, kActSiluMul>(wgs, mt, plan, stream, x, pk, y, lay, M, ws);
        else
            launch_256<BITS, kGWhole, kActSiluMul>(wgs, mt, plan, stream, x, pk, y, lay, M, ws);
    } else if (act == kActF16) {
        if (one)
            launch_256<BITS, kGOneTile, kActF16>(wgs, mt, plan, stream, x, pk, y, lay, M, ws);
        else
            launch_256<BITS, kGWhole, kActF16>(wgs, mt, plan, stream, x, pk, y, lay, M, ws);
    } else {
        if (one)
            launch_256<BITS, kGOneTile, kActNone>(wgs, mt, plan, stream, x, pk, y, lay, M, ws);
        else
            launch_256<BITS, kGWhole, kActNone>(wgs, mt, plan, stream, x, pk, y, lay, M, ws);
    }
}

hipError_t launch_gemm256(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M, const Layout &lay,
                          const GemmPlan &plan, float *ws, hipStream_t stream, int act)
{
    // the epilogue's 32-bit offsets: 128 rows of fp32 partials below 2^32 bytes
    if ((bits != 4 && bits != 8) || !lay.whole_tiles() || plan.rows != kBM || plan.col_tile != kBN ||
        plan.narrow_cols != 0 || lay.N >= (int64_t(1) << 22))
        return hipErrorInvalidValue;
    const uint8_t *pk = static_cast<const uint8_t *>(packed);
    const int64_t wgs = plan.m_tiles * plan.wide_cols * plan.splits;
    const int mt = (int)plan.m_tiles;
    if (bits == 4)
        launch_256_bits<4>(wgs, mt, plan, stream, x, pk, y, lay, M, ws, act);
    else
        launch_256_bits<8>(wgs, mt, plan, stream, x, pk, y, lay, M, ws, act);
    return hipSuccess;
}

} // namespace tf
