// Prefill GEMM with fused dequantization (TileFuse summary, Methodology
// section 1: unpack and dequantize each weight tile once, keep the result in
// core-local memory and reuse it for the following matrix operations).
//
// MI355X design.  A workgroup of 8 waves (two per SIMD) owns a 256 x 128
// output tile; each wave a 64 x 64 sub-tile of 2 x 2 bf16 32x32x16 MFMA tiles
// (64 fp32 accumulators per lane, in arch VGPRs).  The 32x32x16 form is used
// because it keeps the matrix core busy for 32 cycles per instruction, long
// enough for the unpack and rescale arithmetic of the same SIMD to issue in
// its shadow; two waves per SIMD let one wave's MFMAs run while the other
// waits.  K advances in stages of 64 rows, each consumed as four 16-row
// slices whose A and B fragments are read from LDS one slice ahead.
//
// Every global load is an LDS-DMA load (global_load_lds_dwordx4 / _dword),
// so nothing is staged through registers and the number of loads a stage
// issues is fixed; the waits are explicit vmcnt values:
//   - activations: a 3-deep ring of [256][64] bf16 stages, two stages ahead;
//   - codes and metadata records: one k-tile (W4) or two stages (W8) ahead.
// The packed codes of a stage are unpacked once into a [128][64] LDS tile as
// the exact bf16 values q - z (|q - z| <= 255 has at most 8 significant
// bits), double buffered, and all 256 rows of the tile reuse them.  All LDS
// tiles use an XOR swizzle of their 16-byte units so that fragment reads and
// writes are free of bank conflicts.
//
// The per-(group, column) scale is folded by ratio, in two accumulator
// chains: even groups accumulate in chain 0, odd groups in chain 1.  A chain
// holds its partial output divided by the scale of its latest group, so when
// the chain moves from group g to group g + 2 it is multiplied by
// s_g / s_{g+2}; the final output is chain_0 * s_0' + chain_1 * s_1' with the
// chains' last scales.  That multiply runs while the other chain's group g + 1
// is being accumulated, spread over its slices, so no fold ever sits between
// two dependent MFMAs.  A zero scale keeps the chain's previous one and its
// group's operands are written as zeros, so its contribution vanishes as it
// should.  Consecutive scales of a chain must keep their ratios and the
// running sums inside the fp32 range (true for any real checkpoint).
//
// Launch plan.  A grid whose 256 x 128 tiles are not a whole number of
// rounds over the compute units would end with a partial round in which the
// other CUs idle.  When the columns of that last round fit one round as
// 256 x 64 tiles, the launcher runs the whole rounds with wide tiles and those
// columns with narrow tiles in a second launch (eight waves of 32 x 64; only
// four of them fetch and unpack weights).  Every output element is still
// computed by one workgroup with the same operations in the same order, so
// the plan does not change a single bit of the result.
#include <atomic>
#include <type_traits>

#include "tf_common.h"
#include "tf_launch.h"
#include "tf_operands.h"
#include "tf_gemm_common.h"

namespace tf {

constexpr int kGBM = 256;                        // rows per workgroup tile
constexpr int kAStages = 3;
constexpr int a_stage_bytes(int bm) { return bm * kStage * 2; } // 32 / 16 KiB
constexpr int kGWaves = 8;                       // waves per workgroup
constexpr int kGThreads = 64 * kGWaves;
constexpr int kMetaWaveBytes = 256;              // record bytes DMA'd per block per k-tile
constexpr int off_b(int bm) { return kAStages * a_stage_bytes(bm); }
// Tile widths: WN = 2 is the 256 x 128 tile (waves 4 x 2, 64 x 64 each), WN =
// 1 the 256 x 64 tile (waves 8 x 1, 32 x 64 each) that fills the last
// partial round of a grid.  Per width: columns, packed blocks, bytes of one
// dequantized B stage and of one buffer of codes.
constexpr int tile_cols(int wn) { return 64 * wn; }
constexpr int tile_blocks(int wn) { return 4 * wn; }
constexpr int bstage_bytes(int wn) { return tile_cols(wn) * kStage * 2; } // 16 / 8 KiB
constexpr int codebuf_bytes(int wn) { return tile_blocks(wn) * 1024; }    // one k-tile (W4) or stage (W8)
constexpr int metabuf_bytes(int wn) { return tile_blocks(wn) * kMetaWaveBytes; }
constexpr int off_codes(int wn, int bm) { return off_b(bm) + 2 * bstage_bytes(wn); }
// code buffers: W4 two k-tiles, W8 three stages (each fetched two stages
// before it is unpacked)
constexpr int code_bufs(int bits) { return bits == 8 ? 3 : 2; }
constexpr int kMetaBufs = 3;                     // records are fetched two k-tiles ahead
constexpr int off_meta(int bits, int wn, int bm) { return off_codes(wn, bm) + code_bufs(bits) * codebuf_bytes(wn); }
constexpr int gemm_lds(int bits, int wn, int bm)
{
    return off_meta(bits, wn, bm) + kMetaBufs * metabuf_bytes(wn); // <= 158 KiB
}
static_assert(gemm_lds(8, 2, kGBM) <= 160 * 1024, "LDS of one CU");

// The workgroup grid covers `splits` ranges of split_tiles k-tiles each, and
// per range m_tiles row tiles x (gridDim.x / splits / m_tiles) column tiles of
// width 64 WN, starting at output column col0.  With one range the output is
// y (bf16); with several, each range writes its fp32 partial sums to
// ws[range][M][N] and a second kernel adds them.
template <int BITS, int kMode, int WN, int BM, int ACT = kActNone>
__global__ __launch_bounds__(kGThreads, 1) void gemm_kernel(const uint16_t *__restrict__ x,
                                                            const uint8_t *__restrict__ packed,
                                                            uint16_t *__restrict__ y, Layout lay, int64_t M,
                                                            int m_tiles, int64_t col0, int splits,
                                                            int split_tiles, float *__restrict__ ws)
{
    constexpr int kGBN = tile_cols(WN), kGBlocks = tile_blocks(WN);
    constexpr bool F16 = ACT == kActF16; // fp16 x, scales and y (else bf16)
    constexpr int kBStageBytes = bstage_bytes(WN), kCodeBufBytes = codebuf_bytes(WN);
    constexpr int kMetaBufBytes = metabuf_bytes(WN);
    constexpr int kBOct = kGBN * 16; // bytes per k-octet row of a dequantized B stage
    // 32-row MFMA tiles per wave (wave rows: 32 MI): a 256-row tile is 4 x 2
    // waves of 64 x 64 (WN = 2) or 8 x 1 of 32 x 64 (WN = 1); a 128-row tile
    // (128 columns only) 4 x 2 waves of 32 x 64
    static_assert(BM == kGBM || (BM == 128 && WN == 2), "row tile");
    constexpr int MI = BM == kGBM ? WN : 1;
    constexpr int kAStageBytes = a_stage_bytes(BM);
    constexpr int kAJ = BM / 64;     // x DMA instructions (8 rows each) per wave and stage
    constexpr int kARows = BM / kGWaves; // rows of a stage each wave fetches
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int RB = record_bytes(BITS);
    constexpr int kSpg = kMode; // slices per group (0: whole k-tiles per group)
    constexpr bool kSplit = kMode == kGSplit32 || kMode == kGSplit64;
    constexpr bool one_tile = kMode == kGOneTile;
    constexpr int kGpt = kSpg ? 8 / kSpg : 1; // groups per k-tile
    // records a k-tile can touch per block (split: up to four 32-row groups)
    constexpr int kRecs = kSplit ? 4 : 1;
    constexpr int kBlockMeta = kRecs * RB; // <= 192 bytes: one dword per lane
    static_assert(kBlockMeta <= kMetaWaveBytes, "a block's records fit one dword DMA");
    constexpr bool kW8 = BITS == 8;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;   // 32 MI-row and 64-column slot of the wave
    const bool unpacker = WN == 2 || wave < kGBlocks; // waves that fetch and unpack a packed block
    const int r = lane & 15, o = lane >> 4;     // fill: column r of the wave's block, k-octet o
    const int l32 = lane & 31, h32 = lane >> 5; // MFMA fragments: row / column l32, k-octet h32

    // ---- tile order: each XCD (workgroups bid % 8) takes a contiguous range
    //      of tiles, enumerated in bands of kBand row tiles: within a band,
    //      consecutive tiles walk its rows first, then the columns, so the
    //      workgroups an XCD runs at once share a few activation panels and
    //      each weight column tile ----
    const int nwg = gridDim.x, bid = blockIdx.x;
    const int xcd = bid & 7, local = bid >> 3, q8 = nwg >> 3, rem = nwg & 7;
    const int tile_all = xcd < rem ? xcd * (q8 + 1) + local : rem * (q8 + 1) + (xcd - rem) * q8 + local;
    const int per_split = nwg / splits;                    // output tiles of one k range
    const int split = tile_all / per_split, tile = tile_all - split * per_split;
    const int n_tiles = per_split / m_tiles;
    const int band_rows = kBand > 0 && kBand < m_tiles ? kBand : m_tiles;
    const int band = tile / (band_rows * n_tiles), in_band = tile - band * band_rows * n_tiles;
    const int rows_here = m_tiles - band * band_rows < band_rows ? m_tiles - band * band_rows : band_rows;
    const int nt = in_band / rows_here, mt = band * band_rows + (in_band - (in_band / rows_here) * rows_here);
    const int64_t m0 = (int64_t)mt * BM;
    const int64_t blk0 = (col0 >> 4) + (int64_t)nt * kGBlocks;

    // ---- the k range of this split as a layout of its own: its groups,
    //      k-tiles and rows, with the packed block base moved to its first
    //      record and the codes' offset moved to its first k-tile.  Ranges
    //      start on group boundaries (a whole-k-tile group per range when one
    //      group spans all of K). ----
    const int64_t lda = lay.K; // elements per row of x
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
    const uint8_t *const pk = packed + g_begin * RB; // a block's records of this range

    const int ktiles = (int)L.ktiles;
    const int nstages = 2 * ktiles;
    const int steps = (int)L.steps;
    const int64_t K = L.K;

    uint8_t *const sA = lds;
    uint8_t *const sB = lds + off_b(BM);
    uint8_t *const sCodes = lds + off_codes(WN, BM);
    uint8_t *const sMeta = lds + off_meta(BITS, WN, BM);

    // ---- activations.  Wave w fills rows R w .. R w + R - 1 of a stage (R =
    //      BM / 8), 8 rows per instruction j; lane p takes row 8j + p/8 and the
    //      16-byte unit c that the swizzle places at slot p%8 (R w is a
    //      multiple of 16, so the swizzle of those rows repeats every two j).
    //      The address is a wave-uniform base (row R w of the tile, clamped at
    //      M - 1, plus the stage's k) and a 32-bit lane offset; rows past M
    //      read row M - 1 (computed, never stored). ----
    const int a_slot = lane & 7;
    const int a_c[2] = {a_slot ^ ((lane >> 4) & 7), a_slot ^ ((4 + (lane >> 4)) & 7)}; // unit for even / odd j
    const int64_t a_row_base = m0 + kARows * wave < M ? m0 + kARows * wave : M - 1;
    const Rsrc a_rsrc = make_rsrc(reinterpret_cast<const uint8_t *>(x) + (a_row_base * lda + k_begin) * 2);
    uint32_t a_voff[kAJ];
#pragma unroll
    for (int j = 0; j < kAJ; ++j) {
        int64_t row = m0 + kARows * wave + 8 * j + (lane >> 3);
        row = row < M ? row : M - 1;
        a_voff[j] = (uint32_t)((row - a_row_base) * lda * 2);
    }
    // The lane's unit of stage s starts s * 128 + 16 c bytes into the row
    // (c its swizzled unit); a unit that would end past the range's last
    // column (a last stage that runs past K, or a range shorter than a
    // stage) is clamped to the row's last 16 bytes and re-reads its last 8
    // columns (finite values that meet zero weights).  The clamp is on the
    // whole offset, so it holds for every K >= 32 (a row of 64 bytes).
    const uint32_t a_c16[2] = {16u * (uint32_t)a_c[0], 16u * (uint32_t)a_c[1]};
    const uint32_t a_last = (uint32_t)(2 * K - 16);
    // instructions j0 .. j1 - 1 of the kAJ that fill the wave's rows of stage s
    auto dma_a = [&](int s, int j0, int j1) {
        uint8_t *dst = sA + (s % kAStages) * kAStageBytes + kARows * wave * 128;
        const uint32_t ks = (uint32_t)s * kStage * 2;
#pragma unroll
        for (int j = j0; j < j1; ++j)
            dma16(a_rsrc, a_voff[j] + __builtin_elementwise_min(ks + a_c16[j & 1], a_last), 0, dst + j * 1024);
    };
    // ---- codes: wave w < kGBlocks fetches block w (1 KiB per k-tile; W8:
    //      per half).  Only these waves fetch codes and records and unpack;
    //      the others (the 64-column tile's waves 4 .. 7) load x only. ----
    const int64_t my_blk = blk0 + wave < L.nblocks ? blk0 + wave : 0; // blocks past N: any valid block
    // one resource per block: a block (records and codes) is below 2^30 bytes
    const Rsrc blk_rsrc = make_rsrc(pk + my_blk * L.block_bytes);
    auto dma_codes = [&](int t, int half, int buf) {
        const uint32_t soff = (uint32_t)L.meta_bytes + (uint32_t)t * tile_bytes(BITS) + 1024u * half;
        dma16(blk_rsrc, 16 * lane, soff, sCodes + buf * kCodeBufBytes + wave * 1024);
    };
    // ---- records of k-tile t for block w, as dwords, into the buffer of
    //      k-tile tb (tb % 3); lanes past the records, or past the last
    //      group, read a dword of the block's first record instead ----
    // (no division in the loop: G = 32 or 64 gives kGpt groups per k-tile;
    // whole-k-tile groups are t / (k-tiles per group), a multiply-high by a
    // per-launch constant, exact while t * tpg < 2^32, else a division; one
    // group over all of K is group 0)
    const uint32_t tpg = (uint32_t)(L.G == L.K ? 1 : L.G / kTileRows);
    const bool tpg_fast = L.G == L.K || (uint64_t)L.ktiles * tpg < (1ull << 32);
    const uint32_t tpg_m = 0xFFFFFFFFu / tpg + 1u; // unused when tpg == 1
    auto first_group = [&](int t) -> int64_t {
        if constexpr (one_tile)
            return t;
        else if constexpr (kSplit)
            return (int64_t)t * kGpt;
        else if (L.G == L.K)
            return 0;
        else
            return tpg_fast ? (int64_t)__umulhi((uint32_t)t, tpg_m) : (int64_t)((uint32_t)t / tpg);
    };
    // (32-bit: a block's records are below 2^26 bytes; lanes past kBlockMeta
    // re-read the first record's first dword)
    const int m_lane = lane < kBlockMeta / 4 ? lane : 0;
    const int m_grp = (4 * m_lane) / RB;
    const int ngroups32 = (int)L.ngroups;
    auto dma_meta = [&](int t, int tb) {
        const int g_first = (int)first_group(t);
        const uint32_t v = g_first + m_grp < ngroups32 ? (uint32_t)(g_first * RB + 4 * m_lane) : 0u;
        dma4(blk_rsrc, v, 0, sMeta + (tb % kMetaBufs) * kMetaBufBytes + wave * kMetaWaveBytes);
    };
    // the staged record of block bb (0..7) for group g, which k-tile t touches
    auto meta_rec = [&](int bb, int t, int64_t g) -> const uint8_t * {
        const uint8_t *rec = sMeta + (t % kMetaBufs) * kMetaBufBytes + bb * kMetaWaveBytes;
        return one_tile ? rec : rec + (int)(g - first_group(t)) * RB;
    };
    auto code_buf = [&](int s) { return kW8 ? s % 3 : (s >> 1) & 1; };
    // group of 32-row step `step`
    auto group_of_step = [&](int step) -> int64_t {
        if constexpr (one_tile)
            return step >> 2;
        else if constexpr (kSplit)
            return kMode == kGSplit32 ? step : step >> 1; // G = 32 or 64: one or two steps per group
        else
            return first_group(step >> 2);
    };

    // ---- unpack stage sd into B buffer sd % 2 as exact bf16 (q - z), zero
    //      where the row is past K or the group's scale is 0.  Columns past N
    //      need no care: their outputs are never stored.  Wave w unpacks block
    //      w; lane (o, r) column r, rows 32 kk + 8 o .. +7.  A B buffer is
    //      k-octet major ([8][128] units of 16 bytes), so fragment reads and
    //      these writes touch 256 contiguous bytes per 16 lanes and every
    //      offset but the lane's own is an immediate. ----
    struct FillIn {
        u32x2 cw;       // the lane's code words for this stage (W8: 4 words in cw, cw8)
        u32x2 cw8;
        uint32_t sb[2]; // scale bits per 32-row step
        uint32_t zb[2]; // byte holding the zero point per 32-row step
    };
    // Raw loads only: the values are decoded where they are used, so that the
    // loads can issue well before (the LDS counter is waited for in order).
    auto scale_bits = [&](const uint8_t *rec) -> uint32_t { return *reinterpret_cast<const uint16_t *>(rec + 2 * r); };
    auto zero_byte = [&](const uint8_t *rec) -> uint32_t { return rec[32 + (BITS == 4 ? (r >> 1) : r)]; };
    auto zero_of = [&](uint32_t zb) -> uint32_t { return BITS == 4 ? (zb >> (4 * (r & 1))) & 0xFu : zb; };
    const uint8_t *const code_lane = sCodes + wave * 1024 + 16 * lane;
    auto fill_load = [&](int sd, FillIn &in) {
        const int td = sd >> 1, hd = sd & 1;
        const uint8_t *codes = code_lane + code_buf(sd) * kCodeBufBytes;
        if constexpr (kW8) {
            const u32x4 c4 = *reinterpret_cast<const u32x4 *>(codes);
            in.cw = u32x2{c4[0], c4[1]};
            in.cw8 = u32x2{c4[2], c4[3]};
        } else {
            in.cw = *reinterpret_cast<const u32x2 *>(codes + 8 * hd);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int step = 4 * td + 2 * hd + kk;
            const uint8_t *rec = meta_rec(wave, td, group_of_step(step));
            in.sb[kk] = scale_bits(rec);
            in.zb[kk] = zero_byte(rec);
        }
    };
    uint8_t *const fill_lane = sB + o * kBOct + (16 * wave + r) * 16;
    // 32-row step kk (0, 1) of stage sd
    auto fill_store = [&](int sd, const FillIn &in, auto kk_c) {
        constexpr int kk = decltype(kk_c)::value;
        const int step = 4 * (sd >> 1) + 2 * (sd & 1) + kk;
        // (q - z) * live as fma(q, live, -z * live): the mask costs nothing
        const float live = (step < steps && (in.sb[kk] & 0x7FFFu) != 0) ? 1.f : 0.f;
        const float nz = -(float)zero_of(in.zb[kk]) * live;
        u32x4 v;
        if constexpr (kW8)
            v = kk == 0 ? unpack_w8<F16>(in.cw[0], in.cw[1], live, nz)
                        : unpack_w8<F16>(in.cw8[0], in.cw8[1], live, nz);
        else
            v = unpack_w4<F16>(in.cw[kk], live, nz);
        *reinterpret_cast<u32x4 *>(fill_lane + (sd & 1) * kBStageBytes + kk * 4 * kBOct) = v;
    };

    // ---- scales of the lane's two columns: column l32 of the 32-column tiles
    //      j = 0, 1 of the wave, i.e. column r of block 4 wn + 2 j + l32 / 16;
    //      groups past K (slices after the last row) read as 0 ----
    auto scales_of = [&](int64_t g, int t, float (&sc)[2]) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float v = record_scale<BITS, F16>(meta_rec(4 * wn + 2 * j + (l32 >> 4), t, g), r);
            sc[j] = g < L.ngroups ? v : 0.f;
        }
    };
    // the same, split into the raw loads and their decoding
    auto scales_load = [&](int64_t g, int t, uint32_t (&sb)[2]) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            sb[j] = scale_bits(meta_rec(4 * wn + 2 * j + (l32 >> 4), t, g));
    };
    auto scales_decode = [&](int64_t g, const uint32_t (&sb)[2], float (&sc)[2]) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            sc[j] = g < L.ngroups ? half_bits_to_f32<F16>(sb[j]) : 0.f;
    };

    // ---- accumulator chains (even / odd groups) and their current scales ----
    f32x16 acc[2][MI][2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    acc[c][i][j][e] = 0.f;
    float s_last[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
    float ratio[2] = {1.f, 1.f}; // of the chain being folded
    // chain C moves on to group g when `ok`: ratio s_last / s_g (a zero
    // scale keeps s_last); otherwise the ratio is exactly 1.  The records are
    // read either way (in bounds), so there is no branch.
    auto start_fold_with = [&](auto c_c, const float (&sn)[2], bool ok) {
        constexpr int C = decltype(c_c)::value;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float se = ok && sn[j] != 0.f ? sn[j] : s_last[C][j];
            const float rt = s_last[C][j] * __builtin_amdgcn_rcpf(se);
            ratio[j] = ok ? rt : 1.f;
            s_last[C][j] = se;
        }
    };
    auto start_fold = [&](auto c_c, int64_t g, int t, bool ok) {
        float sn[2];
        scales_of(g, t, sn);
        start_fold_with(c_c, sn, ok);
    };
    // first group of chain C: its own scale (1 if zero: the chain stays 0)
    auto start_chain = [&](auto c_c, int64_t g, int t) {
        constexpr int C = decltype(c_c)::value;
        float sn[2];
        scales_of(g, t, sn);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            s_last[C][j] = sn[j] != 0.f ? sn[j] : 1.f;
    };
    // chunk CH of NC of chain C times the ratio (element f = 16 (2 i + j) + e)
    auto fold_chunk = [&](auto c_c, auto ch_c, auto nc_c) {
        constexpr int C = decltype(c_c)::value, CH = decltype(ch_c)::value, NC = decltype(nc_c)::value;
        constexpr int NE = 32 * MI; // accumulator elements per lane and chain
#pragma unroll
        for (int f = CH * NE / NC; f < (CH + 1) * NE / NC; ++f) {
            const int i = f >> 5, j = (f >> 4) & 1, e = f & 15;
            acc[C][i][j][e] *= ratio[j];
        }
    };

    // ---- fragment reads.  A: the swizzled unit (row, 2 sl + h32) of the
    //      lane's row in sub-tile i, one offset per (slice, i) precomputed;
    //      B: unit (2 sl + h32, column) of the k-octet major buffer. ----
    int a_rd[4][MI];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
#pragma unroll
        for (int i = 0; i < MI; ++i)
            a_rd[sl][i] = 16 * swz(32 * MI * wm + 32 * i + l32, 2 * sl + h32);
    const uint8_t *b_rd[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
        b_rd[j] = sB + h32 * kBOct + (64 * wn + 32 * j + l32) * 16;
    auto read_frags = [&](const uint8_t *a_st, int hb, int sl, u32x4 (&af)[MI], u32x4 (&bf)[2]) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
            af[i] = *reinterpret_cast<const u32x4 *>(a_st + a_rd[sl][i]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            bf[j] = *reinterpret_cast<const u32x4 *>(b_rd[j] + hb * kBStageBytes + sl * 2 * kBOct);
    };

    // ---- prologue.  What stage 0 and the loop's first unpack need (records
    //      of k-tiles 0 and 1, codes of k-tile 0, x of stage 0) is waited for
    //      here; x of stage 1 and the next codes are waited for at the end of
    //      stage 0, like every load the loop issues (nstages >= 2). ----
    if (unpacker) {
        dma_meta(0, 0);
        dma_meta(ktiles > 1 ? 1 : 0, 1);
        dma_codes(0, 0, 0);
        if (kW8)
            dma_codes(0, 1, 1);
    }
    dma_a(0, 0, kAJ);
    dma_a(1, 0, kAJ);
    if (unpacker) {
        if (kW8)
            dma_codes(ktiles > 1 ? 1 : 0, ktiles > 1 ? 0 : 1, 2); // stage 2
        else
            dma_codes(ktiles > 1 ? 1 : 0, 0, 1);
        wait_vmcnt<kAJ + 1>();
    } else {
        wait_vmcnt<kAJ>();
    }
    lds_barrier();
    if (unpacker) {
        FillIn f0;
        fill_load(0, f0);
        fill_store(0, f0, ic<0>{});
        fill_store(0, f0, ic<1>{});
    }
    // the chains' first groups: 0 and 1 (one-tile groups: k-tiles 0 and 1)
    start_chain(ic<0>{}, 0, 0);
    if constexpr (kMode != kGWhole)
        start_chain(ic<1>{}, 1, one_tile ? 1 : 0);
    wait_lgkmcnt0();
    lds_barrier();

    // ---- one k-tile (two stages of four slices).  PAR is the chain of
    //      one-tile groups (group t is chain t % 2). ----
    auto ktile = [&](int t, auto par_c) {
        constexpr int PAR = decltype(par_c)::value;
        static_for<0, 2>([&](auto h_c) {
            constexpr int h = decltype(h_c)::value;
            const int s = 2 * t + h;
            // ---- loads for later stages, each waited for at the end of the
            //      next stage: x two stages ahead, then codes (W4: k-tile
            //      t + 2 into the buffer of k-tile t, which stage 2t + 1 no
            //      longer reads; W8: stage s + 3 into the buffer of stage s)
            //      and records (k-tile t + 2 into the buffer of k-tile t - 1).
            //      Past the end they re-read the last stage into buffers
            //      nobody reads, so every stage issues the same loads.  They
            //      and the unpack of the next stage are spread over the four
            //      slices so that they issue between MFMAs. ----
            const int sa = s + 2 < nstages ? s + 2 : nstages - 1;
            const int t2 = t + 2 < ktiles ? t + 2 : ktiles - 1;
            const uint8_t *a_st = sA + (s % kAStages) * kAStageBytes;
            u32x4 af[2][MI], bf[2][2]; // fragments of two slices in flight
            FillIn fin;               // the next stage's codes and records
            read_frags(a_st, h, 0, af[0], bf[0]);

            static_for<0, 4>([&](auto sl_c) {
                constexpr int sl = decltype(sl_c)::value;
                constexpr int cur = sl & 1;
                constexpr int sig = 4 * h + sl; // slice within the k-tile
                // ---- LDS reads first, small ones before the fragments, then
                //      a scheduling fence: the compiler may not sink them to
                //      their uses, so the next slice's fragments load while
                //      this slice's MFMAs run, and waiting for the small
                //      reads never waits for the fragments ----
                constexpr int spg = kSpg ? kSpg : 8;          // (whole k-tiles: unused)
                constexpr int pos = sig % spg;                // slice within its group
                constexpr int gin = sig / spg;                // group within the k-tile
                constexpr bool fold_start = kMode != kGWhole && pos == 0;
                uint32_t fold_sb[2];
                int64_t fold_g = 0;
                if constexpr (fold_start) {
                    // chain F (group g - 1) moves on to group g + 1, whose
                    // records sit in this k-tile or the next one
                    constexpr int tn_off = (gin + 1) / kGpt; // 0 or 1
                    fold_g = first_group(t) + gin + 1;
                    scales_load(fold_g, t + tn_off, fold_sb);
                }
                if constexpr (sl == 1) {
                    if (unpacker)
                        fill_load(s + 1, fin);
                }
                if constexpr (sl + 1 < 4)
                    read_frags(a_st, h, sl + 1, af[cur ^ 1], bf[cur ^ 1]);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (sl == 0) {
                    dma_a(sa, 0, kAJ / 2);
                } else if constexpr (sl == 1) {
                    dma_a(sa, kAJ / 2, kAJ);
                } else if constexpr (sl == 2) {
                    if (unpacker) {
                        if constexpr (kW8) {
                            const int sc = s + 3 < nstages ? s + 3 : nstages - 1;
                            dma_codes(sc >> 1, sc & 1, s % 3);
                        } else if constexpr (h == 1) {
                            dma_codes(t2, 0, t & 1);
                        }
                        if constexpr (h == 0)
                            dma_meta(t2, t + 2);
                        fill_store(s + 1, fin, ic<0>{});
                    }
                } else {
                    if (unpacker)
                        fill_store(s + 1, fin, ic<1>{});
                }
                if constexpr (kMode == kGWhole) {
                    // groups of whole k-tiles: chain 0 only, folded at the end
                    // of each group (the next group's records are staged)
#pragma unroll
                    for (int i = 0; i < MI; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc[0][i][j] = mfma32x32x16<F16>(af[cur][i], bf[cur][j], acc[0][i][j]);
                    if (sig == 7 && (t + 1) % (int)L.tiles_per_group == 0 && t + 1 < ktiles) {
                        start_fold(ic<0>{}, (int64_t)(t + 1) / L.tiles_per_group, t + 1, true);
                        fold_chunk(ic<0>{}, ic<0>{}, ic<1>{});
                    }
                } else {
                    constexpr int C = one_tile ? PAR : (gin & 1); // chain of this group
                    constexpr int F = C ^ 1;                      // chain folded meanwhile
                    if constexpr (fold_start) {
                        float sn[2];
                        scales_decode(fold_g, fold_sb, sn);
                        start_fold_with(ic<F>{}, sn, fold_g >= 2 && fold_g < L.ngroups);
                    }
#pragma unroll
                    for (int i = 0; i < MI; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc[C][i][j] = mfma32x32x16<F16>(af[cur][i], bf[cur][j], acc[C][i][j]);
                    fold_chunk(ic<F>{}, ic<pos>{}, ic<kSpg>{});
                }
            });

            // ---- everything issued before this stage has landed (stage
            //      s + 1's x, the next codes and records); only this stage's
            //      loads may still be in flight (x: kAJ, codes and records: 1
            //      or 2 on the unpacking waves) ----
            if (!unpacker)
                wait_vmcnt<kAJ>();
            else if constexpr (kW8 && h == 0)
                wait_vmcnt<kAJ + 2>();
            else
                wait_vmcnt<kAJ + 1>();
            wait_lgkmcnt0();
            lds_barrier();
        });
    };

    if constexpr (one_tile) {
        int t = 0;
        for (; t + 1 < ktiles; t += 2) {
            ktile(t, ic<0>{});
            ktile(t + 1, ic<1>{});
        }
        if (t < ktiles)
            ktile(t, ic<0>{});
    } else {
        for (int t = 0; t < ktiles; ++t)
            ktile(t, ic<0>{});
    }
    wait_vmcnt<0>();

    // ---- epilogue: y = chain_0 * s_0' + chain_1 * s_1', fp32 -> bf16
    //      (nearest even).  Element e of a 32x32 accumulator is row
    //      8 (e / 4) + 4 h32 + e % 4, column l32. ----
    const int64_t n0 = col0 + (int64_t)nt * kGBN;
    if (splits == 1) {
        // The tile's outputs go through LDS as [BM rows][TC] 16-bit values
        // (TC = the tile's columns, half of them with the SiLU product) and
        // leave in 16-byte units, consecutive lanes on consecutive units of a
        // row, where y and its rows are 16-byte aligned; otherwise per
        // element from the same units.  (Per-element two-byte stores wrote
        // about 1.4 times the output's bytes to HBM.)
        constexpr bool kSilu = ACT == kActSiluMul;
        constexpr int TC = kSilu ? kGBN / 2 : kGBN;
        static_assert(BM * TC * 2 <= off_codes(WN, BM), "the output tile fits the A and B stages");
        uint16_t *const st = reinterpret_cast<uint16_t *>(lds);
        lds_barrier(); // every wave is done with the k loop's LDS
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int ct = 64 * wn + 32 * j + l32; // column within the tile
            // [gate | up] packed by tf_repack_*_gate_up (N % 16 == 0):
            // column c < 8 of a 16-column block is gate, c + 8 (lane l32 ^ 8,
            // same rows) the matching up column; output column 8 (ct / 16) + c
            const int oc = kSilu ? ((ct >> 4) << 3) + (ct & 7) : ct;
            const bool writer = !kSilu || (ct & 8) == 0;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float v = kMode == kGWhole ? acc[0][i][j][e] * s_last[0][j]
                                               : fmaf(acc[0][i][j][e], s_last[0][j], acc[1][i][j][e] * s_last[1][j]);
                    if constexpr (kSilu) {
                        // SiLU as in the GEMV epilogue: v / (1 + e^-v), -0
                        // where e^-v overflows
                        const float u = __shfl_xor(v, 8);
                        v = v / (1.f + expf(-v)) * u;
                    }
                    const int rt = 32 * MI * wm + 32 * i + 8 * (e >> 2) + 4 * h32 + (e & 3);
                    if (writer)
                        st[rt * TC + oc] = f32_to_half_bits<F16>(v);
                }
        }
        lds_barrier();
        const int64_t out_n = kSilu ? (L.N >> 1) : L.N;
        const int64_t oc0 = kSilu ? n0 / 2 : n0;
        constexpr int UPR = TC / 8; // 16-byte units per tile row
        const bool vec = (reinterpret_cast<uintptr_t>(y) & 15) == 0 && (out_n & 7) == 0;
#pragma unroll 4
        for (int u = tid; u < BM * UPR; u += kGThreads) {
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
    // K split: this range's fp32 partial sums, every column (the SiLU
    // product, if any, is applied by the summing kernel)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + 64 * wn + 32 * j + l32;
        if (col >= L.N)
            continue;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + 32 * MI * wm + 32 * i + 8 * (e >> 2) + 4 * h32 + (e & 3);
                const float v = kMode == kGWhole ? acc[0][i][j][e] * s_last[0][j]
                                                 : fmaf(acc[0][i][j][e], s_last[0][j], acc[1][i][j][e] * s_last[1][j]);
                if (row < M)
                    __builtin_nontemporal_store(v, ws + ((int64_t)split * M + row) * L.N + col);
            }
    }
}

// The kernel needs more than the default 64 KiB of dynamic LDS; raise the
// limit once per instantiation.
template <int BITS, int kMode, int WN, int BM, int ACT>
static void launch_mode(int64_t wgs, int m_tiles, int64_t col0, const GemmPlan &plan, hipStream_t stream,
                        const uint16_t *x, const uint8_t *pk, uint16_t *y, const Layout &lay, int64_t M, float *ws)
{
    auto kern = &gemm_kernel<BITS, kMode, WN, BM, ACT>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       gemm_lds(BITS, WN, BM));
    (void)attr;
    kern<<<dim3((unsigned)wgs), kGThreads, gemm_lds(BITS, WN, BM), stream>>>(
        x, pk, y, lay, M, m_tiles, col0, (int)plan.splits, (int)plan.split_tiles, ws);
}

// y = bf16 (fp16 when F16) of the sum over s of ws[s] for the M x N outputs,
// in split order.  The
// split count is a template parameter so that a thread issues all S loads
// at once (one round trip) and then adds them in order.  The partials were
// stored non-temporally on other XCDs and are read the same way.
template <int S, bool F16>
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float *__restrict__ ws, int64_t mn,
                                                         uint16_t *__restrict__ y)
{
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= mn)
        return;
    if (i + 4 <= mn) {
        f32x4 p[S];
#pragma unroll
        for (int s = 0; s < S; ++s)
            p[s] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(ws + s * mn + i));
        f32x4 v = p[0];
#pragma unroll
        for (int s = 1; s < S; ++s)
            v = v + p[s];
        u32x2 o;
        o[0] = pack_half_x2<F16>(v[0], v[1]);
        o[1] = pack_half_x2<F16>(v[2], v[3]);
        *reinterpret_cast<u32x2 *>(y + i) = o;
    } else {
        for (int64_t e = i; e < mn; ++e) {
            float v = ws[e];
#pragma unroll
            for (int s = 1; s < S; ++s)
                v += ws[s * mn + e];
            y[e] = f32_to_half_bits<F16>(v);
        }
    }
}

template <int S> static void launch_sum(const float *ws, int64_t mn, uint16_t *y, hipStream_t stream, bool f16)
{
    const int64_t grid = (mn + 4 * 256 - 1) / (4 * 256);
    if (f16)
        splitk_sum_kernel<S, true><<<dim3((unsigned)grid), 256, 0, stream>>>(ws, mn, y);
    else
        splitk_sum_kernel<S, false><<<dim3((unsigned)grid), 256, 0, stream>>>(ws, mn, y);
}

void launch_splitk_sum(const float *ws, int splits, int64_t mn, uint16_t *y, hipStream_t stream, bool f16)
{
    switch (splits) {
    case 2: launch_sum<2>(ws, mn, y, stream, f16); break;
    case 3: launch_sum<3>(ws, mn, y, stream, f16); break;
    case 4: launch_sum<4>(ws, mn, y, stream, f16); break;
    case 5: launch_sum<5>(ws, mn, y, stream, f16); break;
    case 6: launch_sum<6>(ws, mn, y, stream, f16); break;
    case 7: launch_sum<7>(ws, mn, y, stream, f16); break;
    case 8: launch_sum<8>(ws, mn, y, stream, f16); break;
    case 9: launch_sum<9>(ws, mn, y, stream, f16); break;
    case 10: launch_sum<10>(ws, mn, y, stream, f16); break;
    case 11: launch_sum<11>(ws, mn, y, stream, f16); break;
    case 12: launch_sum<12>(ws, mn, y, stream, f16); break;
    case 13: launch_sum<13>(ws, mn, y, stream, f16); break;
    case 14: launch_sum<14>(ws, mn, y, stream, f16); break;
    case 15: launch_sum<15>(ws, mn, y, stream, f16); break;
    default: launch_sum<16>(ws, mn, y, stream, f16); break;
    }
}

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_cus[kMaxDevices];
} // namespace

// compute units of the current device, queried once per device (the value
// never changes, so concurrent first queries store the same number)
int device_cus()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 256;
    int n = g_device_cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        g_device_cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

bool gemm_uses_gemv(int64_t M, int route)
{
    return M <= kGemvKernelMaxM && route != kRouteTiled && route != kRouteTiled128;
}

// K split for a grid of `tiles` output tiles that fills less than half the
// compute units: 2 to 8 ranges of at least 4 k-tiles, each starting on a
// group boundary, so that the chip fills; each range writes fp32 partial
// sums that a second kernel adds in range order.  Returns false (no split)
// when no split of at least two ranges fits those rules.
static bool plan_split(GemmPlan &p, int64_t tiles, int64_t K, int64_t G, int cus)
{
    const int64_t ktiles = (K + kTileRows - 1) / kTileRows;
    if (2 * tiles > cus || ktiles < 8)
        return false;
    const int64_t unit = (G % kTileRows == 0 && G != K) ? G / kTileRows : 1; // k-tiles per boundary step
    int64_t s = cus / tiles;
    s = s < 8 ? s : 8;
    s = s < ktiles / 4 ? s : ktiles / 4;
    if (s < 2)
        return false;
    int64_t st = (ktiles + s - 1) / s;
    st = (st + unit - 1) / unit * unit;
    s = (ktiles + st - 1) / st;
    if (s < 2)
        return false;
    p.splits = s;
    p.split_tiles = st;
    return true;
}

GemmPlan plan_gemm(int bits, int64_t M, int64_t N, int64_t K, int64_t G, int cus, int route)
{
    const bool allow256 = route != kRouteTiled128;
    GemmPlan p;
    const int64_t ktiles = (K + kTileRows - 1) / kTileRows;
    p.splits = 1;
    p.split_tiles = ktiles;
    p.narrow_cols = 0;
    // Groups of whole k-tiles above 128 rows: 256 x 256 tiles (their
    // epilogue's 32-bit offsets hold rows of fewer than 2^22 columns)
    const bool whole = G % kTileRows == 0 || G == K;
    if (allow256 && whole && M > kShortTileMaxM && N < (int64_t(1) << 22)) {
        p.rows = kGBM;
        p.col_tile = 256;
        p.m_tiles = (M + kGBM - 1) / kGBM;
        p.wide_cols = (N + 255) / 256;
        plan_split(p, p.m_tiles * p.wide_cols, K, G, cus);
        // The automatic choice drops these tiles only where K had to be
        // split and the split launch still fills less than 85 % of the
        // compute units: the split is capped at 8 ranges (often of only a few
        // k-tiles each), and twice as many 256 x 128 tiles fill the chip
        // better.  On the decoder layer's q/k/v, o and down projections at
        // M = 129-256 they took 28-46 us against 30-56.  Without a split a
        // partial round of these tiles still beats the 256 x 128 tiles' one
        // and a half (q/k/v at M = 2048).  A split into ranges of fewer than
        // 8 k-tiles also drops them (each range's fixed costs outweigh the
        // wider tile): the layer's o projection (4096 x 4096) took 30-43 us
        // on 256 x 128 tiles against 33-49 at M = 300-768, and the layer pass
        // at M = 512 went from 270 to 258 us (at M = 300 from 208 to 212).
        // W8 keeps them only without a split: W8 per channel at M = 512,
        // K = N = 8192 took 84 us as 64 tiles x 4 K ranges against 79 as 128
        // tiles of 256 x 128 x 2 ranges, while W8 at M = 2048, K = 4096,
        // N = 14336, G = 128 took 240 us against 273.  The test route
        // kRouteTiled keeps these tiles wherever they apply.
        if (route == kRouteTiled || p.splits == 1 ||
            (bits == 4 && p.split_tiles >= 8 && p.m_tiles * p.wide_cols * p.splits * 20 >= 17 * (int64_t)cus))
            return p;
        p = GemmPlan{};
        p.splits = 1;
        p.split_tiles = ktiles;
        p.narrow_cols = 0;
    }
    // up to 128 rows, 128-row tiles: a 256-row tile would compute at least
    // as many padding rows as real ones
    p.col_tile = tile_cols(2);
    p.rows = M <= kShortTileMaxM ? kShortTileRows : kGBM;
    p.m_tiles = (M + p.rows - 1) / p.rows;
    const int64_t n_wide = (N + tile_cols(2) - 1) / tile_cols(2);
    const int64_t tiles = p.m_tiles * n_wide;
    p.wide_cols = n_wide; // default: one launch of 128-column tiles over all of K
    if (plan_split(p, tiles, K, G, cus))
        return p;
    if (tiles % cus == 0 || p.rows != kGBM)
        return p;
    // the whole rounds with 128-column tiles, the columns left over as
    // 64-column tiles when they fit one round (a last partial round of wide
    // tiles would otherwise leave CUs idle while it runs)
    const int64_t full = (tiles / cus) * cus;
    const int64_t wide = full / p.m_tiles < n_wide ? full / p.m_tiles : n_wide;
    const int64_t rest = N - wide * tile_cols(2);
    const int64_t narrow = (rest + tile_cols(1) - 1) / tile_cols(1);
    if (rest > 0 && p.m_tiles * narrow <= cus) {
        p.wide_cols = wide;
        p.narrow_cols = narrow;
    }
    return p;
}

int64_t gemm_workspace_bytes(int bits, int64_t M, int64_t N, int64_t K, int64_t G, int cus, int route)
{
    const GemmPlan p = plan_gemm(bits, M, N, K, G, cus, route);
    return p.splits > 1 ? p.splits * M * N * (int64_t)sizeof(float) : 0;
}

hipError_t launch_gemm(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M, const Layout &lay,
                       void *workspace, hipStream_t stream, int cus, int act, int route)
{
    if (act == kActSiluMul && lay.N % kBlockCols)
        return hipErrorInvalidValue;
    const GemmPlan plan = plan_gemm(bits, M, lay.N, lay.K, lay.G, cus, route);
    float *ws = plan.splits > 1 ? static_cast<float *>(workspace) : nullptr;
    if (plan.col_tile == 256) {
        if (hipError_t e = launch_gemm256(bits, x, packed, y, M, lay, plan, ws, stream, act))
            return e;
        if (plan.splits > 1) {
            if (act == kActSiluMul)
                launch_splitk_sum_silu(ws, (int)plan.splits, M, lay.N, y, stream);
            else
                launch_splitk_sum(ws, (int)plan.splits, M * lay.N, y, stream, act == kActF16);
        }
        return hipGetLastError();
    }
    const uint8_t *pk = static_cast<const uint8_t *>(packed);
    const int mode = lay.tiles_per_group == 1 ? kGOneTile
                     : lay.whole_tiles()      ? kGWhole
                     : lay.G == 32            ? kGSplit32
                                              : kGSplit64;
    const int mt = (int)plan.m_tiles;
    auto go_act = [&](auto bits_c, auto wn_c, auto bm_c, auto act_c, int64_t n_cols, int64_t col0) {
        constexpr int B = decltype(bits_c)::value, WN = decltype(wn_c)::value, BM = decltype(bm_c)::value;
        constexpr int A = decltype(act_c)::value;
        const int64_t wgs = plan.m_tiles * n_cols * plan.splits;
        switch (mode) {
        case kGOneTile: launch_mode<B, kGOneTile, WN, BM, A>(wgs, mt, col0, plan, stream, x, pk, y, lay, M, ws); break;
        case kGWhole: launch_mode<B, kGWhole, WN, BM, A>(wgs, mt, col0, plan, stream, x, pk, y, lay, M, ws); break;
        case kGSplit32: launch_mode<B, kGSplit32, WN, BM, A>(wgs, mt, col0, plan, stream, x, pk, y, lay, M, ws); break;
        default: launch_mode<B, kGSplit64, WN, BM, A>(wgs, mt, col0, plan, stream, x, pk, y, lay, M, ws); break;
        }
    };
    auto go = [&](auto bits_c, auto wn_c, auto bm_c, int64_t n_cols, int64_t col0) {
        if (act == kActSiluMul)
            go_act(bits_c, wn_c, bm_c, ic<kActSiluMul>{}, n_cols, col0);
        else if (act == kActF16)
            go_act(bits_c, wn_c, bm_c, ic<kActF16>{}, n_cols, col0);
        else
            go_act(bits_c, wn_c, bm_c, ic<kActNone>{}, n_cols, col0);
    };
    auto both = [&](auto bits_c) {
        if (plan.rows != kGBM) { // short tiles: 128 columns only
            go(bits_c, ic<2>{}, ic<kShortTileRows>{}, plan.wide_cols, 0);
            return;
        }
        if (plan.wide_cols > 0)
            go(bits_c, ic<2>{}, ic<kGBM>{}, plan.wide_cols, 0);
        if (plan.narrow_cols > 0)
            go(bits_c, ic<1>{}, ic<kGBM>{}, plan.narrow_cols, plan.wide_cols * tile_cols(2));
    };
    if (bits == 4)
        both(ic<4>{});
    else
        both(ic<8>{});
    if (plan.splits > 1) {
        if (act == kActSiluMul)
            launch_splitk_sum_silu(ws, (int)plan.splits, M, lay.N, y, stream);
        else
            launch_splitk_sum(ws, (int)plan.splits, M * lay.N, y, stream, act == kActF16);
    }
    return hipGetLastError();
}

} // namespace tf
