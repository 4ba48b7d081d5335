// Prefill GEMM with fused dequantization (TileFuse summary, Methodology
// section 1: unpack and dequantize each weight tile once, keep the result in
// core-local memory and reuse it for the following matrix operations).
//
// MI355X design.  A workgroup (8 waves, two per SIMD) owns a 256 x 128 output
// tile; each wave a 64 x 64 sub-tile of 4 x 4 bf16 16x16x32 MFMA tiles (64
// fp32 accumulators per lane, in arch VGPRs).  Two waves per SIMD let one
// wave's MFMAs run while the other waits on LDS or does vector work.  K
// advances in stages of 64 rows.  Every global load is an LDS-DMA load
// (global_load_lds_dwordx4 / _dword), so nothing is staged through registers
// and the number of loads a stage issues is fixed; the waits are explicit
// vmcnt values:
//   - activations: a 3-deep ring of [256][64] bf16 stages, two stages ahead;
//   - codes and metadata records: one k-tile (W4) or two stages (W8) ahead.
// The packed codes of a stage are unpacked once into a [128][64] LDS tile as
// the exact bf16 values q - z (|q - z| <= 255 has at most 8 significant
// bits), double buffered, and all 256 rows of the tile reuse them.  All LDS
// tiles use an XOR swizzle of their 16-byte units so that fragment reads and
// writes are free of bank conflicts.
//
// The per-(group, column) scale is folded without a second accumulator set:
// the accumulator holds y / s_g while group g accumulates, so at a group
// boundary it is multiplied by s_g / s_{g+1} and at the end by the last s:
//     y = s_G * (... (s_0/s_1 * P_0 + P_1) * s_1/s_2 + ... + P_G)
// with P_g = sum_{k in g} x * (q - z) accumulated by the MFMAs in fp32.  A
// zero scale keeps the previous one and its group's operands are written as
// zeros, so its contribution vanishes as it should.  Consecutive scales must
// keep s_g / s_{g+1} and the running sums inside the fp32 range (true for any
// real checkpoint).
#include "tf_common.h"
#include "tf_launch.h"

namespace tf {

constexpr int kGBM = 256;                        // rows per workgroup tile
constexpr int kGBN = 128;                        // columns per workgroup tile
constexpr int kGBlocks = kGBN / kBlockCols;      // 8 packed blocks
constexpr int kStage = 64;                       // k rows per pipeline stage
constexpr int kAStages = 3;
constexpr int kAStageBytes = kGBM * kStage * 2;  // 32 KiB
constexpr int kBStageBytes = kGBN * kStage * 2;  // 16 KiB
constexpr int kCodeBufBytes = kGBlocks * 1024;   // codes of one k-tile (W4) or stage (W8)
constexpr int kGWaves = 8;                       // waves per workgroup (4 x 2 over the tile)
constexpr int kGThreads = 64 * kGWaves;
constexpr int kMetaWaveBytes = 256;              // record bytes DMA'd per wave (one block) per k-tile
constexpr int kMetaBufBytes = kGWaves * kMetaWaveBytes;
constexpr int kOffB = kAStages * kAStageBytes;
constexpr int kOffCodes = kOffB + 2 * kBStageBytes;
constexpr int kOffMeta = kOffCodes + 2 * kCodeBufBytes;
constexpr int kGemmLds = kOffMeta + 2 * kMetaBufBytes; // 148 KiB
static_assert(kGBlocks == kGWaves, "one packed block per wave");

// 16-byte unit (row, c) of a [rows][64] bf16 tile, c = 0..7.  Rows are 128
// bytes, so two share a 256-byte bank line; the XOR with (row / 2) % 8 puts
// the 16 rows a fragment read touches at one c into 16 distinct bank groups.
__device__ __forceinline__ int swz(int row, int c) { return (row << 3) + (c ^ ((row >> 1) & 7)); }

// s_waitcnt immediates (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; counters not named stay at their maximum (no wait).
template <int N> __device__ __forceinline__ void wait_vmcnt()
{
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Workgroup barrier for LDS filled by LDS-DMA: each wave has already waited
// for its own loads; the empty asm statements keep the compiler from moving
// memory operations across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS-DMA: lane i's 16 (or 4) bytes land at lds + 16 i (or 4 i).
__device__ __forceinline__ void dma16(const void *g, void *lds)
{
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *g, void *lds)
{
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds, 4, 0, 0);
}

// kGOneTile: every k-tile is exactly one group (G == 128, or G == K <= 128);
// kGWhole: every k-tile lies inside one group; kGSplit: G is 32 or 64.
enum GemmGroups { kGSplit = 0, kGWhole = 1, kGOneTile = 2 };

template <int BITS, int kMode>
__global__ __launch_bounds__(kGThreads, 1) void gemm_kernel(const uint16_t *__restrict__ x,
                                                            const uint8_t *__restrict__ packed,
                                                            uint16_t *__restrict__ y, Layout lay, int64_t M,
                                                            int m_tiles)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int RB = record_bytes(BITS);
    // records a k-tile can touch per block (split: up to four 32-row groups)
    constexpr int kRecs = kMode == kGSplit ? 4 : 1;
    constexpr int kBlockMeta = kRecs * RB; // <= 192 bytes: one dword per lane
    static_assert(kBlockMeta <= kMetaWaveBytes, "a block's records fit one dword DMA");
    constexpr bool kW8 = BITS == 8;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1; // 64-row and 64-column slot of the wave
    const int r = lane & 15, o = lane >> 4;

    // ---- tile order: consecutive tiles on one XCD share a column tile ----
    const int nwg = gridDim.x, bid = blockIdx.x;
    const int xcd = bid & 7, local = bid >> 3, q8 = nwg >> 3, rem = nwg & 7;
    const int tile = xcd < rem ? xcd * (q8 + 1) + local : rem * (q8 + 1) + (xcd - rem) * q8 + local;
    const int nt = tile / m_tiles, mt = tile - nt * m_tiles;
    const int64_t m0 = (int64_t)mt * kGBM;
    const int64_t blk0 = (int64_t)nt * kGBlocks;

    const int ktiles = (int)lay.ktiles;
    const int nstages = 2 * ktiles;
    const int steps = (int)lay.steps;
    const int sg = (int)(lay.G / kStepRows); // 32-row steps per group
    const int64_t K = lay.K;
    const bool one_tile = kMode == kGOneTile;

    uint8_t *const sA = lds;
    uint8_t *const sB = lds + kOffB;
    uint8_t *const sCodes = lds + kOffCodes;
    uint8_t *const sMeta = lds + kOffMeta;

    // ---- activations: wave w fills rows 32w .. 32w+31 of a stage, 8 rows per
    //      instruction; lane p takes row 8j + p/8 and the 16-byte unit that the
    //      swizzle places at slot p%8. ----
    const int a_row_in = lane >> 3, a_slot = lane & 7;
    // rows 32w + 8j + p/8 (j = 0..3), clamped at M - 1: the lane's base row
    // and 32-bit element offsets of the other three from it
    const uint16_t *a_base;
    int a_off[4];
    {
        const int64_t row0 = m0 + 32 * wave + a_row_in;
        const int64_t g0 = row0 < M ? row0 : M - 1; // rows past M are computed on a copy, never stored
        a_base = x + g0 * K;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int64_t gm = row0 + 8 * j;
            gm = gm < M ? gm : M - 1;
            a_off[j] = (int)((gm - g0) * K);
        }
    }
    // swizzle slot -> unit: (row / 2) % 8 is (4 (j % 2) + p / 16) % 8
    const int a_c8e = 8 * (a_slot ^ ((a_row_in >> 1) & 7));
    const int a_c8o = 8 * (a_slot ^ ((4 + (a_row_in >> 1)) & 7));
    auto dma_a = [&](int s) {
        uint8_t *dst = sA + (s % kAStages) * kAStageBytes + 32 * wave * 128;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int64_t k = (int64_t)s * kStage + ((j & 1) ? a_c8o : a_c8e);
            k = k < K ? k : 0; // rows past K meet zero weights
            dma16(a_base + a_off[j] + k, dst + j * 1024);
        }
    };
    // codes: wave w fetches block w (1 KiB; W8: one half tile)
    const int64_t my_blk = blk0 + wave < lay.nblocks ? blk0 + wave : 0; // blocks past N: any valid block
    auto dma_codes = [&](int t, int half, int buf) {
        const uint8_t *src =
            packed + my_blk * lay.block_bytes + lay.meta_bytes + (int64_t)t * tile_bytes(BITS) + 1024 * half + 16 * lane;
        dma16(src, sCodes + buf * kCodeBufBytes + wave * 1024);
    };
    // records of k-tile t for block w, as dwords
    auto first_group = [&](int t) -> int64_t { return one_tile ? t : ((int64_t)t * kTileRows) / lay.G; };
    auto dma_meta = [&](int t, int buf) {
        const int64_t g_first = first_group(t);
        const int64_t g = g_first + (4 * lane) / RB;
        const bool ok = lane < kBlockMeta / 4 && g < lay.ngroups;
        const uint8_t *src = ok ? packed + my_blk * lay.block_bytes + g_first * RB + 4 * lane : packed;
        dma4(src, sMeta + buf * kMetaBufBytes + wave * kMetaWaveBytes);
    };
    // the staged record of block bb (0..7) for group g, which k-tile t touches
    auto meta_rec = [&](int bb, int t, int64_t g) -> const uint8_t * {
        const uint8_t *rec = sMeta + (t & 1) * kMetaBufBytes + bb * kMetaWaveBytes;
        return one_tile ? rec : rec + (int)(g - first_group(t)) * RB;
    };
    auto code_buf = [&](int s) { return kW8 ? (s & 1) : ((s >> 1) & 1); };

    // ---- unpack stage sd into B buffer sd % 2: exact bf16 (q - z), zero where
    //      the row is past K or the group's scale is 0.  Columns past N need
    //      no care: their outputs are never stored.  Wave w unpacks block w;
    //      lane (o, r) column r, rows 32 kk + 8 o .. +7.  Split in two so the
    //      LDS reads are issued early and the arithmetic overlaps MFMAs. ----
    struct FillIn {
        u32x4 cw;        // the lane's code words
        float sv[2];     // scale per 32-row step
        uint32_t z[2];   // zero point per 32-row step
    };
    auto fill_load = [&](int sd, FillIn &in) {
        const int td = sd >> 1, hd = sd & 1;
        const uint8_t *codes = sCodes + code_buf(sd) * kCodeBufBytes + wave * 1024 + 16 * lane;
        if constexpr (kW8) {
            in.cw = *reinterpret_cast<const u32x4 *>(codes);
        } else {
            const u32x2 c2 = *reinterpret_cast<const u32x2 *>(codes + 8 * hd);
            in.cw = u32x4{c2[0], c2[1], 0u, 0u};
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int step = 4 * td + 2 * hd + kk;
            const int64_t g = one_tile ? td : (int64_t)step / sg;
            const uint8_t *rec = meta_rec(wave, td, g);
            in.sv[kk] = record_scale<BITS>(rec, r);
            in.z[kk] = record_zero<BITS>(rec, r);
        }
    };
    auto fill_store = [&](int sd, const FillIn &in) {
        const int td = sd >> 1, hd = sd & 1;
        uint8_t *dst = sB + (sd & 1) * kBStageBytes;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int step = 4 * td + 2 * hd + kk;
            // (q - z) * live as fma(q, live, -z * live): the mask costs nothing
            const float live = (step < steps && in.sv[kk] != 0.f) ? 1.f : 0.f;
            const float nz = -(float)in.z[kk] * live;
            float f[8];
            if constexpr (kW8)
                dequant_w8_pair(in.cw[2 * kk], in.cw[2 * kk + 1], live, nz, f);
            else
                dequant_w4_word(in.cw[kk], live, nz, f);
            const u32x4 v = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                             pack_bf16x2(f[6], f[7])};
            *reinterpret_cast<u32x4 *>(dst + 16 * swz(16 * wave + r, 4 * kk + o)) = v;
        }
    };

    // ---- scales of the lane's four columns (blocks 4 wn + j, column r) ----
    auto scales_of = [&](int64_t g, int t, float (&s)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s[j] = record_scale<BITS>(meta_rec(4 * wn + j, t, g), r);
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float seff[4];

    // ---- prologue: k-tile 0's codes and records, stages 0 and 1 of x ----
    dma_codes(0, 0, 0);
    dma_meta(0, 0);
    dma_a(0);
    if (nstages > 1) {
        if (kW8)
            dma_codes(0, 1, 1);
        dma_a(1);
        wait_vmcnt<4>();
    } else {
        wait_vmcnt<0>();
    }
    lds_barrier();
    {
        FillIn f0;
        fill_load(0, f0);
        fill_store(0, f0);
        float s0[4];
        scales_of(0, 0, s0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            seff[j] = s0[j] != 0.f ? s0[j] : 1.f;
    }
    wait_lgkmcnt0();
    lds_barrier();

    for (int t = 0; t < ktiles; ++t)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int s = 2 * t + h;
        // ---- loads for later stages: codes and records first, x last.  Past
        //      the end they re-read the last stage into slots nobody reads, so
        //      every stage issues the same loads. ----
        const int tn = t + 1 < ktiles ? t + 1 : ktiles - 1;
        const int sa = s + 2 < nstages ? s + 2 : nstages - 1;
        if (kW8)
            dma_codes(sa >> 1, sa & 1, s & 1);
        else if (h == 0)
            dma_codes(tn, 0, (t + 1) & 1);
        if (h == 0)
            dma_meta(tn, (t + 1) & 1);
        dma_a(sa);

        // ---- the next stage's codes and records (past the last stage this
        //      reads and later writes buffers nobody reads) ----
        FillIn fin;
        fill_load(s + 1, fin);

        // ---- MFMAs of stage s ----
        const uint8_t *a_st = sA + (s % kAStages) * kAStageBytes;
        const uint8_t *b_st = sB + h * kBStageBytes;
        // one-tile groups: the stage that ends k-tile t ends group t; fold in
        // s_t / s_{t+1} row tile by row tile right after each one's MFMAs
        const bool fold_here = one_tile && h == 1;
        float ratio[4];
        if (fold_here) {
            float sn[4];
            scales_of(tn, tn, sn);
            const bool more = t + 1 < ktiles;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // computed unconditionally (the asm pins it) so the last
                // k-tile's select stays a select, not a branch
                const float se = sn[j] != 0.f ? sn[j] : seff[j];
                float rt = seff[j] * __builtin_amdgcn_rcpf(se);
                asm volatile("" : "+v"(rt));
                ratio[j] = more ? rt : 1.f;
                seff[j] = more ? se : seff[j];
            }
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int step = 4 * t + 2 * h + kk;
            u32x4 bf[4], af[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *reinterpret_cast<const u32x4 *>(b_st + 16 * swz(64 * wn + 16 * j + r, 4 * kk + o));
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const u32x4 *>(a_st + 16 * swz(64 * wm + 16 * i + r, 4 * kk + o));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
                    if (fold_here && kk == 1) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[i][j][e] *= ratio[j];
                    }
                }
            }
            // group boundary after this step: rescale by s_g / s_{g+1}
            if (!one_tile && (step + 1) % sg == 0 && step + 1 < steps) {
                const int64_t gn = (int64_t)(step + 1) / sg;
                const int tg = (step + 1) >> 2; // k-tile holding the next group's first step
                float sn[4], rt[4];
                scales_of(gn, tg, sn);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float se = sn[j] != 0.f ? sn[j] : seff[j];
                    rt[j] = seff[j] * __builtin_amdgcn_rcpf(se);
                    seff[j] = se;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[i][j][e] *= rt[j];
            }
        }

        // ---- unpack the next stage's weights into the other B buffer ----
        fill_store(s + 1, fin);

        // ---- stage s + 1's x (issued one stage ago) must have landed: only
        //      this stage's four x loads may still be in flight ----
        wait_vmcnt<4>();
        wait_lgkmcnt0();
        lds_barrier();
    }
    wait_vmcnt<0>();

    // ---- epilogue: y = acc * s_last, fp32 -> bf16 (nearest even) ----
    const int64_t n0 = (int64_t)nt * kGBN;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = m0 + 64 * wm + 16 * i + 4 * o + e;
                const int64_t col = n0 + 64 * wn + 16 * j + r;
                if (row < M && col < lay.N)
                    y[row * lay.N + col] = f32_to_bf16_bits(acc[i][j][e] * seff[j]);
            }
}

// The kernel needs more than the default 64 KiB of dynamic LDS; raise the
// limit once per instantiation.
template <int BITS, int kMode> static void launch_mode(dim3 grid, hipStream_t stream, const uint16_t *x,
                                                       const uint8_t *pk, uint16_t *y, const Layout &lay, int64_t M,
                                                       int m_tiles)
{
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_kernel<BITS, kMode>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
    (void)attr;
    gemm_kernel<BITS, kMode><<<grid, kGThreads, kGemmLds, stream>>>(x, pk, y, lay, M, m_tiles);
}

hipError_t launch_gemm(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M, const Layout &lay,
                       hipStream_t stream)
{
    const int64_t m_tiles = (M + kGBM - 1) / kGBM;
    const int64_t n_tiles = (lay.N + kGBN - 1) / kGBN;
    const dim3 grid((unsigned)(m_tiles * n_tiles));
    const uint8_t *pk = static_cast<const uint8_t *>(packed);
    const int mode = lay.tiles_per_group == 1 ? kGOneTile : lay.whole_tiles() ? kGWhole : kGSplit;
    if (bits == 4) {
        if (mode == kGOneTile)
            launch_mode<4, kGOneTile>(grid, stream, x, pk, y, lay, M, (int)m_tiles);
        else if (mode == kGWhole)
            launch_mode<4, kGWhole>(grid, stream, x, pk, y, lay, M, (int)m_tiles);
        else
            launch_mode<4, kGSplit>(grid, stream, x, pk, y, lay, M, (int)m_tiles);
    } else {
        if (mode == kGOneTile)
            launch_mode<8, kGOneTile>(grid, stream, x, pk, y, lay, M, (int)m_tiles);
        else if (mode == kGWhole)
            launch_mode<8, kGWhole>(grid, stream, x, pk, y, lay, M, (int)m_tiles);
        else
            launch_mode<8, kGSplit>(grid, stream, x, pk, y, lay, M, (int)m_tiles);
    }
    return hipGetLastError();
}

} // namespace tf
