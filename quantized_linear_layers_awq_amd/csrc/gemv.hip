// Token-generation GEMV, M = 1..16 (TileFuse summary, Methodology section 3:
// batch-1 GEMV, memory-bound at full precision; spread the weight stream over
// the whole machine instead of a slice of it), and the same dataflow with
// 16-row chunks of x (gemv_mid_kernel below) for up to 64 rows, which GEMM
// calls of up to 64 rows run as well.
//
// MI355X design.  One workgroup owns one 16-column block of the packed buffer
// -- a single contiguous byte range -- and its waves split K between them, so
// partial sums combine in LDS and no cross-workgroup reduction, workspace,
// atomic or device-wide fence is needed.  The waves per workgroup are chosen
// so the grid holds about 16 waves per CU (up to 16 per workgroup for narrow
// layers).  The chunk of activations and metadata a workgroup needs is staged
// in LDS; a wave then streams its k-tiles with one 16-byte non-temporal load
// per lane per 128 rows (W8: two), a fixed number of k-tiles ahead.
//
// Unpack happens in registers: for W4 a single and/or per pair of codes turns
// nibbles into the bf16 values 128 + q (exact), which feed a 16x16x32 bf16
// MFMA as the B operand with the activations as A (rows >= M are zero).  The
// zero point goes through the same MFMA: a B operand holding bf16(128 + z) in
// every row gives sum_k x * (128 + z).  At each group end the group's scale is
// folded in once per (group, column):
//     y += s * (sum_k x * (128 + q)  -  sum_k x * (128 + z))
// which is sum_k x * (q - z) * s rearranged.  Both sums see the same
// activations in the same order, so where q == z they are bitwise equal and
// the contribution is exactly zero.  W8 uses bf16(q) and bf16(z) (exact).  No
// bf16 weight is formed, none is written anywhere.  The waves of a workgroup
// combine in a fixed order, so results are deterministic.
#include "tf_common.h"
#include "tf_launch.h"
#include "tf_operands.h"

namespace tf {

constexpr int kGemvMaxWaves = 16;
constexpr int kGemvTargetWaves = 4096; // about 16 per CU
// K ranges of the 16-row-chunk GEMV: at least 2 k-tiles, at most 16 ranges
constexpr int kGemvMinSplitTiles = 2;
constexpr int kGemvMaxSplits = 16;

// SiLU, x * sigmoid(x) = x / (1 + e^-x); at large negative x the
// exponential overflows to +inf and the quotient is -0, the limit.
__device__ __forceinline__ float silu(float v) { return v / (1.f + expf(-v)); }

// The codes of one k-tile held by one lane: W4 16 bytes, W8 32 bytes.
template <int BITS> struct TileCodes {
    u32x4 w[BITS == 4 ? 1 : 2];
};

template <int BITS, bool F16>
__device__ __forceinline__ u32x4 code_operand(const TileCodes<BITS> &c, int u, uint32_t magic)
{
    if constexpr (BITS == 4)
        return w4_operand<F16>(c.w[0][u], magic);
    else
        return w8_operand<F16>(c.w[u >> 1][2 * (u & 1)], c.w[u >> 1][2 * (u & 1) + 1]);
}

// A wave's code tiles are read through a buffer resource whose range ends
// at the wave's last k-tile.  The ring's look-ahead loads past that end
// return zero without a memory access, so every slot can be refilled
// unconditionally (the wait counts stay exact) and no tile is read twice.
typedef __amdgpu_buffer_rsrc_t CodeRange;
__device__ __forceinline__ CodeRange code_range(const uint8_t *tiles, uint32_t bytes)
{
    // stride 0, range [0, bytes), dword data format (required on gfx9)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(tiles), 0, (int)bytes, 0x00020000);
}

// The codes of tile byte offset off (lane offset included).  kPolicy is the
// load's cache-policy field: 2 = non-temporal, 0 = the default policy.
template <int BITS, int kPolicy = 2>
__device__ __forceinline__ void load_codes(TileCodes<BITS> &c, CodeRange cr, uint32_t off)
{
    c.w[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(cr, (int)off, 0, kPolicy));
    if constexpr (BITS == 8)
        c.w[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(cr, (int)off + 1024, 0, kPolicy));
}

__device__ __forceinline__ void fold(f32x4 &yacc, f32x4 &gacc, f32x4 &zacc, float s)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        yacc[i] = fmaf(s, gacc[i] - zacc[i], yacc[i]);
    gacc = zacc = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Launch-time geometry: the blocks a workgroup covers and the K chunks it
// stages in LDS.
struct GemvChunks {
    int bpw;      // 16-column blocks per workgroup (they share the staged x)
    int tiles;    // k-tiles per chunk
    int xpitch;   // bf16 elements per staged activation row (chunk rows + 8)
    int meta_cap; // bytes reserved per block for the chunk's metadata records
    int lds;      // dynamic LDS bytes per workgroup
};

// How the k-tiles of a block map onto metadata groups.
enum GroupMode {
    kSplitTiles = 0, // G in {32, 64}: a k-tile holds several groups
    kMultiTile = 1,  // a group spans several k-tiles (G a multiple of 256, or G == K)
    kOneTile = 2     // every k-tile is exactly one group (G == 128, or G == K <= 128)
};

// A chunk of K is staged per workgroup: activations x[0:M][chunk] (zero past
// K) and the metadata records of the groups the chunk touches, loaded before
// the chunk's first codes so that the staging barrier does not wait for the
// codes.  The only vector-memory loads in the main loop are then the code
// stream, issued in the order it is consumed, a fixed D k-tiles ahead;
// vector-memory counters retire in order, so waiting for tile t never waits
// for anything issued after it.  Each ring slot is unpacked into MFMA operands before it is
// refilled, so the slot keeps its registers and no wait drains the ring.
//
// ACT = kActSiluMul: a [gate | up] layer of N = 2 N' columns packed by
// tf_repack_*_gate_up, so that columns c and c + 8 of block j are gate and up
// column 8 j + c; the kernel writes y[m][8 j + c] = silu(g) * u from the fp32
// sums, rounded once.
template <int BITS, int kMode, int D, int BPW, int ACT = kActNone>
__global__ __launch_bounds__(1024) void gemv_kernel(const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed,
                                                    uint16_t *__restrict__ y, Layout lay, int M, GemvChunks ch)
{
    // Launches whose waves stream at most 3 k-tiles each (ring depth 2) ran
    // faster with the default cache policy than with non-temporal loads;
    // longer streams ran faster non-temporal (the decoder layer's launches,
    // queued back to back).
    constexpr int kCodePolicy = D == 2 ? 0 : 2;
    // D: k-tiles of codes in flight per wave
    constexpr uint32_t TB = tile_bytes(BITS), RB = record_bytes(BITS);
    constexpr bool F16 = ACT == kActF16; // fp16 x, scales and y (else bf16)
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint16_t *sx = reinterpret_cast<uint16_t *>(smem + BPW * ch.meta_cap);
    float *red = reinterpret_cast<float *>(smem); // reused after the last chunk

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int W = blockDim.x >> 6;
    const int Wb = W / BPW;                               // waves per block
    const int bi = BPW == 1 ? 0 : wave / Wb;              // this wave's block
    const int ws = wave - bi * Wb;                        // and its share of K
    const int r = lane & 15, o = lane >> 4;
    const int64_t blk0 = (int64_t)blockIdx.x * BPW;       // first block of the workgroup
    const int64_t blk = blk0 + bi;
    const bool blk_ok = blk < lay.nblocks;                // a last workgroup may be partial
    const uint8_t *meta = packed + (blk_ok ? blk : 0) * lay.block_bytes;
    const uint8_t *tiles = meta + lay.meta_bytes;
    const uint32_t lane_off = 16 * lane;
    uint8_t *smeta = smem + bi * ch.meta_cap;             // this block's staged records
    // MFMA rows >= M are never stored, so their lanes read row 0 instead of
    // being masked off.
    const int xr = r < M ? r : 0;
    const uint32_t magic = magic_in_vgpr<F16>();
    const int ktiles = (int)lay.ktiles;
    const f32x4 zf = {0.f, 0.f, 0.f, 0.f};
    // One block per workgroup with one group per k-tile: the waves' k-tile
    // ranges, and so the x columns and the records each reads, are disjoint.
    // Each wave then stages only its own part, and no workgroup barrier
    // separates the staging from the loop.
    constexpr bool kPerWave = kMode == kOneTile && BPW == 1;

    f32x4 yacc = zf, gacc = zf, zacc = zf;
    TileCodes<BITS> ring[D];

    for (int c0 = 0; c0 < ktiles; c0 += ch.tiles) {
        const int c1 = c0 + ch.tiles < ktiles ? c0 + ch.tiles : ktiles;
        const int nct = c1 - c0;
        const int a = c0 + nct * ws / Wb, b = c0 + nct * (ws + 1) / Wb; // this wave's k-tiles
        const int n = blk_ok ? b - a : 0;
        const int64_t k0 = (int64_t)c0 * kTileRows;
        const int64_t k1 = (int64_t)c1 * kTileRows < lay.K ? (int64_t)c1 * kTileRows : lay.K;
        const int64_t g0 = (uint32_t)k0 / (uint32_t)lay.G, g1 = (uint32_t)(k1 - 1) / (uint32_t)lay.G;
        const CodeRange cr = code_range(tiles, (uint32_t)(n > 0 ? b : 0) * TB);
        if constexpr (kPerWave) {
            // ---- this wave's k-tiles a .. b - 1 only: x[m][128 a .. 128 b)
            //      (zero past K) and the records of groups a .. b - 1, loaded
            //      before the codes, then stored to the same LDS places the
            //      shared staging uses; LDS operations of one wave complete in
            //      order, so the loop's reads see them without a barrier ----
            const int wupr = n * (kTileRows / 8); // 16-byte units per row of x
            const int wx_units = M * wupr;
            const uint32_t wupr_m = 0xFFFFFFFFu / (uint32_t)(wupr > 0 ? wupr : 1) + 1u;
            constexpr int XR = 4;
            u32x4 xv[XR];
#pragma unroll
            for (int i = 0; i < XR; ++i) {
                const int e = lane + 64 * i;
                xv[i] = u32x4{0u, 0u, 0u, 0u};
                if (e < wx_units) {
                    const int m = (int)__umulhi((uint32_t)e, wupr_m), u8 = (a - c0) * 16 + e - m * wupr;
                    const int64_t k = k0 + 8 * u8;
                    if (k < lay.K)
                        xv[i] = load16(x + (int64_t)m * lay.K + k);
                }
            }
            const int rec_words = n * (int)RB / 8;
            u32x2 mv = {0u, 0u};
            if (lane < rec_words)
                mv = *reinterpret_cast<const u32x2 *>(meta + (int64_t)a * RB + 8 * lane);
            if (n > 0) {
#pragma unroll
                for (int j = 0; j < D; ++j)
                    load_codes<BITS, kCodePolicy>(ring[j], cr, lane_off + (uint32_t)(a + j) * TB);
            }
            // the waves' ranges move between chunks: another wave may still
            // read the previous chunk where this one stores
            if (c0 > 0)
                __syncthreads();
#pragma unroll
            for (int i = 0; i < XR; ++i) {
                const int e = lane + 64 * i;
                if (e < wx_units) {
                    const int m = (int)__umulhi((uint32_t)e, wupr_m), u8 = (a - c0) * 16 + e - m * wupr;
                    *reinterpret_cast<u32x4 *>(sx + m * ch.xpitch + 8 * u8) = xv[i];
                }
            }
            for (int e = lane + 64 * XR; e < wx_units; e += 64) { // more than XR per lane
                const int m = (int)__umulhi((uint32_t)e, wupr_m), u8 = (a - c0) * 16 + e - m * wupr;
                const int64_t k = k0 + 8 * u8;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (k < lay.K)
                    v = load16(x + (int64_t)m * lay.K + k);
                *reinterpret_cast<u32x4 *>(sx + m * ch.xpitch + 8 * u8) = v;
            }
            uint8_t *const srec = smeta + (a - c0) * RB;
            if (lane < rec_words)
                *reinterpret_cast<u32x2 *>(srec + 8 * lane) = mv;
            for (int e = lane + 64; e < rec_words; e += 64) // more than one per lane
                *reinterpret_cast<u32x2 *>(srec + 8 * e) =
                    *reinterpret_cast<const u32x2 *>(meta + (int64_t)a * RB + 8 * e);
            __builtin_amdgcn_wave_barrier();
        } else {
            // ---- x[m][k0 .. k0 + 128 nct) (zero past K) and the chunk's records
            //      are loaded first, into registers: they come from L2 and are
            //      stored to LDS before the barrier, and vector-memory loads
            //      retire in order, so loads issued after the codes would wait for
            //      the codes' HBM latency before the barrier ----
            const int units_per_row = nct * (kTileRows / 8);
            const int x_units = M * units_per_row;
            // unit e is row e / units_per_row: a multiply-high by a per-chunk
            // constant instead of a division, exact since e * units_per_row <
            // 2^32 (the chunk fits LDS: units_per_row < 10^4, e < 16 of them)
            const uint32_t upr_m = 0xFFFFFFFFu / (uint32_t)units_per_row + 1u;
            constexpr int XR = 4; // x units per thread held in registers
            u32x4 xv[XR];
#pragma unroll
            for (int i = 0; i < XR; ++i) {
                const int e = tid + i * (int)blockDim.x;
                xv[i] = u32x4{0u, 0u, 0u, 0u};
                if (e < x_units) {
                    const int m = (int)__umulhi((uint32_t)e, upr_m), u8 = e - m * units_per_row;
                    const int64_t k = k0 + 8 * u8;
                    if (k < lay.K)
                        xv[i] = load16(x + (int64_t)m * lay.K + k);
                }
            }
            const int rec_words = (int)((g1 - g0 + 1) * RB / 8);
            u32x2 mv[BPW];
#pragma unroll
            for (int eb = 0; eb < BPW; ++eb) {
                mv[eb] = u32x2{0u, 0u};
                if (tid < rec_words && blk0 + eb < lay.nblocks)
                    mv[eb] = *reinterpret_cast<const u32x2 *>(packed + (blk0 + eb) * lay.block_bytes + g0 * RB + 8 * tid);
            }
            // ---- then the codes (loads past the wave's range are dropped) ----
            if (n > 0) {
#pragma unroll
                for (int j = 0; j < D; ++j)
                    load_codes<BITS, kCodePolicy>(ring[j], cr, lane_off + (uint32_t)(a + j) * TB);
            }

            if (c0 > 0)
                __syncthreads(); // the previous chunk's LDS is no longer read
#pragma unroll
            for (int i = 0; i < XR; ++i) {
                const int e = tid + i * (int)blockDim.x;
                if (e < x_units) {
                    const int m = (int)__umulhi((uint32_t)e, upr_m), u8 = e - m * units_per_row;
                    *reinterpret_cast<u32x4 *>(sx + m * ch.xpitch + 8 * u8) = xv[i];
                }
            }
            for (int e = tid + XR * (int)blockDim.x; e < x_units; e += blockDim.x) { // more than XR per thread
                const int m = (int)__umulhi((uint32_t)e, upr_m), u8 = e - m * units_per_row;
                const int64_t k = k0 + 8 * u8;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (k < lay.K)
                    v = load16(x + (int64_t)m * lay.K + k);
                *reinterpret_cast<u32x4 *>(sx + m * ch.xpitch + 8 * u8) = v;
            }
#pragma unroll
            for (int eb = 0; eb < BPW; ++eb) {
                if (blk0 + eb < lay.nblocks) {
                    if (tid < rec_words)
                        *reinterpret_cast<u32x2 *>(smem + eb * ch.meta_cap + 8 * tid) = mv[eb];
                    const uint8_t *src = packed + (blk0 + eb) * lay.block_bytes + g0 * RB;
                    for (int e = tid + (int)blockDim.x; e < rec_words; e += blockDim.x) // more than one per thread
                        *reinterpret_cast<u32x2 *>(smem + eb * ch.meta_cap + 8 * e) =
                            *reinterpret_cast<const u32x2 *>(src + 8 * e);
                }
            }
            __syncthreads();
        }
        if (n <= 0)
            continue;
        const uint16_t *xl = sx + xr * ch.xpitch + 8 * o - c0 * kTileRows;
        // kMultiTile: tiles left in the current group and the group's record
        const int tpg = kMode == kMultiTile ? (int)lay.tiles_per_group : 1;
        const int ga = a / tpg;
        int tg_left = tpg - (a - ga * tpg);
        const uint8_t *rec = smeta + (ga - (int)g0) * RB;
        const int sh = lay.G == kStepRows ? 0 : 1; // kSplitTiles: G is 32 or 64

        for (int i = 0; i < n; i += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                const int ti = i + j;
                const int t = a + ti;
                // consume the slot, then refill it with the tile D ahead
                u32x4 ops[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    ops[u] = code_operand<BITS, F16>(ring[j], u, magic);
                load_codes<BITS, kCodePolicy>(ring[j], cr, lane_off + (uint32_t)(t + D) * TB);
                if (ti < n) {
                    u32x4 xa[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        xa[u] = *reinterpret_cast<const u32x4 *>(xl + t * kTileRows + kStepRows * u);
                    if constexpr (kMode == kOneTile) {
                        const uint8_t *rg = smeta + (t - (int)g0) * RB;
                        const u32x4 zop = zero_operand<BITS, F16>(record_zero<BITS>(rg, r));
                        f32x4 ga4 = mfma16x16x32<F16>(xa[0], ops[0], zf);
                        f32x4 za4 = mfma16x16x32<F16>(xa[0], zop, zf);
#pragma unroll
                        for (int u = 1; u < 4; ++u) {
                            ga4 = mfma16x16x32<F16>(xa[u], ops[u], ga4);
                            za4 = mfma16x16x32<F16>(xa[u], zop, za4);
                        }
                        const float sc = record_scale<BITS, F16>(rg, r);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            yacc[e] = fmaf(sc, ga4[e] - za4[e], yacc[e]);
                    } else if constexpr (kMode == kMultiTile) {
                        const u32x4 zop = zero_operand<BITS, F16>(record_zero<BITS>(rec, r));
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            gacc = mfma16x16x32<F16>(xa[u], ops[u], gacc);
                            zacc = mfma16x16x32<F16>(xa[u], zop, zacc);
                        }
                        --tg_left;
                        if (tg_left == 0 || ti + 1 == n)
                            fold(yacc, gacc, zacc, record_scale<BITS, F16>(rec, r));
                        if (tg_left == 0) {
                            tg_left = tpg;
                            rec += RB;
                        }
                    } else {
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int64_t st = 4 * (int64_t)t + u;
                            if (st < lay.steps) {
                                const uint8_t *rg = smeta + ((st >> sh) - g0) * RB;
                                const f32x4 ga4 = mfma16x16x32<F16>(xa[u], ops[u], zf);
                                const f32x4 za4 =
                                    mfma16x16x32<F16>(xa[u], zero_operand<BITS, F16>(record_zero<BITS>(rg, r)), zf);
                                gacc += ga4;
                                zacc += za4;
                                if (((st + 1) & ((1 << sh) - 1)) == 0)
                                    fold(yacc, gacc, zacc, record_scale<BITS, F16>(rg, r));
                            }
                        }
                    }
                }
            }
        }
    }

    // ---- combine the waves (C layout: lane holds rows 4o + i of column r) ----
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e)
        red[(wave * 16 + 4 * o + e) * kBlockCols + r] = yacc[e];
    __syncthreads();
    // each block sums its own waves, in wave order
    if constexpr (ACT != kActSiluMul) {
#pragma unroll
        for (int eb = 0; eb < BPW; ++eb) {
            for (int e = tid; e < M * kBlockCols; e += blockDim.x) {
                const int row = e >> 4, col = e & 15;
                float v = 0.f;
                for (int w = eb * Wb; w < (eb + 1) * Wb; ++w)
                    v += red[(w * 16 + row) * kBlockCols + col];
                const int64_t nn = (blk0 + eb) * kBlockCols + col;
                if (nn < lay.N)
                    y[(int64_t)row * lay.N + nn] = f32_to_half_bits<F16>(v);
            }
        }
    } else {
        auto block_sum = [&](int eb, int row, int col) {
            float v = 0.f;
            for (int w = eb * Wb; w < (eb + 1) * Wb; ++w)
                v += red[(w * 16 + row) * kBlockCols + col];
            return v;
        };
        const int64_t n2 = lay.N >> 1;
        constexpr int kHalf = kBlockCols / 2;
#pragma unroll
        for (int eb = 0; eb < BPW; ++eb) {
            if (blk0 + eb >= lay.nblocks)
                break;
            for (int e = tid; e < M * kHalf; e += blockDim.x) {
                const int row = e >> 3, c = e & 7;
                const float g = block_sum(eb, row, c), u = block_sum(eb, row, c + kHalf);
                y[(int64_t)row * n2 + (blk0 + eb) * kHalf + c] = f32_to_bf16_bits(silu(g) * u);
            }
        }
    }
}

// ---- GEMV for 2..64 activation rows, 16-row chunks ----
//
// Every weight operand feeds MT = 1, 2 or 4 row chunks of 16, so one unpack
// serves up to 64 rows.  A workgroup is eight waves, one
// 16-column block each (the activations staged in LDS serve 128 columns),
// and K may be split over workgroups (gridDim.y ranges of split_tiles
// k-tiles) whose fp32 partial sums a second kernel adds in range order.  Each
// wave walks its range of k-tiles in one continuous ring of D code loads;
// the range is staged in chunks of `tiles` k-tiles, double buffered: the
// next chunk's activations and records are loaded into registers before the
// current chunk's code refills are issued (vector-memory loads retire in
// order, so storing them to LDS at the chunk's end never waits for codes in
// flight), and one barrier per chunk separates the buffers' uses.
constexpr int kMidWaves = 8;   // waves (blocks) per workgroup
// activation units of 16 bytes staged per thread per chunk, by row chunks
constexpr int mid_xregs(int) { return 8; }
constexpr int kMidRecRegs = 4; // record words of 8 bytes per thread per chunk
// k-tiles of codes in flight per wave: the chunk length, 8 or 4 (a chunk
// holds 4096 / (16 M) k-tiles of activations: 8 up to 32 rows, 4 above)

struct MidChunks {
    int tiles;       // k-tiles per staged chunk (a multiple of the ring depth)
    int xpitch;      // bf16 elements per staged activation row (chunk rows + 8)
    int meta_cap;    // bytes per block of a chunk's records
    int lds;         // dynamic LDS bytes: two record buffers, two x buffers
    int split_tiles; // k-tiles per K range (gridDim.y ranges)
};

// ACT = kActSiluMul: as in gemv_kernel, a [gate | up] layer packed by
// tf_repack_*_gate_up; lanes r and r + 8 hold gate and up column 8 blk + r.
// With K split, the partials are the plain ones and the summing kernel
// applies the product.
template <int BITS, int kMode, int MT, int D, int ACT = kActNone>
__global__ __launch_bounds__(64 * kMidWaves) void gemv_mid_kernel(const uint16_t *__restrict__ x,
                                                                 const uint8_t *__restrict__ packed,
                                                                 uint16_t *__restrict__ y, Layout lay, int M,
                                                                 MidChunks ch, float *__restrict__ ws)
{
    constexpr uint32_t TB = tile_bytes(BITS), RB = record_bytes(BITS);
    constexpr bool F16 = ACT == kActF16; // fp16 x, scales and y (else bf16)
    constexpr int kThreads = 64 * kMidWaves;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int meta_buf_bytes = kMidWaves * ch.meta_cap;
    const int x_buf_bytes = M * ch.xpitch * 2;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, o = lane >> 4;
    const int64_t blk0 = (int64_t)blockIdx.x * kMidWaves;
    const int64_t blk = blk0 + wave;
    const bool blk_ok = blk < lay.nblocks;
    const int ktiles = (int)lay.ktiles;
    const int split = blockIdx.y;
    const int kt_begin = split * ch.split_tiles;
    const int kt_end = kt_begin + ch.split_tiles < ktiles ? kt_begin + ch.split_tiles : ktiles;
    // the wave's k range of its block; a wave past the last block loads nothing
    const CodeRange cr = code_range(packed + (blk_ok ? blk : 0) * lay.block_bytes + lay.meta_bytes,
                                    (uint32_t)(blk_ok ? kt_end : 0) * TB);
    const uint32_t lane_off = 16 * lane;
    const int nchunks = (kt_end - kt_begin + ch.tiles - 1) / ch.tiles;
    // rows >= M are never stored; their lanes read row 0
    const int xr = r < M ? r : 0;
    int xoff[MT]; // row chunk c relative to chunk 0
#pragma unroll
    for (int c = 0; c < MT; ++c)
        xoff[c] = c == 0 ? 0 : ((16 * c + r < M ? 16 * c + r : 0) - xr) * ch.xpitch;
    const uint32_t magic = magic_in_vgpr<F16>();
    const f32x4 zf = {0.f, 0.f, 0.f, 0.f};

    // ---- staging of chunk cc: activations x[0:M][chunk] (zero past K) and
    //      the records of the groups the chunk touches, for all eight blocks.
    //      A thread's units are split into (row, unit) and (block, word) by a
    //      multiply-high with a per-chunk constant instead of a division:
    //      floor(n / d) = umulhi(n, floor((2^32 - 1) / d) + 1) exactly for
    //      2 <= d and n d < 2^32 (here n < 8192, d <= 2048). ----
    constexpr int XR = mid_xregs(MT);
    u32x4 xv[XR];
    u32x2 mv[kMidRecRegs];
    struct Chunk {
        int c0, c1, upr, rw;
        uint32_t upr_m, rw_m;
        uint32_t g0;
    };
    auto chunk_info = [&](int cc) {
        Chunk c;
        c.c0 = kt_begin + cc * ch.tiles;
        c.c1 = c.c0 + ch.tiles < kt_end ? c.c0 + ch.tiles : kt_end;
        c.upr = (c.c1 - c.c0) * (kTileRows / 8);
        const uint32_t k0 = (uint32_t)c.c0 * kTileRows;
        const uint32_t k1 = (uint32_t)c.c1 * kTileRows < (uint32_t)lay.K ? (uint32_t)c.c1 * kTileRows : (uint32_t)lay.K;
        c.g0 = k0 / (uint32_t)lay.G;
        c.rw = (int)(((k1 - 1) / (uint32_t)lay.G - c.g0 + 1) * RB / 8);
        c.upr_m = 0xFFFFFFFFu / (uint32_t)c.upr + 1u;
        c.rw_m = 0xFFFFFFFFu / (uint32_t)c.rw + 1u;
        return c;
    };
    // Every thread issues the same loads on every path (addresses clamped
    // into the buffers, unused values zeroed afterwards), so the
    // vector-memory wait before the LDS stores counts exactly the loads
    // issued after them and never drains the code ring.
    auto stage_load = [&](const Chunk &c) {
        const int64_t k0 = (int64_t)c.c0 * kTileRows;
        const int x_units = M * c.upr;
#pragma unroll
        for (int i = 0; i < XR; ++i) {
            const int e = tid + i * kThreads;
            const int ec = e < x_units ? e : x_units - 1;
            const int m = (int)__umulhi((uint32_t)ec, c.upr_m), u8 = ec - m * c.upr;
            const int64_t k = k0 + 8 * u8;
            xv[i] = load16(x + (int64_t)m * lay.K + (k < lay.K ? k : lay.K - 8));
        }
#pragma unroll
        for (int i = 0; i < kMidRecRegs; ++i) {
            const int e = tid + i * kThreads;
            const int eb = (int)__umulhi((uint32_t)e, c.rw_m), w = e - eb * c.rw;
            const bool ok = eb < kMidWaves && blk0 + eb < lay.nblocks;
            const int64_t b = ok ? blk0 + eb : 0;
            mv[i] = *reinterpret_cast<const u32x2 *>(packed + b * lay.block_bytes + (int64_t)c.g0 * RB + 8 * (ok ? w : 0));
        }
    };
    auto stage_store = [&](const Chunk &c, int cc) {
        uint8_t *mbuf = smem + (cc & 1) * meta_buf_bytes;
        uint16_t *xbuf = reinterpret_cast<uint16_t *>(smem + 2 * meta_buf_bytes + (cc & 1) * x_buf_bytes);
        const int x_units = M * c.upr;
        const int64_t k0 = (int64_t)c.c0 * kTileRows;
#pragma unroll
        for (int i = 0; i < XR; ++i) {
            const int e = tid + i * kThreads;
            if (e < x_units) {
                const int m = (int)__umulhi((uint32_t)e, c.upr_m), u8 = e - m * c.upr;
                const bool in_k = k0 + 8 * u8 < lay.K; // columns past K stage as zero
                *reinterpret_cast<u32x4 *>(xbuf + m * ch.xpitch + 8 * u8) = in_k ? xv[i] : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < kMidRecRegs; ++i) {
            const int e = tid + i * kThreads;
            const int eb = (int)__umulhi((uint32_t)e, c.rw_m), w = e - eb * c.rw;
            if (eb < kMidWaves && blk0 + eb < lay.nblocks)
                *reinterpret_cast<u32x2 *>(mbuf + eb * ch.meta_cap + 8 * w) = mv[i];
        }
    };

    f32x4 yacc[MT], gacc[MT], zacc[MT];
#pragma unroll
    for (int c = 0; c < MT; ++c)
        yacc[c] = gacc[c] = zacc[c] = zf;
    TileCodes<BITS> ring[D];

    // ---- prologue: chunk 0 staged, the ring filled with the first D tiles.
    //      A wave past the last block computes on zeros and stores nothing.
    Chunk cur = chunk_info(0);
    stage_load(cur);
#pragma unroll
    for (int j = 0; j < D; ++j)
        load_codes<BITS>(ring[j], cr, lane_off + (uint32_t)(kt_begin + j) * TB);
    stage_store(cur, 0);
    __syncthreads();

    // kMultiTile: tiles left in the current group, and the group
    const int tpg = kMode == kMultiTile ? (int)lay.tiles_per_group : 1;
    int64_t gcur = kt_begin / tpg;
    int tg_left = tpg - (kt_begin - (int)gcur * tpg);
    const int sh = lay.G == kStepRows ? 0 : 1; // kSplitTiles: G is 32 or 64

    for (int cc = 0; cc < nchunks; ++cc) {
        const int c0 = cur.c0, c1 = cur.c1;
        const int64_t g0 = cur.g0;
        const bool more = cc + 1 < nchunks;
        const Chunk nxt = more ? chunk_info(cc + 1) : cur;
        const uint8_t *smeta = smem + (cc & 1) * meta_buf_bytes + wave * ch.meta_cap;
        const uint16_t *xl = reinterpret_cast<const uint16_t *>(smem + 2 * meta_buf_bytes + (cc & 1) * x_buf_bytes) +
                             xr * ch.xpitch + 8 * o - c0 * kTileRows;
        // D k-tiles from tile i.  The next chunk's staging loads are issued
        // after the chunk's first tile, ahead of its code refills: at that
        // tile only codes are in flight, so its wait is exact, and storing
        // the staged values at the chunk's end waits for none of the refills.
        auto group = [&](int i, bool first) {
#pragma unroll
                for (int j = 0; j < D; ++j) {
                    const int t = i + j;
                    if (t < c1) {
                        u32x4 ops[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            ops[u] = code_operand<BITS, F16>(ring[j], u, magic);
                        auto xfrag = [&](int c, int u) {
                            return *reinterpret_cast<const u32x4 *>(xl + xoff[c] + t * kTileRows + kStepRows * u);
                        };
                        if constexpr (kMode == kOneTile) {
                            const uint8_t *rg = smeta + (t - (int)g0) * RB;
                            const u32x4 zop = zero_operand<BITS, F16>(record_zero<BITS>(rg, r));
#pragma unroll
                            for (int c = 0; c < MT; ++c) {
                                u32x4 xa[4];
#pragma unroll
                                for (int u = 0; u < 4; ++u)
                                    xa[u] = xfrag(c, u);
                                f32x4 ga4 = mfma16x16x32<F16>(xa[0], ops[0], zf);
                                f32x4 za4 = mfma16x16x32<F16>(xa[0], zop, zf);
#pragma unroll
                                for (int u = 1; u < 4; ++u) {
                                    ga4 = mfma16x16x32<F16>(xa[u], ops[u], ga4);
                                    za4 = mfma16x16x32<F16>(xa[u], zop, za4);
                                }
                                const float sc = record_scale<BITS, F16>(rg, r);
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    yacc[c][e] = fmaf(sc, ga4[e] - za4[e], yacc[c][e]);
                            }
                        } else if constexpr (kMode == kMultiTile) {
                            const uint8_t *rec = smeta + (gcur - g0) * RB;
                            const u32x4 zop = zero_operand<BITS, F16>(record_zero<BITS>(rec, r));
#pragma unroll
                            for (int c = 0; c < MT; ++c) {
#pragma unroll
                                for (int u = 0; u < 4; ++u) {
                                    const u32x4 xa = xfrag(c, u);
                                    gacc[c] = mfma16x16x32<F16>(xa, ops[u], gacc[c]);
                                    zacc[c] = mfma16x16x32<F16>(xa, zop, zacc[c]);
                                }
                            }
                            --tg_left;
                            if (tg_left == 0 || t + 1 == kt_end) {
                                const float sc = record_scale<BITS, F16>(rec, r);
#pragma unroll
                                for (int c = 0; c < MT; ++c)
                                    fold(yacc[c], gacc[c], zacc[c], sc);
                            }
                            if (tg_left == 0) {
                                tg_left = tpg;
                                ++gcur;
                            }
                        } else {
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
                                const int64_t st = 4 * (int64_t)t + u;
                                if (st < lay.steps) {
                                    const uint8_t *rg = smeta + ((st >> sh) - g0) * RB;
                                    const u32x4 zop = zero_operand<BITS, F16>(record_zero<BITS>(rg, r));
                                    const bool last = ((st + 1) & ((1 << sh) - 1)) == 0;
#pragma unroll
                                    for (int c = 0; c < MT; ++c) {
                                        const u32x4 xa = xfrag(c, u);
                                        gacc[c] += mfma16x16x32<F16>(xa, ops[u], zf);
                                        zacc[c] += mfma16x16x32<F16>(xa, zop, zf);
                                    }
                                    if (last) {
                                        const float sc = record_scale<BITS, F16>(rg, r);
#pragma unroll
                                        for (int c = 0; c < MT; ++c)
                                            fold(yacc[c], gacc[c], zacc[c], sc);
                                    }
                                }
                            }
                        }
                    }
                    if (first && j == 0 && more)
                        stage_load(nxt);
                    // refill the slot with the tile D ahead, across chunk
                    // boundaries (past the range: dropped, never used);
                    // issued on every path
                    load_codes<BITS>(ring[j], cr, lane_off + (uint32_t)(t + D) * TB);
                }
        };
        group(c0, true);
        for (int i = c0 + D; i < c1; i += D)
            group(i, false);
        if (more)
            stage_store(nxt, cc + 1); // the buffer was last read in chunk cc - 1
        __syncthreads();
        cur = nxt;
    }

    // ---- outputs straight from the accumulators (C layout: lane holds rows
    //      16 c + 4 o + e of column r); with K split, fp32 partials, stored
    //      non-temporally: the summing kernel reads them on other XCDs, so
    //      they need not stay in this XCD's L2
    if constexpr (ACT != kActSiluMul) {
        if (blk_ok) {
            const int64_t nn = blk * kBlockCols + r;
            if (nn < lay.N) {
#pragma unroll
                for (int c = 0; c < MT; ++c)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = 16 * c + 4 * o + e;
                        if (row < M) {
                            if (gridDim.y > 1)
                                __builtin_nontemporal_store(yacc[c][e], ws + ((int64_t)split * M + row) * lay.N + nn);
                            else
                                y[(int64_t)row * lay.N + nn] = f32_to_half_bits<F16>(yacc[c][e]);
                        }
                    }
            }
        }
    } else if (blk_ok) { // blk_ok is uniform over the wave; N % 16 == 0: every column exists
        const int64_t nn = blk * kBlockCols + r, n2 = lay.N >> 1;
#pragma unroll
        for (int c = 0; c < MT; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * c + 4 * o + e;
                const float u = __shfl_xor(yacc[c][e], kBlockCols / 2); // lane r + 8: the up column
                if (row < M) {
                    if (gridDim.y > 1)
                        __builtin_nontemporal_store(yacc[c][e], ws + ((int64_t)split * M + row) * lay.N + nn);
                    else if (r < kBlockCols / 2)
                        y[(int64_t)row * n2 + blk * (kBlockCols / 2) + r] = f32_to_bf16_bits(silu(yacc[c][e]) * u);
                }
            }
    }
}

// Sum of a SiLU-product launch's K ranges: y[m][8 j + c] = silu(g) * u, g
// and u the in-order sums of the ranges' partials of columns 16 j + c and
// 16 j + c + 8.  One thread per output.
__global__ __launch_bounds__(256) void splitk_sum_silu_kernel(const float *__restrict__ ws, int splits, int64_t M,
                                                              int64_t N, uint16_t *__restrict__ y)
{
    const int64_t n2 = N >> 1;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= M * n2)
        return;
    const int64_t m = i / n2, h = i - m * n2;
    const int64_t col = (h >> 3) * kBlockCols + (h & 7);
    float g = 0.f, u = 0.f;
    for (int s = 0; s < splits; ++s) {
        const float *row = ws + ((int64_t)s * M + m) * N;
        g += __builtin_nontemporal_load(row + col);
        u += __builtin_nontemporal_load(row + col + kBlockCols / 2);
    }
    y[i] = f32_to_bf16_bits(silu(g) * u);
}

// Blocks per workgroup: one at M = 1 (x is small); with several activation
// rows, x is M times larger and every workgroup stages all of it, so wide
// layers give each workgroup up to four blocks (still at least 256
// workgroups) and stage x once for all of them.
static int gemv_bpw(const Layout &lay, int64_t M)
{
    if (M < 2)
        return 1;
    int64_t b = lay.nblocks / 256;
    return b >= 4 ? 4 : b >= 2 ? 2 : 1;
}

int gemv_waves(const Layout &lay, int64_t M)
{
    const int bpw = gemv_bpw(lay, M);
    const int64_t wgs = (lay.nblocks + bpw - 1) / bpw;
    int64_t wb = ((kGemvTargetWaves + wgs - 1) / wgs + bpw - 1) / bpw; // waves per block
    if (wb * bpw > kGemvMaxWaves)
        wb = kGemvMaxWaves / bpw;
    if (wb > lay.ktiles)
        wb = lay.ktiles;
    return (int)(wb < 1 ? 1 : wb) * bpw;
}

// Chunk size: as many k-tiles as fit the LDS share of one workgroup when
// 16 / W workgroups run per CU (at most kGemvMaxLds).
constexpr int kGemvMaxLds = 156 * 1024;
static GemvChunks plan_chunks(int bits, const Layout &lay, int64_t M, int W, int bpw)
{
    const int RB = record_bytes(bits);
    int wgs = kGemvMaxWaves / W;
    wgs = wgs < 1 ? 1 : wgs;
    int64_t budget = (160 * 1024) / wgs - 1024;
    if (budget > kGemvMaxLds)
        budget = kGemvMaxLds;
    const int64_t recs_per_tile = lay.whole_tiles() ? 1 : lay.groups_per_tile;
    const int64_t per_tile = M * kTileRows * 2 + bpw * recs_per_tile * RB;
    int64_t tiles = (budget - bpw * (2 * RB + 16) - 16 * M) / per_tile;
    if (tiles > lay.ktiles)
        tiles = lay.ktiles;
    if (tiles < 1)
        tiles = 1;
    GemvChunks c;
    c.bpw = bpw;
    c.tiles = (int)tiles;
    c.xpitch = (int)(tiles * kTileRows + 8);
    // records of a chunk: groups g0..g1 of its rows, at most tiles * recs_per_tile + 1
    c.meta_cap = (int)(((tiles * recs_per_tile + 1) * RB + 15) / 16 * 16);
    int64_t lds = (int64_t)bpw * c.meta_cap + M * c.xpitch * 2;
    const int64_t red = (int64_t)W * 16 * kBlockCols * 4;
    c.lds = (int)(lds > red ? lds : red);
    return c;
}

// Dynamic LDS above the default 64 KiB needs the limit raised, once per
// instantiation.
template <int BITS, int kMode, int D, int BPW, int ACT>
static void launch_gemv_mode(const Layout &lay, dim3 grid, dim3 block, const GemvChunks &ch, hipStream_t stream,
                             const uint16_t *x, const uint8_t *pk, uint16_t *y, int M)
{
    auto kern = &gemv_kernel<BITS, kMode, D, BPW, ACT>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kGemvMaxLds);
    (void)attr;
    kern<<<grid, block, ch.lds, stream>>>(x, pk, y, lay, M, ch);
}

template <int BITS, int D, int BPW, int ACT>
static void launch_gemv_bpw(const Layout &lay, dim3 grid, dim3 block, const GemvChunks &ch, hipStream_t stream,
                            const uint16_t *x, const uint8_t *pk, uint16_t *y, int M)
{
    if (lay.tiles_per_group == 1)
        launch_gemv_mode<BITS, kOneTile, D, BPW, ACT>(lay, grid, block, ch, stream, x, pk, y, M);
    else if (lay.whole_tiles())
        launch_gemv_mode<BITS, kMultiTile, D, BPW, ACT>(lay, grid, block, ch, stream, x, pk, y, M);
    else
        launch_gemv_mode<BITS, kSplitTiles, D, BPW, ACT>(lay, grid, block, ch, stream, x, pk, y, M);
}

template <int BITS, int D, int ACT>
static void launch_gemv_depth(const Layout &lay, dim3 grid, dim3 block, const GemvChunks &ch, hipStream_t stream,
                              const uint16_t *x, const uint8_t *pk, uint16_t *y, int M)
{
    if (ch.bpw == 4)
        launch_gemv_bpw<BITS, D, 4, ACT>(lay, grid, block, ch, stream, x, pk, y, M);
    else if (ch.bpw == 2)
        launch_gemv_bpw<BITS, D, 2, ACT>(lay, grid, block, ch, stream, x, pk, y, M);
    else
        launch_gemv_bpw<BITS, D, 1, ACT>(lay, grid, block, ch, stream, x, pk, y, M);
}

// Prefetch depth: measured on MI355X, two k-tiles in flight per wave suit
// short per-wave ranges (at most 3 tiles), four the longer ones; deeper rings
// only add redundant loads and registers.
template <int BITS, int ACT = kActNone>
static void launch_gemv_bits(const Layout &lay, dim3 grid, dim3 block, const GemvChunks &ch, hipStream_t stream,
                             const uint16_t *x, const uint8_t *pk, uint16_t *y, int M)
{
    const int64_t per_wave = lay.ktiles / (block.x / 64 / ch.bpw);
    if (per_wave <= 3)
        launch_gemv_depth<BITS, 2, ACT>(lay, grid, block, ch, stream, x, pk, y, M);
    else
        launch_gemv_depth<BITS, 4, ACT>(lay, grid, block, ch, stream, x, pk, y, M);
}

// ---- launch of the 16-row-chunk GEMV ----

static int mid_mt(int64_t M) { return M <= 16 ? 1 : M <= 32 ? 2 : 4; }

// K ranges over workgroups of the 16-row-chunk kernel.  One workgroup runs per compute
// unit (its LDS and registers), so a launch takes ceil(groups * s / cus)
// rounds of ceil(ktiles / s) k-tiles each plus a fixed cost per round
// (staging the first chunk, the outputs: about kMidRoundTiles k-tiles); a
// split adds the summing launch, about as long as kMidSumTiles k-tiles.  The
// split count minimises that, from 1 to kGemvMaxSplits ranges of at least
// kGemvMinSplitTiles k-tiles.  (Measured on MI355X.)
constexpr int64_t kMidRoundTiles = 4;
constexpr int64_t kMidSumTiles = 8;
static int64_t mid_splits(const Layout &lay, int cus, int64_t *split_tiles)
{
    const int64_t groups = (lay.nblocks + kMidWaves - 1) / kMidWaves;
    auto cost = [&](int64_t s) {
        const int64_t st = (lay.ktiles + s - 1) / s;
        return (groups * s + cus - 1) / cus * (st + kMidRoundTiles) + (s > 1 ? kMidSumTiles : 0);
    };
    int64_t best = 1;
    for (int64_t s = 2; s <= kGemvMaxSplits && (lay.ktiles + s - 1) / s >= kGemvMinSplitTiles; ++s)
        if (cost(s) < cost(best))
            best = s;
    const int64_t st = (lay.ktiles + best - 1) / best;
    if (split_tiles)
        *split_tiles = st;
    return (lay.ktiles + st - 1) / st;
}

// Which kernel a call of M rows runs.  Above 16 rows, the 16-row-chunk
// kernel.  Below, it is faster where it needs no K split (a layer wide
// enough to fill the chip) from 2 rows, and where it splits K from 8 rows
// if its ranges hold at least kMidMinRangeTiles k-tiles; elsewhere the
// summing launch outweighs the gain and the kernel for up to 16 rows, which
// splits K inside a workgroup, is kept.  At M = 1 that kernel is always the
// faster.  Measured on the decoder layer: gate_up (no split) 18.6 -> 17.3 us
// at M = 2; down (8 ranges of 14 k-tiles) 16.2 -> 14.5 us at M = 8; q/k/v (5
// ranges of 7) 12.3 -> 9.8 us at M = 10; o (8 ranges of 4) slower at every
// M up to 16.
constexpr int64_t kMidSplitFromRows = 8;
constexpr int64_t kMidMinRangeTiles = 6;
static bool use_mid(const Layout &lay, int64_t M, int cus)
{
    if (M > 16)
        return true;
    if (M < 2)
        return false;
    int64_t st = 0;
    if (mid_splits(lay, cus, &st) == 1)
        return true;
    return M >= kMidSplitFromRows && st >= kMidMinRangeTiles;
}

int64_t gemv_splits(const Layout &lay, int64_t M, int cus, int64_t *split_tiles)
{
    if (use_mid(lay, M, cus))
        return mid_splits(lay, cus, split_tiles);
    if (split_tiles)
        *split_tiles = lay.ktiles;
    return 1;
}

int64_t gemv_workspace_bytes(const Layout &lay, int64_t M, int cus)
{
    const int64_t s = gemv_splits(lay, M, cus, nullptr);
    return s > 1 ? s * M * lay.N * (int64_t)sizeof(float) : 0;
}

// Chunk: as many k-tiles as the threads' staging registers hold for M rows
// (16 M units of 16 bytes per k-tile), rounded down to a multiple of the
// ring depth (8 when that leaves at least 8, else 4), and whose records fit
// the record registers; two such chunks of activations take at most
// 2 * 64 * 4 * 128 * 2 bytes = 130 KiB of LDS.
static int64_t mid_xunits(int64_t M) { return (int64_t)mid_xregs(mid_mt(M)) * 64 * kMidWaves; }
static int mid_depth(int64_t M) { return mid_xunits(M) / (16 * M) >= 8 ? 8 : 4; }

static MidChunks plan_mid(int bits, const Layout &lay, int64_t M, int64_t split_tiles)
{
    const int RB = record_bytes(bits);
    const int D = mid_depth(M);
    const int64_t gpt = lay.whole_tiles() ? 1 : lay.groups_per_tile;
    int64_t t = mid_xunits(M) / (16 * M);
    t = t / D * D;
    while (t > D && kMidWaves * ((t * gpt + 1) * RB / 8) > kMidRecRegs * 64 * kMidWaves)
        t -= D;
    const int64_t span = (split_tiles + D - 1) / D * D;
    if (t > span)
        t = span;
    MidChunks c;
    c.tiles = (int)t;
    c.xpitch = (int)(t * kTileRows + 8);
    c.meta_cap = (int)(((t * gpt + 1) * RB + 15) / 16 * 16);
    c.lds = (int)(2 * (int64_t)kMidWaves * c.meta_cap + 2 * M * c.xpitch * 2);
    c.split_tiles = (int)split_tiles;
    return c;
}

template <int BITS, int kMode, int MT, int D, int ACT>
static void launch_mid_mode(dim3 grid, const MidChunks &ch, hipStream_t stream, const uint16_t *x,
                            const uint8_t *pk, uint16_t *y, const Layout &lay, int M, float *ws)
{
    auto kern = &gemv_mid_kernel<BITS, kMode, MT, D, ACT>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kGemvMaxLds);
    (void)attr;
    kern<<<grid, 64 * kMidWaves, ch.lds, stream>>>(x, pk, y, lay, M, ch, ws);
}

template <int BITS, int MT, int D, int ACT>
static void launch_mid_mt(dim3 grid, const MidChunks &ch, hipStream_t stream, const uint16_t *x, const uint8_t *pk,
                          uint16_t *y, const Layout &lay, int M, float *ws)
{
    if (lay.tiles_per_group == 1)
        launch_mid_mode<BITS, kOneTile, MT, D, ACT>(grid, ch, stream, x, pk, y, lay, M, ws);
    else if (lay.whole_tiles())
        launch_mid_mode<BITS, kMultiTile, MT, D, ACT>(grid, ch, stream, x, pk, y, lay, M, ws);
    else
        launch_mid_mode<BITS, kSplitTiles, MT, D, ACT>(grid, ch, stream, x, pk, y, lay, M, ws);
}

template <int BITS, int ACT>
static void launch_mid_bits(dim3 grid, const MidChunks &ch, hipStream_t stream, const uint16_t *x, const uint8_t *pk,
                            uint16_t *y, const Layout &lay, int M, float *ws)
{
    // M <= 16: one row chunk, M <= 32: two, depth 8; above: four, depth 4
    if (mid_mt(M) == 1)
        launch_mid_mt<BITS, 1, 8, ACT>(grid, ch, stream, x, pk, y, lay, M, ws);
    else if (mid_mt(M) == 2)
        launch_mid_mt<BITS, 2, 8, ACT>(grid, ch, stream, x, pk, y, lay, M, ws);
    else
        launch_mid_mt<BITS, 4, 4, ACT>(grid, ch, stream, x, pk, y, lay, M, ws);
}

// Most 8-byte record words one chunk of `tiles` k-tiles touches in a block:
// the groups from the chunk's first row to its last.  A chunk starting
// mid-group touches one group more than its k-tiles alone would hold.
static int64_t mid_max_rec_words(int bits, const Layout &lay, int64_t tiles)
{
    const int64_t gpt = lay.whole_tiles() ? 1 : lay.groups_per_tile;
    return (tiles * gpt + 1) * record_bytes(bits) / 8;
}

// The staging registers of gemv_mid_kernel hold kMidRecRegs words per
// thread: kMidRecRegs * 64 * kMidWaves over the workgroup's blocks.
constexpr int64_t kMidRecCapacity = (int64_t)kMidRecRegs * 64 * kMidWaves;

template <int ACT = kActNone>
static hipError_t launch_gemv_mid(int bits, const uint16_t *x, const uint8_t *pk, uint16_t *y, int64_t M,
                                  const Layout &lay, void *workspace, hipStream_t stream, int cus)
{
    int64_t split_tiles = 0;
    const int64_t splits = gemv_splits(lay, M, cus, &split_tiles);
    const MidChunks ch = plan_mid(bits, lay, M, split_tiles);
    // the kernel stages a chunk's activations with mid_xregs loads per
    // thread and its records with kMidRecRegs loads per thread, walks chunks
    // of ch.tiles > 0 k-tiles, and needs its LDS; a plan outside those
    // limits is refused rather than launched
    const int D = mid_depth(M);
    const int64_t rec_words = mid_max_rec_words(bits, lay, ch.tiles);
    if (ch.tiles < 1 || (ch.tiles % D != 0 && ch.tiles < split_tiles) ||
        M * ch.tiles * (kTileRows / 8) > mid_xunits(M) || ch.lds > kGemvMaxLds ||
        kMidWaves * rec_words > kMidRecCapacity || 8 * rec_words > ch.meta_cap)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)((lay.nblocks + kMidWaves - 1) / kMidWaves), (unsigned)splits);
    float *ws = splits > 1 ? static_cast<float *>(workspace) : nullptr;
    if (bits == 4)
        launch_mid_bits<4, ACT>(grid, ch, stream, x, pk, y, lay, (int)M, ws);
    else
        launch_mid_bits<8, ACT>(grid, ch, stream, x, pk, y, lay, (int)M, ws);
    if (splits > 1) {
        if constexpr (ACT != kActSiluMul)
            launch_splitk_sum(ws, (int)splits, M * lay.N, y, stream, ACT == kActF16);
        else
            launch_splitk_sum_silu(ws, (int)splits, M, lay.N, y, stream);
    }
    return hipGetLastError();
}

GemvPlanInfo gemv_plan_info(int bits, const Layout &lay, int64_t M, int cus)
{
    GemvPlanInfo p{};
    p.lds_limit = kGemvMaxLds;
    if (use_mid(lay, M, cus)) {
        int64_t st = 0;
        p.kernel = 1;
        p.splits = gemv_splits(lay, M, cus, &st);
        p.split_tiles = st;
        const MidChunks ch = plan_mid(bits, lay, M, st);
        p.waves = kMidWaves;
        p.bpw = kMidWaves;
        p.chunk_tiles = ch.tiles;
        p.depth = mid_depth(M);
        p.row_chunks = mid_mt(M);
        p.lds = ch.lds;
        p.x_capacity = mid_xunits(M);
        p.rec_capacity = kMidRecCapacity;
        p.meta_cap = ch.meta_cap;
        p.xpitch = ch.xpitch;
        return p;
    }
    const int W = gemv_waves(lay, M);
    const int bpw = gemv_bpw(lay, M);
    const GemvChunks ch = plan_chunks(bits, lay, M, W, bpw);
    p.kernel = 0;
    p.waves = W;
    p.bpw = bpw;
    p.splits = 1;
    p.split_tiles = lay.ktiles;
    p.chunk_tiles = ch.tiles;
    p.depth = lay.ktiles / (W / bpw) <= 3 ? 2 : 4;
    p.row_chunks = 1;
    p.lds = ch.lds;
    p.x_capacity = 0; // staged by a loop: no fixed capacity
    p.rec_capacity = 0;
    p.meta_cap = ch.meta_cap;
    p.xpitch = ch.xpitch;
    return p;
}

template <int ACT>
static hipError_t launch_gemv_plain(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M,
                                    const Layout &lay, void *workspace, hipStream_t stream, int cus)
{
    const uint8_t *pk = static_cast<const uint8_t *>(packed);
    if (use_mid(lay, M, cus))
        return launch_gemv_mid<ACT>(bits, x, pk, y, M, lay, workspace, stream, cus);
    const int W = gemv_waves(lay, M);
    const int bpw = gemv_bpw(lay, M);
    const GemvChunks ch = plan_chunks(bits, lay, M, W, bpw);
    if (ch.tiles < 1 || ch.lds > kGemvMaxLds)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)((lay.nblocks + bpw - 1) / bpw)), block(64 * W);
    if (bits == 4)
        launch_gemv_bits<4, ACT>(lay, grid, block, ch, stream, x, pk, y, (int)M);
    else
        launch_gemv_bits<8, ACT>(lay, grid, block, ch, stream, x, pk, y, (int)M);
    return hipGetLastError();
}

hipError_t launch_gemv(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M, const Layout &lay,
                       void *workspace, hipStream_t stream, int cus, bool f16)
{
    if (f16)
        return launch_gemv_plain<kActF16>(bits, x, packed, y, M, lay, workspace, stream, cus);
    return launch_gemv_plain<kActNone>(bits, x, packed, y, M, lay, workspace, stream, cus);
}

void launch_splitk_sum_silu(const float *ws, int splits, int64_t M, int64_t N, uint16_t *y, hipStream_t stream)
{
    splitk_sum_silu_kernel<<<(unsigned)((M * (N / 2) + 255) / 256), 256, 0, stream>>>(ws, splits, M, N, y);
}

// The gate/up GEMV with the SiLU product: the kernel the plain GEMV of the
// same shape runs, on its grid (each block pairs its own columns).
hipError_t launch_gemv_silu_mul(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M,
                                const Layout &lay, void *workspace, hipStream_t stream, int cus)
{
    if (lay.N % kBlockCols || M < 1 || M > kGemvKernelMaxM)
        return hipErrorInvalidValue;
    if (use_mid(lay, M, cus))
        return launch_gemv_mid<kActSiluMul>(bits, x, static_cast<const uint8_t *>(packed), y, M, lay, workspace,
                                            stream, cus);
    const int W = gemv_waves(lay, M);
    const int bpw = gemv_bpw(lay, M);
    const GemvChunks ch = plan_chunks(bits, lay, M, W, bpw);
    if (ch.tiles < 1 || ch.lds > kGemvMaxLds)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)((lay.nblocks + bpw - 1) / bpw)), block(64 * W);
    const uint8_t *pk = static_cast<const uint8_t *>(packed);
    if (bits == 4)
        launch_gemv_bits<4, kActSiluMul>(lay, grid, block, ch, stream, x, pk, y, (int)M);
    else
        launch_gemv_bits<8, kActSiluMul>(lay, grid, block, ch, stream, x, pk, y, (int)M);
    return hipGetLastError();
}

} // namespace tf
