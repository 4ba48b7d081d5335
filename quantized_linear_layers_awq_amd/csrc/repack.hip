// Offline interleaved pre-tiling (TileFuse summary, Methodology section 2) and
// the fp32 dequantization test hook.
//
// Repack is a copy-class gather: every thread writes one 16-byte unit of the
// packed layout (or one metadata record), so stores are coalesced and every
// byte of the layout, padding included, is written exactly once.  The
// checkpoint reads are gathers the caches absorb; this runs once per weight.
#include "tf_common.h"
#include "tf_launch.h"
#include "tf_operands.h"

namespace tf {

// Checkpoint column of packed column n: n itself, or, for a [gate | up]
// checkpoint packed for the SiLU-product GEMV (half = N/2, a multiple of 8),
// gate column 8 j + c for c = n % 16 < 8 of block j = n / 16 and up column
// 8 j + c - 8 for c >= 8.  Runs of eight columns stay runs of eight, so
// n % 8 (an AWQ word's nibble) is unchanged.
__device__ __forceinline__ int64_t source_col(int64_t n, int64_t half)
{
    return half == 0 ? n : ((n & 8) ? half : 0) + ((n >> 4) << 3) + (n & 7);
}

// ---------------------------------------------------------------------------
// Codes.  W4: 64 units of 16 bytes per k-tile (lane L = 16o + r: word u holds
// rows 32u + 8o .. +7 of column r).  W8: 128 units (half h = u / 2 at 1024h).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void repack_w4_codes(const uint32_t *__restrict__ qweight, Layout lay,
                                                       uint8_t *__restrict__ packed, int64_t units, int64_t half)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= units)
        return;
    const int L = (int)(idx & 63);
    const int64_t bt = idx >> 6; // blk * ktiles + t
    const int64_t blk = bt / lay.ktiles, t = bt - blk * lay.ktiles;
    const int o = L >> 4, r = L & 15;
    const int64_t n = blk * kBlockCols + r, sn = source_col(n, half);
    const int64_t words_per_row = lay.N / 8;
    u32x4 out = {0u, 0u, 0u, 0u};
    if (n < lay.N) {
        const uint32_t sh = awq_nibble_shift((int)(sn & 7));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint32_t wd = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t k = t * kTileRows + kStepRows * u + 8 * o + i;
                if (k < lay.K)
                    wd |= ((qweight[k * words_per_row + (sn >> 3)] >> sh) & 0xFu) << w4_row_shift(i);
            }
            out[u] = wd;
        }
    }
    *reinterpret_cast<u32x4 *>(packed + lay.tile(4, blk, t) + 16 * L) = out;
}

__global__ __launch_bounds__(256) void repack_w8_codes(const uint8_t *__restrict__ qweight, Layout lay,
                                                       uint8_t *__restrict__ packed, int64_t units, int64_t half)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= units)
        return;
    const int L = (int)(idx & 63);
    const int h = (int)((idx >> 6) & 1);
    const int64_t bt = idx >> 7;
    const int64_t blk = bt / lay.ktiles, t = bt - blk * lay.ktiles;
    const int o = L >> 4, r = L & 15;
    const int64_t n = blk * kBlockCols + r, sn = source_col(n, half);
    u32x4 out = {0u, 0u, 0u, 0u};
    if (n < lay.N) {
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
            const int u = 2 * h + uu;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t k = t * kTileRows + kStepRows * u + 8 * o + i;
                if (k < lay.K)
                    out[2 * uu + (i >> 2)] |= (uint32_t)qweight[k * lay.N + sn] << (8 * (i & 3));
            }
        }
    }
    *reinterpret_cast<u32x4 *>(packed + lay.tile(8, blk, t) + 1024 * h + 16 * L) = out;
}

// ---------------------------------------------------------------------------
// Metadata: one thread per (block, group) writes the whole record (16 scales,
// 16 zero points); the thread of a block's last group also zeroes the
// record region's padding.
// ---------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(256) void repack_records(const void *__restrict__ qzeros,
                                                      const uint16_t *__restrict__ scales, Layout lay,
                                                      uint8_t *__restrict__ packed, int64_t units, int64_t half)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= units)
        return;
    const int64_t blk = idx / lay.ngroups, g = idx - blk * lay.ngroups;
    uint32_t sc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t zz[4] = {0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < kBlockCols; ++c) {
        const int64_t n = blk * kBlockCols + c;
        if (n >= lay.N)
            continue;
        const int64_t sn = source_col(n, half);
        sc[c >> 1] |= (uint32_t)scales[g * lay.N + sn] << (16 * (c & 1));
        // no zero-point tensor: symmetric quantization, z = 2^(b-1)
        if constexpr (BITS == 4) {
            const uint32_t *qz = static_cast<const uint32_t *>(qzeros);
            const uint32_t z =
                qz ? (qz[g * (lay.N / 8) + (sn >> 3)] >> awq_nibble_shift((int)(sn & 7))) & 0xFu : 8u;
            zz[c >> 3] |= z << (4 * (c & 7));
        } else {
            const uint32_t z = qzeros ? static_cast<const uint8_t *>(qzeros)[g * lay.N + sn] : 128u;
            zz[c >> 2] |= z << (8 * (c & 3));
        }
    }
    uint8_t *rec = packed + lay.record(BITS, blk, g);
    // records start 8-byte aligned (W4, 40 bytes) or 16-byte aligned (W8, 48)
    u32x2 *p2 = reinterpret_cast<u32x2 *>(rec);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        p2[i] = u32x2{sc[2 * i], sc[2 * i + 1]};
    p2[4] = u32x2{zz[0], zz[1]};
    if constexpr (BITS == 8)
        p2[5] = u32x2{zz[2], zz[3]};
    if (g == lay.ngroups - 1) {
        uint8_t *end = rec + record_bytes(BITS);
        uint8_t *meta_end = packed + blk * lay.block_bytes + lay.meta_bytes;
        for (; end < meta_end; end += 8)
            *reinterpret_cast<u32x2 *>(end) = u32x2{0u, 0u};
    }
}

// ---------------------------------------------------------------------------
// Dequantization test hooks: w[k][n] = (q - z) * s in fp32, decoded by the
// kernels' own operand builders (tf_operands.h), so that a bit-exact match
// with the oracle pins the code the kernels run:
//   GEMV = false: the GEMM's unpack_w4 / unpack_w8, the exact bf16 q - z of
//                 its LDS weight tile, times s;
//   GEMV = true:  the GEMV's w4_operand / w8_operand and zero_operand (bf16
//                 128 + q and 128 + z, or q and z), their difference times s.
// Both products are exact in fp32 (at most 8 significant bits each).
// ---------------------------------------------------------------------------
template <int BITS, bool GEMV>
__global__ __launch_bounds__(256) void dequant_f32(const uint8_t *__restrict__ packed, Layout lay,
                                                   float *__restrict__ w, int64_t units)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= units)
        return;
    constexpr int kUnitsPerTile = BITS == 4 ? 64 : 128;
    const int L = (int)(idx & 63);
    const int h = BITS == 4 ? 0 : (int)((idx >> 6) & 1);
    const int64_t bt = idx / kUnitsPerTile;
    const int64_t blk = bt / lay.ktiles, t = bt - blk * lay.ktiles;
    const int o = L >> 4, r = L & 15;
    const int64_t n = blk * kBlockCols + r;
    if (n >= lay.N)
        return;
    const u32x4 cw = load16(packed + lay.tile(BITS, blk, t) + 1024 * h + 16 * L);
    const uint32_t magic = magic_in_vgpr();
    constexpr int kSteps = BITS == 4 ? 4 : 2;
#pragma unroll
    for (int uu = 0; uu < kSteps; ++uu) {
        const int u = BITS == 4 ? uu : 2 * h + uu;
        const int64_t k0 = t * kTileRows + kStepRows * u + 8 * o;
        if (k0 >= lay.K)
            continue;
        const uint8_t *rec = packed + lay.record(BITS, blk, k0 / lay.G);
        const float sv = record_scale<BITS>(rec, r);
        const uint32_t zq = record_zero<BITS>(rec, r);
        // eight rows of column n as bf16 pairs (rows 2i, 2i + 1 in word i)
        u32x4 op, zop = {0u, 0u, 0u, 0u};
        if constexpr (GEMV) {
            if constexpr (BITS == 4)
                op = w4_operand(cw[u], magic);
            else
                op = w8_operand(cw[2 * uu], cw[2 * uu + 1]);
            zop = zero_operand<BITS>(zq);
        } else {
            if constexpr (BITS == 4)
                op = unpack_w4(cw[u], 1.f, -(float)zq);
            else
                op = unpack_w8(cw[2 * uu], cw[2 * uu + 1], 1.f, -(float)zq);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t sh = 16u * (uint32_t)(i & 1);
            const float b = bf16_bits_to_f32((op[i >> 1] >> sh) & 0xFFFFu);
            const float d = GEMV ? b - bf16_bits_to_f32((zop[i >> 1] >> sh) & 0xFFFFu) : b;
            w[(k0 + i) * lay.N + n] = d * sv;
        }
    }
}

static inline unsigned grid_for(int64_t units) { return (unsigned)((units + 255) / 256); }

hipError_t launch_repack(int bits, const void *qweight, const void *qzeros, const uint16_t *scales,
                         const Layout &lay, void *packed, hipStream_t stream, int64_t pair_half)
{
    if (pair_half && (pair_half % 8 || 2 * pair_half != lay.N))
        return hipErrorInvalidValue;
    uint8_t *out = static_cast<uint8_t *>(packed);
    const int64_t code_units = lay.nblocks * lay.ktiles * (bits == 4 ? 64 : 128);
    const int64_t rec_units = lay.nblocks * lay.ngroups;
    if (bits == 4) {
        repack_w4_codes<<<grid_for(code_units), 256, 0, stream>>>(static_cast<const uint32_t *>(qweight), lay, out,
                                                                  code_units, pair_half);
        repack_records<4><<<grid_for(rec_units), 256, 0, stream>>>(qzeros, scales, lay, out, rec_units, pair_half);
    } else {
        repack_w8_codes<<<grid_for(code_units), 256, 0, stream>>>(static_cast<const uint8_t *>(qweight), lay, out,
                                                                  code_units, pair_half);
        repack_records<8><<<grid_for(rec_units), 256, 0, stream>>>(qzeros, scales, lay, out, rec_units, pair_half);
    }
    return hipGetLastError();
}

hipError_t launch_dequant_f32(int bits, const void *packed, const Layout &lay, float *w, hipStream_t stream,
                              bool gemv)
{
    const uint8_t *in = static_cast<const uint8_t *>(packed);
    const int64_t units = lay.nblocks * lay.ktiles * (bits == 4 ? 64 : 128);
    if (bits == 4) {
        if (gemv)
            dequant_f32<4, true><<<grid_for(units), 256, 0, stream>>>(in, lay, w, units);
        else
            dequant_f32<4, false><<<grid_for(units), 256, 0, stream>>>(in, lay, w, units);
    } else {
        if (gemv)
            dequant_f32<8, true><<<grid_for(units), 256, 0, stream>>>(in, lay, w, units);
        else
            dequant_f32<8, false><<<grid_for(units), 256, 0, stream>>>(in, lay, w, units);
    }
    return hipGetLastError();
}

} // namespace tf
