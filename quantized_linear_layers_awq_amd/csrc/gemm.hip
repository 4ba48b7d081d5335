// Prefill GEMM with fused dequantization (TileFuse summary, Methodology
// section 1: unpack and dequantize each weight tile once, keep the result in
// core-local memory and reuse it for the following matrix operations).
//
// MI355X design.  A workgroup owns a BM x BN output tile.  Per K-batch of 128
// rows it stages the activation tile [BM][128] in LDS and unpacks the packed
// weight tile once into LDS as bf16 (q - z) -- exact, since |q - z| <= 255 has
// at most 8 significant bits -- laid out [BN][128] (k contiguous per column,
// the 16x16x32 MFMA B operand a lane reads).  All BM rows reuse that tile
// through bf16 MFMAs; each group's products accumulate in fp32 and the group's
// bf16 scale is folded in once per (group, column):
//     y += s[g][n] * sum_{k in g} x[m][k] * (q[k][n] - z[g][n])
// i.e. the definition with the per-group factor taken out of the sum.  (A
// bf16 copy of (q - z) * s would round every weight to 8 significant bits,
// an error the elementwise output bound does not absorb.)  No dequantized
// weight leaves LDS.
#include "tf_common.h"
#include "tf_launch.h"

namespace tf {

constexpr int kGemmBM = 128;
constexpr int kGemmBN = 128;         // eight packed 16-column blocks
constexpr int kGemmBK = kTileRows;   // one k-tile (four 32-row steps) per stage
constexpr int kGemmLd = kGemmBK + 8; // LDS row pitch in bf16 (pad: spreads 16 rows over the banks)

template <int BITS, bool kWhole>
__global__ __launch_bounds__(256) void gemm_kernel(const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed,
                                                   uint16_t *__restrict__ y, Layout lay, int64_t M, int64_t m_tiles)
{
    __shared__ __attribute__((aligned(16))) uint16_t sA[kGemmBM * kGemmLd];
    __shared__ __attribute__((aligned(16))) uint16_t sB[kGemmBN * kGemmLd];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int o = lane >> 4, r = lane & 15;
    // consecutive workgroups share a weight tile (column tile outer)
    const int64_t nt = blockIdx.x / m_tiles;
    const int64_t mt = blockIdx.x - nt * m_tiles;
    const int64_t m0 = mt * kGemmBM;
    const int64_t blk0 = nt * (kGemmBN / kBlockCols);
    const uint32_t spg = (uint32_t)(lay.G / kStepRows);
    constexpr int RB = record_bytes(BITS);
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    const f32x4 zf = {0.f, 0.f, 0.f, 0.f};

    f32x4 yacc[4][4], gacc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            yacc[i][j] = gacc[i][j] = zf;

    for (int64_t t = 0; t < lay.ktiles; ++t) {
        // ---- activations: 128 rows x 256 bytes, 16 bytes per thread x 8 ----
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int idx = tid + 256 * it;
            const int row = idx >> 4, c16 = idx & 15;
            const int64_t gm = m0 + row;
            const int64_t k = t * kTileRows + 8 * c16;
            u32x4 v = zero4;
            if (gm < M && k < lay.K)
                v = load16(x + gm * lay.K + k);
            *reinterpret_cast<u32x4 *>(&sA[row * kGemmLd + 8 * c16]) = v;
        }
        // ---- weights: unpack each 16-byte unit of codes once into LDS as the
        //      exact bf16 values q - z.  Units map wave-uniformly to blocks. ----
        constexpr int kUnitIters = BITS == 4 ? 2 : 4;
#pragma unroll
        for (int it = 0; it < kUnitIters; ++it) {
            const int bb = BITS == 4 ? wave + 4 * it : (wave + 4 * it) >> 1;
            const int h = BITS == 4 ? 0 : wave & 1;
            const int64_t blk = blk0 + bb;
            constexpr int kSteps = BITS == 4 ? 4 : 2;
            const int nl = kBlockCols * bb + r;
            if (blk < lay.nblocks) {
                const uint8_t *meta = packed + blk * lay.block_bytes;
                const u32x4 cw = load16(meta + lay.meta_bytes + t * tile_bytes(BITS) + 1024 * h + 16 * lane);
                uint32_t zt = 0;
                if constexpr (kWhole)
                    zt = record_zero<BITS>(meta + (int64_t)((uint32_t)t / (uint32_t)lay.tiles_per_group) * RB, r);
#pragma unroll
                for (int uu = 0; uu < kSteps; ++uu) {
                    const int u = BITS == 4 ? uu : 2 * h + uu;
                    const int64_t s = 4 * t + u;
                    u32x4 bf = zero4;
                    if (s < lay.steps) {
                        uint32_t z = zt;
                        if constexpr (!kWhole)
                            z = record_zero<BITS>(meta + (int64_t)((uint32_t)s / spg) * RB, r);
                        float f[8];
                        if constexpr (BITS == 4)
                            dequant_w4_word(cw[u], 1.f, -(float)z, f);
                        else
                            dequant_w8_pair(cw[2 * uu], cw[2 * uu + 1], 1.f, -(float)z, f);
                        bf = u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                                   pack_bf16x2(f[6], f[7])};
                    }
                    *reinterpret_cast<u32x4 *>(&sB[nl * kGemmLd + kStepRows * u + 8 * o]) = bf;
                }
            } else {
#pragma unroll
                for (int uu = 0; uu < kSteps; ++uu) {
                    const int u = BITS == 4 ? uu : 2 * h + uu;
                    *reinterpret_cast<u32x4 *>(&sB[nl * kGemmLd + kStepRows * u + 8 * o]) = zero4;
                }
            }
        }
        // ---- scales of the groups that end inside this k-tile: this wave's
        //      column j sits in block blk0 + 4 wn + j, column r ----
        float scv[4][4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int64_t s = 4 * t + kk;
            const bool ends = s < lay.steps && ((uint32_t)s + 1) % spg == 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t blk = blk0 + 4 * wn + j;
                scv[kk][j] = 0.f;
                if (ends && blk < lay.nblocks)
                    scv[kk][j] = record_scale<BITS>(
                        packed + blk * lay.block_bytes + (int64_t)((uint32_t)s / spg) * RB, r);
            }
        }
        __syncthreads();

        // ---- MFMA: each wave a 64 x 64 sub-tile, 4 x 4 MFMA tiles ----
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int64_t s = 4 * t + kk;
            if (s >= lay.steps)
                break;
            u32x4 a[4], b[4];
            const int kof = kStepRows * kk + 8 * o;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *reinterpret_cast<const u32x4 *>(&sA[(64 * wm + 16 * i + r) * kGemmLd + kof]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *reinterpret_cast<const u32x4 *>(&sB[(64 * wn + 16 * j + r) * kGemmLd + kof]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    gacc[i][j] = mfma16x16x32(a[i], b[j], gacc[i][j]);
            if (((uint32_t)s + 1) % spg == 0) {
                // group end: y += s[g][n] * (this group's sum), once per element
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            yacc[i][j][e] = fmaf(scv[kk][j], gacc[i][j][e], yacc[i][j][e]);
                        gacc[i][j] = zf;
                    }
            }
        }
        __syncthreads();
    }

    // ---- epilogue: fp32 -> bf16 (nearest even), masked to M x N ----
    const int64_t n0 = nt * kGemmBN;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = m0 + 64 * wm + 16 * i + 4 * o + e;
                const int64_t col = n0 + 64 * wn + 16 * j + r;
                if (row < M && col < lay.N)
                    y[row * lay.N + col] = f32_to_bf16_bits(yacc[i][j][e]);
            }
}

hipError_t launch_gemm(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M, const Layout &lay,
                       hipStream_t stream)
{
    const int64_t m_tiles = (M + kGemmBM - 1) / kGemmBM;
    const int64_t n_tiles = (lay.N + kGemmBN - 1) / kGemmBN;
    const dim3 grid((unsigned)(m_tiles * n_tiles));
    const uint8_t *pk = static_cast<const uint8_t *>(packed);
    const bool whole = lay.whole_tiles();
    if (bits == 4) {
        if (whole)
            gemm_kernel<4, true><<<grid, 256, 0, stream>>>(x, pk, y, lay, M, m_tiles);
        else
            gemm_kernel<4, false><<<grid, 256, 0, stream>>>(x, pk, y, lay, M, m_tiles);
    } else {
        if (whole)
            gemm_kernel<8, true><<<grid, 256, 0, stream>>>(x, pk, y, lay, M, m_tiles);
        else
            gemm_kernel<8, false><<<grid, 256, 0, stream>>>(x, pk, y, lay, M, m_tiles);
    }
    return hipGetLastError();
}

} // namespace tf
