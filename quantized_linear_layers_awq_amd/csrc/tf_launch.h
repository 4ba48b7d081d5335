// Host-side launchers of the kernels; called by the C ABI after validation.
#pragma once

#include "tf_common.h"

namespace tf {

// pair_half = 0: the checkpoint's columns in order.  pair_half = N/2 (a
// multiple of 8): a [gate | up] checkpoint, packed so that column c of block
// j is gate column 8 j + c (c < 8) or up column 8 j + c - 8 (c >= 8).
hipError_t launch_repack(int bits, const void *qweight, const void *qzeros, const uint16_t *scales,
                         const Layout &lay, void *packed, hipStream_t stream, int64_t pair_half = 0);
hipError_t launch_dequant_f32(int bits, const void *packed, const Layout &lay, float *w, hipStream_t stream);

// Waves per GEMV workgroup for M <= 16 activation rows (one workgroup per
// 16-column block, or per two or four blocks of a wide layer at M >= 2).
int gemv_waves(const Layout &lay, int64_t M);
// K ranges the GEMV splits over workgroups (the 16-row-chunk kernel, which
// runs above 16 rows, from 2 rows where it needs no split and from 8 where
// its K ranges are long enough, on a layer too narrow to fill `cus` compute
// units; 1 otherwise) and k-tiles per range.
int64_t gemv_splits(const Layout &lay, int64_t M, int cus, int64_t *split_tiles);
// Workspace bytes of a GEMV launch: fp32 partial sums when it splits K.
int64_t gemv_workspace_bytes(const Layout &lay, int64_t M, int cus);
// Largest M the GEMV kernel takes (16-row chunks, up to four per wave).
constexpr int64_t kGemvKernelMaxM = 64;
hipError_t launch_gemv(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M, const Layout &lay,
                       void *workspace, hipStream_t stream);
// Epilogue of the GEMV kernel: none, or silu(gate) * up over a [gate | up]
// layer (launch_gemv_silu_mul).
constexpr int kActNone = 0, kActSiluMul = 1;
// y[m][8 j + c] = silu(g) * u with g, u the fp32 sums of columns c and c + 8
// of block j of a [gate | up] layer packed with pair_half = N/2 (N % 16 ==
// 0), 1 <= M <= kGemvKernelMaxM; y is [M][N/2].  Same kernel choice, and so
// the same workspace (gemv_workspace_bytes), as launch_gemv of that shape.
hipError_t launch_gemv_silu_mul(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M,
                                const Layout &lay, void *workspace, hipStream_t stream);
// Sum of a SiLU-product launch's K ranges: y[m][8 j + c] = silu(g) * u from
// the in-order sums of the partials ws[s][m][16 j + c] and ws[s][m][16 j + c + 8].
void launch_splitk_sum_silu(const float *ws, int splits, int64_t M, int64_t N, uint16_t *y, hipStream_t stream);
// y = bf16(sum of the splits' fp32 partials ws[s][mn]), added in split order;
// 2 <= splits <= 16 (both plans stay within that).
void launch_splitk_sum(const float *ws, int splits, int64_t mn, uint16_t *y, hipStream_t stream);
// How the GEMM covers the output: m_tiles row tiles of `rows` rows (256, or
// 128 up to kShortTileMaxM rows), then wide_cols column tiles of 128 columns
// from column 0 in one launch and (256-row tiles only) narrow_cols tiles of
// 64 columns after them in a second one.  With splits > 1 (small M), K is
// cut into ranges of split_tiles k-tiles that run in the same launch and
// write fp32 partial sums to the workspace.
constexpr int64_t kShortTileRows = 128;
constexpr int64_t kShortTileMaxM = 128;
struct GemmPlan {
    int64_t m_tiles, wide_cols, narrow_cols, splits, split_tiles, rows;
};
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int64_t G, int cus);
// Compute units plan_gemm assumes: the forced count, else the device's.
int planning_cus();
// Force the compute units plan_gemm assumes (0: the current device's).
void set_planning_cus(int n);
// Workspace bytes of the tiled GEMM (0 unless it splits K).
int64_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t G);
// Which kernel a GEMM call of M rows runs: the GEMV kernel (M <= 64: the
// tiled GEMM would compute 256-row tiles) or the tiled GEMM.  The route can
// be forced for tests: 0 automatic, 1 tiled GEMM, 2 GEMV kernel where M <= 64.
bool gemm_uses_gemv(int64_t M);
void set_gemm_route(int route);
// act = kActSiluMul: a [gate | up] layer packed with pair_half = N/2, y is
// [M][N/2] = silu(gate) * up (as launch_gemv_silu_mul).
hipError_t launch_gemm(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M, const Layout &lay,
                       void *workspace, hipStream_t stream, int act = kActNone);

// Measurement probes (not on the hot path).
hipError_t launch_probe_read(const void *buf, uint64_t bytes, uint32_t *sink, hipStream_t stream);
hipError_t launch_probe_mfma(int workgroups, int iters, float *sink, hipStream_t stream);
int64_t probe_mfma_flops(int workgroups, int iters);

} // namespace tf
