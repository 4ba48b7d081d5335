// Host-side launchers of the kernels; called by the C ABI after validation.
#pragma once

#include "tf_common.h"

namespace tf {

// pair_half = 0: the checkpoint's columns in order.  pair_half = N/2 (a
// multiple of 8): a [gate | up] checkpoint, packed so that column c of block
// j is gate column 8 j + c (c < 8) or up column 8 j + c - 8 (c >= 8).
hipError_t launch_repack(int bits, const void *qweight, const void *qzeros, const uint16_t *scales,
                         const Layout &lay, void *packed, hipStream_t stream, int64_t pair_half = 0);
// The fp32 weights (q - z) * s decoded from a packed buffer by the GEMM's
// operand builder (gemv = false: exact bf16 q - z, times s) or the GEMV's
// (gemv = true: bf16 128 + q and 128 + z for W4, q and z for W8, their
// difference times s).
hipError_t launch_dequant_f32(int bits, const void *packed, const Layout &lay, float *w, hipStream_t stream,
                              bool gemv);

// Waves per GEMV workgroup for M <= 16 activation rows (one workgroup per
// 16-column block, or per two or four blocks of a wide layer at M >= 2).
int gemv_waves(const Layout &lay, int64_t M);
// K ranges the GEMV splits over workgroups (the 16-row-chunk kernel, which
// runs above 16 rows, from 2 rows where it needs no split and from 8 where
// its K ranges are long enough, on a layer too narrow to fill `cus` compute
// units; 1 otherwise) and k-tiles per range.
int64_t gemv_splits(const Layout &lay, int64_t M, int cus, int64_t *split_tiles);
// The GEMV launch plan a call of (bits, M) rows would run on `cus` compute
// units, for host-side checks of its invariants (no GPU work):
struct GemvPlanInfo {
    int64_t kernel;       // 0: the kernel for up to 16 rows, 1: the 16-row-chunk kernel
    int64_t waves;        // waves per workgroup
    int64_t bpw;          // 16-column blocks per workgroup
    int64_t splits;       // K ranges over workgroups
    int64_t split_tiles;  // k-tiles per range
    int64_t chunk_tiles;  // k-tiles per staged chunk
    int64_t depth;        // code loads in flight per wave (k-tiles)
    int64_t row_chunks;   // 16-row chunks per wave (kernel 1)
    int64_t lds;          // dynamic LDS bytes per workgroup
    int64_t lds_limit;    // the most the launcher allows
    int64_t x_capacity;   // 16-byte activation units one staging pass holds (kernel 1)
    int64_t rec_capacity; // 8-byte record words one staging pass holds over all blocks (kernel 1)
    int64_t meta_cap;     // bytes reserved per block for a chunk's records
    int64_t xpitch;       // bf16 elements per staged activation row
};
GemvPlanInfo gemv_plan_info(int bits, const Layout &lay, int64_t M, int cus);
// Workspace bytes of a GEMV launch: fp32 partial sums when it splits K.
int64_t gemv_workspace_bytes(const Layout &lay, int64_t M, int cus);
// Largest M the GEMV kernel takes (16-row chunks, up to four per wave).
constexpr int64_t kGemvKernelMaxM = 64;
// f16: x, the scales in the packed records and y are IEEE fp16 (else bf16).
hipError_t launch_gemv(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M, const Layout &lay,
                       void *workspace, hipStream_t stream, int cus, bool f16 = false);
// y[m][8 j + c] = silu(g) * u with g, u the fp32 sums of columns c and c + 8
// of block j of a [gate | up] layer packed with pair_half = N/2 (N % 16 ==
// 0), 1 <= M <= kGemvKernelMaxM; y is [M][N/2].  Same kernel choice, and so
// the same workspace (gemv_workspace_bytes), as launch_gemv of that shape.
hipError_t launch_gemv_silu_mul(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M,
                                const Layout &lay, void *workspace, hipStream_t stream, int cus);
// Sum of a SiLU-product launch's K ranges: y[m][8 j + c] = silu(g) * u from
// the in-order sums of the partials ws[s][m][16 j + c] and ws[s][m][16 j + c + 8].
void launch_splitk_sum_silu(const float *ws, int splits, int64_t M, int64_t N, uint16_t *y, hipStream_t stream);
// y = bf16 (fp16 when f16) of the sum of the splits' fp32 partials
// ws[s][mn], added in split order; 2 <= splits <= 16 (both plans stay within
// that).
void launch_splitk_sum(const float *ws, int splits, int64_t mn, uint16_t *y, hipStream_t stream, bool f16 = false);
// How the GEMM covers the output: m_tiles row tiles of `rows` rows (256, or
// 128 up to kShortTileMaxM rows), then wide_cols column tiles of col_tile
// columns from column 0 in one launch and (256 x 128 tiles only)
// narrow_cols tiles of 64 columns after them in a second one.  col_tile is
// 256 (the 256 x 256 kernel, gemm256.hip: W4 with groups of whole k-tiles,
// above kShortTileMaxM rows) or 128 (the kernel of gemm.hip).  With
// splits > 1 (small M), K is cut into ranges of split_tiles k-tiles that run
// in the same launch and write fp32 partial sums to the workspace.
constexpr int64_t kShortTileRows = 128;
constexpr int64_t kShortTileMaxM = 128;
struct GemmPlan {
    int64_t m_tiles, wide_cols, narrow_cols, splits, split_tiles, rows, col_tile;
};
// route: the automatic choice (kRouteAuto; kRouteGemv plans the same),
// kRouteTiled (256 x 256 tiles wherever they apply) or kRouteTiled128
// (256 x 128 tiles only)
GemmPlan plan_gemm(int bits, int64_t M, int64_t N, int64_t K, int64_t G, int cus, int route);
// Compute units of the current device (queried once per device and kept:
// the library's only process-wide state).
int device_cus();
// Workspace bytes of the tiled GEMM planned for `cus` compute units (0
// unless it splits K).
int64_t gemm_workspace_bytes(int bits, int64_t M, int64_t N, int64_t K, int64_t G, int cus, int route);
// Which kernel a GEMM call of M rows runs: the GEMV kernels (M <= 64: the
// tiled GEMM would compute 128- or 256-row tiles) or the tiled GEMM.  The
// route is an argument: kRouteAuto in every product call; the test hooks
// may pass kRouteTiled (the tiled GEMM at any M), kRouteGemv (the GEMV
// kernels up to 64 rows) or kRouteTiled128 (the tiled GEMM at any M, with
// 256 x 128 tiles only).
constexpr int kRouteAuto = 0, kRouteTiled = 1, kRouteGemv = 2, kRouteTiled128 = 3;
bool gemm_uses_gemv(int64_t M, int route);
// act = kActSiluMul: a [gate | up] layer packed with pair_half = N/2, y is
// [M][N/2] = silu(gate) * up (as launch_gemv_silu_mul); act = kActF16: x, the
// scales and y are fp16.
hipError_t launch_gemm(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M, const Layout &lay,
                       void *workspace, hipStream_t stream, int cus, int act = kActNone, int route = kRouteAuto);
// The 256 x 256 kernel for a plan with col_tile 256 (W4 or W8, groups of
// whole k-tiles); ws holds the split partials when plan.splits > 1.
hipError_t launch_gemm256(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M, const Layout &lay,
                          const GemmPlan &plan, float *ws, hipStream_t stream, int act);

// Measurement probes (not on the hot path).
hipError_t launch_probe_read(const void *buf, uint64_t bytes, uint32_t *sink, hipStream_t stream);
hipError_t launch_probe_mfma(int workgroups, int iters, float *sink, hipStream_t stream);
hipError_t launch_probe_block_read(int bits, const void *packed, const Layout &lay, int waves, int depth,
                                  uint32_t *sink, hipStream_t stream);
int64_t probe_mfma_flops(int workgroups, int iters);

} // namespace tf
