// Host-side launchers of the kernels; called by the C ABI after validation.
#pragma once

#include "tf_common.h"

namespace tf {

hipError_t launch_repack(int bits, const void *qweight, const void *qzeros, const uint16_t *scales,
                         const Layout &lay, void *packed, hipStream_t stream);
hipError_t launch_dequant_f32(int bits, const void *packed, const Layout &lay, float *w, hipStream_t stream);

// Waves per GEMV workgroup for M activation rows (one workgroup per 16-column
// block, or per two or four blocks of a wide layer at M >= 2).
int gemv_waves(const Layout &lay, int64_t M);
hipError_t launch_gemv(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M, const Layout &lay,
                       hipStream_t stream);
// How the GEMM covers the output: m_tiles row tiles of 256 rows, then
// wide_cols column tiles of 128 columns from column 0 in one launch and
// narrow_cols tiles of 64 columns after them in a second one.  With splits
// > 1 (small M), K is cut into ranges of split_tiles k-tiles that run in the
// same launch and write fp32 partial sums to the workspace.
struct GemmPlan {
    int64_t m_tiles, wide_cols, narrow_cols, splits, split_tiles;
};
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int64_t G, int cus);
// Compute units plan_gemm assumes: the forced count, else the device's.
int planning_cus();
// Force the compute units plan_gemm assumes (0: the current device's).
void set_planning_cus(int n);
// Workspace bytes of a GEMM call (0 unless it splits K).
int64_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t G);
hipError_t launch_gemm(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M, const Layout &lay,
                       void *workspace, hipStream_t stream);

// Measurement probes (not on the hot path).
hipError_t launch_probe_read(const void *buf, uint64_t bytes, uint32_t *sink, hipStream_t stream);
hipError_t launch_probe_mfma(int workgroups, int iters, float *sink, hipStream_t stream);
int64_t probe_mfma_flops(int workgroups, int iters);

} // namespace tf
