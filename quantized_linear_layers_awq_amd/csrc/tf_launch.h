// Host-side launchers of the kernels; called by the C ABI after validation.
#pragma once

#include "tf_common.h"

namespace tf {

hipError_t launch_repack(int bits, const void *qweight, const void *qzeros, const uint16_t *scales,
                         const Layout &lay, void *packed, hipStream_t stream);
hipError_t launch_dequant_f32(int bits, const void *packed, const Layout &lay, float *w, hipStream_t stream);

// Waves per GEMV workgroup (one workgroup per 16-column block).
int gemv_waves(const Layout &lay);
hipError_t launch_gemv(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M, const Layout &lay,
                       hipStream_t stream);
hipError_t launch_gemm(int bits, const uint16_t *x, const void *packed, uint16_t *y, int64_t M, const Layout &lay,
                       hipStream_t stream);

} // namespace tf
