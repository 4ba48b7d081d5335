// C ABI of the fused W4A16 / W8A16 linear layer: argument validation on the
// host (before any HIP call), then one launch sequence on the caller's stream.
// The declarations and their documentation live in include/tilefuse.h.
#include "tilefuse.h"

#include <atomic>
#include <mutex>

#include "tf_launch.h"

// Split-K partial sums of tf_gemm_w4a16_noalloc: a fixed device array, one
// copy per GPU the library runs on, held until the process ends.  Host code
// never uses this name as an address (on the host it is a stand-in for the
// symbol); it uses the device address hipGetSymbolAddress returns for the
// current device.  64 MiB holds every split plan on a device of up to 256
// compute units: the tiled GEMM splits K only while its tiles fill at most
// half the units, so S ranges of M x N fp32 partials stay within
// cus x 256 x 256 x 4 bytes, and the GEMV kernels' splits stay below that.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {

using tf::Layout;

constexpr int64_t kDimLimit = int64_t(1) << 31;
// 32-bit offsets: a row of x in the GEMM, and a code tile within a
// 16-column block (K / 128 tiles of up to 2 KiB) in the GEMV kernels
constexpr int64_t kKernelKLimit = int64_t(1) << 25;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shape rules shared by every entry point; returns TF_OK or the error.
int check_kng(int bits, int64_t K, int64_t N, int64_t G)
{
    if (K <= 0 || N <= 0 || K >= kDimLimit || N >= kDimLimit || K % tf::kStepRows)
        return TF_ERR_SHAPE;
    if (bits == 4 && N % 8)
        return TF_ERR_SHAPE;
    if (G <= 0 || G % tf::kStepRows || K % G)
        return TF_ERR_GROUP;
    // a 128-row k-tile must lie inside one group or hold whole groups
    if (!(tf::kTileRows % G == 0 || G % tf::kTileRows == 0 || G == K))
        return TF_ERR_GROUP;
    return TF_OK;
}

size_t packed_bytes(int bits, int64_t K, int64_t N, int64_t G)
{
    if (check_kng(bits, K, N, G) != TF_OK)
        return 0;
    return (size_t)Layout::make(bits, K, N, G).total_bytes();
}

// gate_up: a [gate | up] checkpoint (N / 2 a multiple of 8), packed for the
// SiLU-product GEMV with the two halves interleaved in runs of 8 columns.
int repack(int bits, const void *qweight, const void *qzeros, const uint16_t *scales, int64_t K, int64_t N, int64_t G,
           void *packed, size_t nbytes, void *stream, bool gate_up = false)
{
    if (!qweight || !scales || !packed) // qzeros may be NULL: symmetric quantization
        return TF_ERR_NULL;
    if (int st = check_kng(bits, K, N, G))
        return st;
    if (gate_up && N % (2 * 8))
        return TF_ERR_SHAPE;
    if (!aligned(packed, 16) || !aligned(scales, 2) || (bits == 4 && (!aligned(qweight, 4) || !aligned(qzeros, 4))))
        return TF_ERR_ALIGN;
    const Layout lay = Layout::make(bits, K, N, G);
    if (nbytes < (size_t)lay.total_bytes())
        return TF_ERR_BUFFER_TOO_SMALL;
    if (tf::launch_repack(bits, qweight, qzeros, scales, lay, packed, static_cast<hipStream_t>(stream),
                          gate_up ? N / 2 : 0) != hipSuccess)
        return TF_ERR_HIP;
    return TF_OK;
}

// The six kinds of linear call (the TF_OP_* values of the header).
constexpr int kOpGemv = 0, kOpGemm = 1, kOpGemvSiluMul = 2, kOpGemmSiluMul = 3, kOpGemvF16 = 4, kOpGemmF16 = 5;
bool op_is_gemm(int op) { return op == kOpGemm || op == kOpGemmSiluMul || op == kOpGemmF16; }
bool op_is_silu(int op) { return op == kOpGemvSiluMul || op == kOpGemmSiluMul; }
bool op_is_f16(int op) { return op == kOpGemvF16 || op == kOpGemmF16; }
int64_t op_max_m(int op) { return op_is_gemm(op) ? (int64_t(1) << 30) : 16; }

// fp32 partial sums, S x M x N floats, when a call splits K over workgroups:
// the tiled GEMM with few output tiles (small M), the 16-row-chunk GEMV
// kernel (8..64 rows) on a layer too narrow to fill the chip.  Otherwise
// none: the GEMV kernel for up to 16 rows combines its K split inside a
// workgroup.  A SiLU-product call needs what the plain call of its shape
// needs.
size_t workspace_bytes(int bits, int op, int64_t M, int64_t K, int64_t N, int64_t G, int cus, int route)
{
    if (M < 1 || M > op_max_m(op) || check_kng(bits, K, N, G) != TF_OK)
        return 0;
    const Layout lay = Layout::make(bits, K, N, G);
    if (!op_is_gemm(op) || tf::gemm_uses_gemv(M, route))
        return (size_t)tf::gemv_workspace_bytes(lay, M, cus);
    return (size_t)tf::gemm_workspace_bytes(bits, M, N, K, G, cus, route);
}

// Validation of one linear call on the host (no HIP call): TF_OK, or the
// error the call returns.  ws_known: the workspace is the library's own (its
// pointer and size are checked by the caller), so only the size rule holds.
int validate(int bits, int op, const uint16_t *x, const void *packed, size_t nbytes, uint16_t *y, int64_t M,
             int64_t K, int64_t N, int64_t G, void *ws, size_t ws_bytes, int cus, int route)
{
    if (M < 0 || M > op_max_m(op))
        return TF_ERR_SHAPE;
    if (int st = check_kng(bits, K, N, G))
        return st;
    // the [gate | up] halves are whole 8-column runs
    if (op_is_silu(op) && N % (2 * 8))
        return TF_ERR_SHAPE;
    if (K >= kKernelKLimit)
        return TF_ERR_SHAPE;
    if (M == 0)
        return TF_OK;
    if (!x || !packed || !y)
        return TF_ERR_NULL;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(y, 2))
        return TF_ERR_ALIGN;
    const Layout lay = Layout::make(bits, K, N, G);
    if (nbytes < (size_t)lay.total_bytes())
        return TF_ERR_BUFFER_TOO_SMALL;
    const size_t need = workspace_bytes(bits, op, M, K, N, G, cus, route);
    if (need) {
        if (!ws)
            return TF_ERR_NULL;
        if (!aligned(ws, 256))
            return TF_ERR_ALIGN;
        if (ws_bytes < need)
            return TF_ERR_BUFFER_TOO_SMALL;
    }
    return TF_OK;
}

// The launches of a validated call (M > 0).
int launch(int bits, int op, const uint16_t *x, const void *packed, uint16_t *y, int64_t M, int64_t K, int64_t N,
           int64_t G, void *ws, int cus, int route, void *stream)
{
    const Layout lay = Layout::make(bits, K, N, G);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const bool tiled = op_is_gemm(op) && !tf::gemm_uses_gemv(M, route);
    hipError_t e;
    const int act = op_is_silu(op) ? tf::kActSiluMul : op_is_f16(op) ? tf::kActF16 : tf::kActNone;
    if (tiled)
        e = tf::launch_gemm(bits, x, packed, y, M, lay, ws, st, cus, act, route);
    else if (op_is_silu(op))
        e = tf::launch_gemv_silu_mul(bits, x, packed, y, M, lay, ws, st, cus);
    else
        e = tf::launch_gemv(bits, x, packed, y, M, lay, ws, st, cus, op_is_f16(op));
    return e == hipSuccess ? TF_OK : TF_ERR_HIP;
}

// One linear call: validation on the host, then the launches.  cus and
// route are the plan's inputs: the device's compute units and the automatic
// route for every product entry point.
int linear(int bits, int op, const uint16_t *x, const void *packed, size_t nbytes, uint16_t *y, int64_t M, int64_t K,
           int64_t N, int64_t G, void *ws, size_t ws_bytes, int cus, int route, void *stream)
{
    if (int st = validate(bits, op, x, packed, nbytes, y, M, K, N, G, ws, ws_bytes, cus, route))
        return st;
    if (M == 0)
        return TF_OK;
    return launch(bits, op, x, packed, y, M, K, N, G, ws, cus, route, stream);
}

int dequant(int bits, const void *packed, size_t nbytes, float *w, int64_t K, int64_t N, int64_t G, void *stream,
            bool gemv)
{
    if (!packed || !w)
        return TF_ERR_NULL;
    if (int st = check_kng(bits, K, N, G))
        return st;
    if (!aligned(packed, 16) || !aligned(w, 4))
        return TF_ERR_ALIGN;
    const Layout lay = Layout::make(bits, K, N, G);
    if (nbytes < (size_t)lay.total_bytes())
        return TF_ERR_BUFFER_TOO_SMALL;
    if (tf::launch_dequant_f32(bits, packed, lay, w, static_cast<hipStream_t>(stream), gemv) != hipSuccess)
        return TF_ERR_HIP;
    return TF_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; NULL if the lookup fails.
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_lock;

void *device_scratch()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    if (void *p = g_scratch[dev].load(std::memory_order_acquire))
        return p;
    std::lock_guard<std::mutex> hold(g_scratch_lock);
    if (void *p = g_scratch[dev].load(std::memory_order_relaxed))
        return p;
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
        return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
    return p;
}

bool plan_inputs_ok(int bits, int op, int cus, int route)
{
    return (bits == 4 || bits == 8) && op >= kOpGemv && op <= kOpGemmF16 && cus >= 1 && cus <= (1 << 20) &&
           (route == tf::kRouteAuto || route == tf::kRouteTiled || route == tf::kRouteGemv ||
            route == tf::kRouteTiled128);
}

} // namespace

extern "C" {

const char *tf_status_string(int s)
{
    switch (s) {
    case TF_OK: return "TF_OK";
    case TF_ERR_NULL: return "TF_ERR_NULL: a required pointer is NULL";
    case TF_ERR_SHAPE: return "TF_ERR_SHAPE: M, K or N outside the supported shapes";
    case TF_ERR_GROUP: return "TF_ERR_GROUP: group size must be a multiple of 32 dividing K that divides 128, is a multiple of 128, or equals K";
    case TF_ERR_ALIGN: return "TF_ERR_ALIGN: a pointer misses its required alignment";
    case TF_ERR_BUFFER_TOO_SMALL: return "TF_ERR_BUFFER_TOO_SMALL: packed or workspace buffer too small";
    case TF_ERR_UNSUPPORTED: return "TF_ERR_UNSUPPORTED";
    case TF_ERR_HIP: return "TF_ERR_HIP: the HIP runtime reported a launch error";
    default: return "unknown tf_status";
    }
}

int tf_format_version(void) { return tf::kFormatVersion; }

size_t tf_packed_bytes_w4(int64_t K, int64_t N, int64_t G) { return packed_bytes(4, K, N, G); }
size_t tf_packed_bytes_w8(int64_t K, int64_t N, int64_t G) { return packed_bytes(8, K, N, G); }

int tf_repack_w4(const uint32_t *qweight, const uint32_t *qzeros, const uint16_t *scales, int64_t K, int64_t N,
                 int64_t G, void *packed, size_t nbytes, void *stream)
{
    return repack(4, qweight, qzeros, scales, K, N, G, packed, nbytes, stream);
}

int tf_repack_w8(const uint8_t *qweight, const uint8_t *zeros, const uint16_t *scales, int64_t K, int64_t N,
                 int64_t G, void *packed, size_t nbytes, void *stream)
{
    return repack(8, qweight, zeros, scales, K, N, G, packed, nbytes, stream);
}

int tf_repack_w4_gate_up(const uint32_t *qweight, const uint32_t *qzeros, const uint16_t *scales, int64_t K,
                         int64_t N, int64_t G, void *packed, size_t nbytes, void *stream)
{
    return repack(4, qweight, qzeros, scales, K, N, G, packed, nbytes, stream, true);
}

int tf_repack_w8_gate_up(const uint8_t *qweight, const uint8_t *zeros, const uint16_t *scales, int64_t K, int64_t N,
                         int64_t G, void *packed, size_t nbytes, void *stream)
{
    return repack(8, qweight, zeros, scales, K, N, G, packed, nbytes, stream, true);
}

size_t tf_workspace_bytes(int bits, int is_gemm, int64_t M, int64_t K, int64_t N, int64_t G)
{
    if (bits != 4 && bits != 8)
        return 0;
    return workspace_bytes(bits, is_gemm ? kOpGemm : kOpGemv, M, K, N, G, tf::device_cus(), tf::kRouteAuto);
}

#define TF_LINEAR(name, bits, op)                                                                                     \
    int name(const uint16_t *x, const void *packed, size_t nbytes, uint16_t *y, int64_t M, int64_t K, int64_t N,      \
             int64_t G, void *ws, size_t ws_bytes, void *stream)                                                      \
    {                                                                                                                 \
        return linear(bits, op, x, packed, nbytes, y, M, K, N, G, ws, ws_bytes, tf::device_cus(), tf::kRouteAuto,   \
                      stream);                                                                                        \
    }
TF_LINEAR(tf_gemv_w4a16, 4, kOpGemv)
TF_LINEAR(tf_gemv_w8a16, 8, kOpGemv)
TF_LINEAR(tf_gemm_w4a16, 4, kOpGemm)
TF_LINEAR(tf_gemm_w8a16, 8, kOpGemm)
TF_LINEAR(tf_gemv_w4a16_silu_mul, 4, kOpGemvSiluMul)
TF_LINEAR(tf_gemv_w8a16_silu_mul, 8, kOpGemvSiluMul)
TF_LINEAR(tf_gemm_w4a16_silu_mul, 4, kOpGemmSiluMul)
TF_LINEAR(tf_gemm_w8a16_silu_mul, 8, kOpGemmSiluMul)
TF_LINEAR(tf_gemv_w4a16_f16, 4, kOpGemvF16)
TF_LINEAR(tf_gemv_w8a16_f16, 8, kOpGemvF16)
TF_LINEAR(tf_gemm_w4a16_f16, 4, kOpGemmF16)
TF_LINEAR(tf_gemm_w8a16_f16, 8, kOpGemmF16)
#undef TF_LINEAR

int tf_gemm_w4a16_noalloc(const uint16_t *x, const void *packed, size_t nbytes, uint16_t *y, int64_t M, int64_t K,
                          int64_t N, int64_t G, void *stream)
{
    const int cus = tf::device_cus();
    // the size rule, then every check of tf_gemm_w4a16 (the workspace stands
    // in as a valid 256-byte-aligned buffer of the array's size): no HIP
    // call for a request that will be refused
    if (workspace_bytes(4, kOpGemm, M, K, N, G, cus, tf::kRouteAuto) > kNoallocScratchBytes)
        return TF_ERR_UNSUPPORTED;
    void *const stand_in = reinterpret_cast<void *>(uintptr_t(256));
    if (int st = validate(4, kOpGemm, x, packed, nbytes, y, M, K, N, G, stand_in, kNoallocScratchBytes, cus,
                          tf::kRouteAuto))
        return st;
    if (M == 0)
        return TF_OK;
    void *ws = nullptr;
    if (workspace_bytes(4, kOpGemm, M, K, N, G, cus, tf::kRouteAuto) > 0) {
        ws = device_scratch();
        if (!ws)
            return TF_ERR_HIP;
    }
    return launch(4, kOpGemm, x, packed, y, M, K, N, G, ws, cus, tf::kRouteAuto, stream);
}

int tf_dequant_w4_f32(const void *packed, size_t nbytes, float *w, int64_t K, int64_t N, int64_t G, void *stream)
{
    return dequant(4, packed, nbytes, w, K, N, G, stream, false);
}

int tf_dequant_w8_f32(const void *packed, size_t nbytes, float *w, int64_t K, int64_t N, int64_t G, void *stream)
{
    return dequant(8, packed, nbytes, w, K, N, G, stream, false);
}

int tf_dequant_gemv_w4_f32(const void *packed, size_t nbytes, float *w, int64_t K, int64_t N, int64_t G,
                           void *stream)
{
    return dequant(4, packed, nbytes, w, K, N, G, stream, true);
}

int tf_dequant_gemv_w8_f32(const void *packed, size_t nbytes, float *w, int64_t K, int64_t N, int64_t G,
                           void *stream)
{
    return dequant(8, packed, nbytes, w, K, N, G, stream, true);
}

size_t tf_workspace_bytes_planned(int bits, int op, int64_t M, int64_t K, int64_t N, int64_t G, int cus, int route)
{
    if (!plan_inputs_ok(bits, op, cus, route))
        return 0;
    return workspace_bytes(bits, op, M, K, N, G, cus, route);
}

int tf_linear_planned(int bits, int op, const uint16_t *x, const void *packed, size_t nbytes, uint16_t *y, int64_t M,
                      int64_t K, int64_t N, int64_t G, void *ws, size_t ws_bytes, int cus, int route, void *stream)
{
    if (!plan_inputs_ok(bits, op, cus, route))
        return TF_ERR_UNSUPPORTED;
    return linear(bits, op, x, packed, nbytes, y, M, K, N, G, ws, ws_bytes, cus, route, stream);
}

int tf_gemm_plan(int bits, int64_t M, int64_t K, int64_t N, int64_t G, int cus, int route, int64_t *out)
{
    if (!out)
        return TF_ERR_NULL;
    if (!plan_inputs_ok(bits, kOpGemm, cus < 1 ? 1 : cus, route))
        return TF_ERR_UNSUPPORTED;
    if (M < 1 || cus < 1 || M > (int64_t(1) << 30))
        return TF_ERR_SHAPE;
    if (int st = check_kng(bits, K, N, G))
        return st;
    if (tf::gemm_uses_gemv(M, route)) {
        const Layout lay = Layout::make(bits, K, N, G);
        int64_t st = 0;
        out[0] = 0;
        out[1] = 0;
        out[2] = 0;
        out[3] = tf::gemv_splits(lay, M, cus, &st);
        out[4] = st;
        out[5] = 1;
        out[6] = 0;
        out[7] = 0;
        return TF_OK;
    }
    const tf::GemmPlan p = tf::plan_gemm(bits, M, N, K, G, cus, route);
    out[0] = p.m_tiles;
    out[1] = p.wide_cols;
    out[2] = p.narrow_cols;
    out[3] = p.splits;
    out[4] = p.split_tiles;
    out[5] = 0;
    out[6] = p.rows;
    out[7] = p.col_tile;
    return TF_OK;
}

int tf_gemv_plan(int bits, int64_t M, int64_t K, int64_t N, int64_t G, int cus, int64_t *out)
{
    if (!out)
        return TF_ERR_NULL;
    if (bits != 4 && bits != 8)
        return TF_ERR_UNSUPPORTED;
    if (M < 1 || M > tf::kGemvKernelMaxM || cus < 1 || cus > (1 << 20))
        return TF_ERR_SHAPE;
    if (int st = check_kng(bits, K, N, G))
        return st;
    const tf::GemvPlanInfo p = tf::gemv_plan_info(bits, Layout::make(bits, K, N, G), M, cus);
    const int64_t v[14] = {p.kernel, p.waves,  p.bpw,        p.splits,       p.split_tiles, p.chunk_tiles, p.depth,
                           p.row_chunks, p.lds, p.lds_limit, p.x_capacity, p.rec_capacity, p.meta_cap,  p.xpitch};
    for (int i = 0; i < 14; ++i)
        out[i] = v[i];
    return TF_OK;
}

int tf_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream)
{
    if (!buf || !sink)
        return TF_ERR_NULL;
    if (bytes == 0 || bytes % 16 || bytes / 16 / 1024 >= (size_t(1) << 31))
        return TF_ERR_SHAPE;
    if (!aligned(buf, 16) || !aligned(sink, 4))
        return TF_ERR_ALIGN;
    return tf::launch_probe_read(buf, bytes, sink, static_cast<hipStream_t>(stream)) == hipSuccess ? TF_OK
                                                                                                  : TF_ERR_HIP;
}

int tf_probe_block_read(int bits, const void *packed, size_t nbytes, int64_t K, int64_t N, int64_t G, int waves,
                        int depth, uint32_t *sink, void *stream)
{
    if (!packed || !sink)
        return TF_ERR_NULL;
    if (bits != 4 && bits != 8)
        return TF_ERR_UNSUPPORTED;
    if (int st = check_kng(bits, K, N, G))
        return st;
    const Layout lay = Layout::make(bits, K, N, G);
    if (K >= kKernelKLimit || waves < 1 || waves > 16 || waves > lay.ktiles || (depth != 2 && depth != 4 && depth != 8))
        return TF_ERR_SHAPE;
    if (nbytes < packed_bytes(bits, K, N, G))
        return TF_ERR_BUFFER_TOO_SMALL;
    if (!aligned(packed, 16) || !aligned(sink, 4))
        return TF_ERR_ALIGN;
    return tf::launch_probe_block_read(bits, packed, lay, waves, depth, sink, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? TF_OK
               : TF_ERR_HIP;
}

int tf_probe_mfma(int workgroups, int iters, float *sink, int64_t *flops, void *stream)
{
    if (!sink || !flops)
        return TF_ERR_NULL;
    if (workgroups < 1 || workgroups > (1 << 20) || iters < 1)
        return TF_ERR_SHAPE;
    if (!aligned(sink, 4))
        return TF_ERR_ALIGN;
    *flops = tf::probe_mfma_flops(workgroups, iters);
    return tf::launch_probe_mfma(workgroups, iters, sink, static_cast<hipStream_t>(stream)) == hipSuccess
               ? TF_OK
               : TF_ERR_HIP;
}

} // extern "C"
