/*
 * tilefuse.h -- C ABI of the fused W4A16 / W8A16 linear layer for AMD MI355X
 * (gfx950).
 *
 * The operation (TileFuse technical summary, Methodology section 1, "Fused
 * mixed-precision microkernels"): unpack INT4/INT8 weights, dequantize them
 * as (q - zero) * scale with per-group or per-channel metadata, and run the
 * GEMM (prefill) or GEMV (token generation, Methodology section 3) in one
 * kernel flow, never writing full-precision weights to global memory.  The
 * weights are AWQ-style checkpoints (Contribution 1).  An offline step
 * re-lays them out as interleaved pre-tiled blocks with the metadata packed
 * next to the codes (Methodology section 2, "Interleaved pre-tiling").
 *
 *   y[m][n] = sum_k x[m][k] * (q[k][n] - z[g][n]) * s[g][n],  g = k / G
 *
 * Conventions shared by every call:
 *  - All data pointers are HIP device pointers owned by the caller; the
 *    library allocates nothing and keeps no pointer after a call returns.
 *  - Arrays are row-major and contiguous.  bf16 values travel as uint16_t
 *    bit patterns.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls are
 *    asynchronous on it; faults inside kernels surface at the caller's next
 *    synchronisation, as usual for HIP.
 *  - Arguments are validated on the host before any HIP work is queued (the
 *    only HIP calls before are device-property queries).  A call that
 *    returns anything but TF_OK has launched nothing and written nothing.
 *  - M == 0 is a valid empty problem: TF_OK, nothing launched.
 *  - Outputs must not alias inputs, the packed buffer or the workspace.
 *
 * Shape rules (TF_ERR_SHAPE / TF_ERR_GROUP when broken):
 *  - K > 0, N > 0, K % 32 == 0; W4 also needs N % 8 == 0 (eight columns per
 *    packed word).
 *  - G > 0, G % 32 == 0, K % G == 0, and G divides 128, is a multiple of
 *    128, or equals K.  Per-channel metadata is G == K.
 *  - GEMV: 1 <= M <= 16.  GEMM: 1 <= M <= 2^30.  Both: K < 2^25 (the
 *    kernels' offsets within a row of x and within a packed block are
 *    32-bit; tf_packed_bytes_* and the repack take K up to 2^31).
 *  - The [gate | up] calls (tf_repack_*_gate_up, tf_gemv_*_silu_mul,
 *    tf_gemm_*_silu_mul) also need N % 16 == 0: each half a whole number of
 *    8-column runs.
 *  - Sizes are 64-bit; every dimension must be below 2^31.
 */
#ifndef TILEFUSE_H
#define TILEFUSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TF_OK = 0,
    TF_ERR_NULL = 1,              /* a required pointer is NULL */
    TF_ERR_SHAPE = 2,             /* M, K or N outside the rules above */
    TF_ERR_GROUP = 3,             /* G outside the rules above */
    TF_ERR_ALIGN = 4,             /* a pointer misses its required alignment */
    TF_ERR_BUFFER_TOO_SMALL = 5,  /* packed_bytes or ws_bytes below the size query */
    TF_ERR_UNSUPPORTED = 6,       /* valid request the library does not implement */
    TF_ERR_HIP = 7                /* the HIP runtime reported a launch error */
} tf_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *tf_status_string(int status);

/* Version of the packed (pre-tiled) layout written by tf_repack_*.  A packed
 * buffer is only valid for the version that wrote it. */
int tf_format_version(void);

/* ------------------------------------------------------------------------ */
/* Offline interleaved pre-tiling (Methodology section 2).                   */
/*                                                                           */
/* Layout, version 2 (the pages fix no geometry; this is the library's):     */
/*  - Output columns in blocks of 16, block-major; ceil(N/16) blocks, padding */
/*    columns carry code 0, zero 0, scale 0.  A block is one contiguous       */
/*    range: its metadata, then its codes.                                   */
/*  - Metadata: one record per group in ascending k -- W4 40 bytes (16 bf16   */
/*    scales, then 16 zero-point nibbles), W8 48 bytes (16 scales, 16 zero   */
/*    bytes) -- the region zero-padded to a multiple of 16 bytes.  Column c: */
/*    scale bits at byte 2c; W4 zero in nibble c%2 of byte 32 + c/2; W8     */
/*    zero at byte 32 + c.                                                   */
/*  - Codes: ceil(K/128) k-tiles of 128 rows (W4 1024 bytes, W8 2048); rows  */
/*    past K are padding.  Row 32u + 8o + i of a k-tile (u, o < 4, i < 8),   */
/*    column r: W4 in the 32-bit word at byte 16(16o + r) + 4u, nibble       */
/*    i/2 + 4(i%2); W8 at byte 1024(u/2) + 16(16o + r) + 8(u%2) + i.         */
/*  So lane L = 16o + r of a 64-lane wavefront reading 16 bytes at 16L (W4)   */
/*  receives, for each of the k-tile's four 32-row steps, eight consecutive  */
/*  rows of column r: the B operand of a 16x16x32 bf16 MFMA after unpacking. */
/*  Group sizes must keep every 128-row k-tile inside one group or made of   */
/*  whole groups: G in {32, 64}, G a multiple of 128, or G == K.             */
/* ------------------------------------------------------------------------ */

/* Bytes of the packed buffer for (K, N, G); 0 if the shape is invalid. */
size_t tf_packed_bytes_w4(int64_t K, int64_t N, int64_t G);
size_t tf_packed_bytes_w8(int64_t K, int64_t N, int64_t G);

/* Re-lay out an AWQ W4 checkpoint.
 *   qweight  uint32 [K][N/8]: word (k, c) holds columns 8c..8c+7 of row k,
 *            column 8c + j in nibble p(j), p = (0, 4, 1, 5, 2, 6, 3, 7).
 *            4-byte aligned.
 *   qzeros   uint32 [K/G][N/8], same packing.  4-byte aligned.  NULL for
 *            symmetric quantization: every zero point is 8 (Methodology
 *            section 1 names zero points; this is their common special
 *            case), packed exactly as an explicit tensor of 8s would be.
 *   scales   bf16 [K/G][N] (fp16 for the *_f16 calls: the 16-bit scale
 *            bits are copied into the records unchanged).  2-byte aligned.
 *   packed   output, packed_bytes >= tf_packed_bytes_w4(K, N, G); 16-byte
 *            aligned.  Every byte of the layout is written. */
int tf_repack_w4(const uint32_t *qweight, const uint32_t *qzeros, const uint16_t *scales,
                 int64_t K, int64_t N, int64_t G, void *packed, size_t packed_bytes, void *stream);

/* Re-lay out a W8 checkpoint: qweight uint8 [K][N], zeros uint8 [K/G][N]
 * (unsigned codes, zero points stored as bytes), scales bf16 (or fp16, as
 * for tf_repack_w4) [K/G][N].
 * zeros NULL: symmetric quantization, every zero point 128. */
int tf_repack_w8(const uint8_t *qweight, const uint8_t *zeros, const uint16_t *scales,
                 int64_t K, int64_t N, int64_t G, void *packed, size_t packed_bytes, void *stream);

/* Re-lay out a fused [gate | up] checkpoint (N = 2 N' columns, gate first,
 * N % 16 == 0) for tf_gemv_*_silu_mul: arguments, size and errors as
 * tf_repack_w4 / _w8, but column c of 16-column block j holds gate column
 * 8 j + c (c < 8) or up column 8 j + c - 8 (c >= 8), so that every block
 * holds matching gate and up columns.  The result is the plain layout of the
 * checkpoint with its columns so permuted; N % 16 != 0 is TF_ERR_SHAPE. */
int tf_repack_w4_gate_up(const uint32_t *qweight, const uint32_t *qzeros, const uint16_t *scales,
                         int64_t K, int64_t N, int64_t G, void *packed, size_t packed_bytes, void *stream);
int tf_repack_w8_gate_up(const uint8_t *qweight, const uint8_t *zeros, const uint16_t *scales,
                         int64_t K, int64_t N, int64_t G, void *packed, size_t packed_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Fused linear layer.                                                       */
/*   x          bf16 [M][K], 16-byte aligned                                 */
/*   packed     a buffer written by tf_repack_w4 / _w8 with the same K, N, G  */
/*   y          bf16 [M][N] output (fp32 accumulation, one rounding to bf16, */
/*              nearest-even), 2-byte aligned                                */
/*   workspace  device scratch of ws_bytes >= tf_workspace_bytes(...), 256-  */
/*              byte aligned.  NULL is fine when the size query returns 0, */
/*              i.e. unless the call splits K over workgroups: the GEMM at   */
/*              small M, or either call at 8 <= M <= 64 on a layer too      */
/*              narrow to fill the device (the 16-row-chunk kernel).  Below  */
/*              8 rows tf_gemv_* never needs one.  The size depends on the   */
/*              device the query runs on (its compute-unit count): query on  */
/*              the device the call will run on.                             */
/* ------------------------------------------------------------------------ */
size_t tf_workspace_bytes(int bits, int is_gemm, int64_t M, int64_t K, int64_t N, int64_t G);

/* Token-generation GEMV, 1 <= M <= 16 (Methodology section 3).  From 2
 * rows, wide layers (and from 8 rows, layers whose K ranges stay long
 * enough) run the kernel that serves 16-row chunks of x with one unpack
 * (the one GEMM calls of up to 64 rows run), which may split K over
 * workgroups and then needs the workspace. */
int tf_gemv_w4a16(const uint16_t *x, const void *packed, size_t packed_bytes, uint16_t *y,
                  int64_t M, int64_t K, int64_t N, int64_t G,
                  void *workspace, size_t ws_bytes, void *stream);
int tf_gemv_w8a16(const uint16_t *x, const void *packed, size_t packed_bytes, uint16_t *y,
                  int64_t M, int64_t K, int64_t N, int64_t G,
                  void *workspace, size_t ws_bytes, void *stream);

/* Token-generation GEMV over a fused [gate | up] layer with the SiLU product
 * in its epilogue, so that a decode step needs no separate activation
 * launch (the summary's Results section finds token generation dominated by
 * per-kernel dispatch overhead, and Methodology section 4 amortises it).
 * SiLU itself is not on the pages: silu(v) = v / (1 + e^-v), the activation
 * of the Llama-style MLP whose gate and up projections this fuses.
 *   packed  written by tf_repack_w4_gate_up / _w8_gate_up for the layer of
 *           N = 2 N' columns (gate in checkpoint columns 0 .. N'-1, up in
 *           N' .. N-1), N % 16 == 0.
 *   y       bf16 [M][N']: y[m][n] = silu(g) * u, where g and u are the fp32
 *           sums of checkpoint columns n and N' + n, rounded once to bf16
 *           (nearest-even).  Neither sum is rounded to bf16 first.
 * 0 <= M <= 16 (M == 0 does nothing), K < 2^25.  The call runs the kernel
 * tf_gemv_* runs for the same (M, K, N, G), so it needs the workspace that
 * tf_workspace_bytes(bits, 0, M, K, N, G) reports (none below 8 rows).
 * Other arguments and errors as tf_gemv_*; N % 16 != 0 is TF_ERR_SHAPE.  A
 * buffer from plain tf_repack_* gives wrong results here (not detectable). */
int tf_gemv_w4a16_silu_mul(const uint16_t *x, const void *packed, size_t packed_bytes, uint16_t *y,
                           int64_t M, int64_t K, int64_t N, int64_t G,
                           void *workspace, size_t ws_bytes, void *stream);
int tf_gemv_w8a16_silu_mul(const uint16_t *x, const void *packed, size_t packed_bytes, uint16_t *y,
                           int64_t M, int64_t K, int64_t N, int64_t G,
                           void *workspace, size_t ws_bytes, void *stream);

/* Prefill GEMM over the same fused [gate | up] layer with the SiLU product in
 * its epilogue: arguments, output and errors as tf_gemv_*_silu_mul, for any
 * 1 <= M <= 2^30.  The call runs the kernels and launch plan tf_gemm_* runs
 * for the same (M, K, N, G), so it needs the workspace
 * tf_workspace_bytes(bits, 1, M, K, N, G) reports; with K split, the
 * product is applied after the ranges are added.  The [M][N] gate/up
 * output is never written to memory. */
int tf_gemm_w4a16_silu_mul(const uint16_t *x, const void *packed, size_t packed_bytes, uint16_t *y,
                           int64_t M, int64_t K, int64_t N, int64_t G,
                           void *workspace, size_t ws_bytes, void *stream);
int tf_gemm_w8a16_silu_mul(const uint16_t *x, const void *packed, size_t packed_bytes, uint16_t *y,
                           int64_t M, int64_t K, int64_t N, int64_t G,
                           void *workspace, size_t ws_bytes, void *stream);

/* Prefill GEMM, any M >= 1 (Methodology section 1): each weight tile is
 * unpacked once into LDS as the exact bf16 values q - z and reused by every
 * row of a 256-row tile; each group's scale is applied once per (group,
 * column) to its fp32 partial sum.  For M <= 64 a 256-row tile would mostly
 * compute padding, so the call runs the GEMV kernels instead (as tf_gemv_*
 * does up to 16 rows; above, up to four 16-row chunks of x per wave, K split
 * over workgroups on narrow layers); the result meets the same tolerance,
 * not the tiled kernel's bits.
 *
 * Scale domain of the tiled kernels (above 64 rows).  They carry each
 * column's running sum divided by the scale of its latest group and
 * multiply it by s_prev / s_next at each group start (256 x 256 tiles: one
 * chain over the call's K range; 256 x 128 and narrower tiles: two chains,
 * over the even and the odd groups; each K range of a split plan starts its
 * own chains).  Every nonzero scale must be at least 2^-126 in magnitude,
 * and every quotient the chain holds (the partial output sum x (q - z) s up
 * to a group, divided by that group's scale) and every ratio of consecutive
 * nonzero scales in a chain must stay below 2^127 in magnitude; otherwise
 * the output overflows to +-inf or NaN.  A column whose nonzero scales lie
 * within a factor of 2^60 of each other, with |x| <= 2^32, always meets
 * this (K < 2^25).  Zero scales are exact: the chain keeps its previous
 * scale and the group adds nothing.  The GEMV kernels multiply each group's
 * sum by its own scale and have no such limit. */
int tf_gemm_w4a16(const uint16_t *x, const void *packed, size_t packed_bytes, uint16_t *y,
                  int64_t M, int64_t K, int64_t N, int64_t G,
                  void *workspace, size_t ws_bytes, void *stream);
int tf_gemm_w8a16(const uint16_t *x, const void *packed, size_t packed_bytes, uint16_t *y,
                  int64_t M, int64_t K, int64_t N, int64_t G,
                  void *workspace, size_t ws_bytes, void *stream);

/* The same four calls for checkpoints in IEEE fp16 (the 16-bit format of
 * many AWQ checkpoints; the summary's Contribution 1 consumes AWQ-style
 * checkpoints directly, its Methodology section 1 names the BF16 form):
 * x is fp16 [M][K], the packed buffer was written by tf_repack_w4 / _w8
 * from fp16 scales [K/G][N] (repacking copies scale bits unchanged, so the
 * same repack serves both formats), and y is fp16 [M][N], one rounding of
 * the fp32 sum to nearest-even, magnitudes past 65504 becoming infinity.
 * The weights are still exact: (q - z) is an integer of at most 9 bits and
 * the MFMAs take fp16 operands; each group's fp16 scale, widened exactly,
 * is applied in fp32 as in the bf16 calls.  Kernels, launch plans,
 * workspace sizes (tf_workspace_bytes with is_gemm 0 or 1), shape rules
 * and errors are those of the bf16 call of the same name.  A buffer
 * repacked from bf16 scales gives wrong results here, and one from fp16
 * scales wrong results in the bf16 calls (not detectable). */
int tf_gemv_w4a16_f16(const uint16_t *x, const void *packed, size_t packed_bytes, uint16_t *y,
                      int64_t M, int64_t K, int64_t N, int64_t G,
                      void *workspace, size_t ws_bytes, void *stream);
int tf_gemv_w8a16_f16(const uint16_t *x, const void *packed, size_t packed_bytes, uint16_t *y,
                      int64_t M, int64_t K, int64_t N, int64_t G,
                      void *workspace, size_t ws_bytes, void *stream);
int tf_gemm_w4a16_f16(const uint16_t *x, const void *packed, size_t packed_bytes, uint16_t *y,
                      int64_t M, int64_t K, int64_t N, int64_t G,
                      void *workspace, size_t ws_bytes, void *stream);
int tf_gemm_w8a16_f16(const uint16_t *x, const void *packed, size_t packed_bytes, uint16_t *y,
                      int64_t M, int64_t K, int64_t N, int64_t G,
                      void *workspace, size_t ws_bytes, void *stream);

/* tf_gemm_w4a16 for callers that cannot allocate device memory: code under
 * HIP-graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels, plan and results as tf_gemm_w4a16 (bit for bit),
 * but no workspace argument: when the plan splits K, the fp32 partial sums go
 * to a fixed device array of 64 MiB inside the library, one per GPU, held
 * from the first such call on that GPU until the process ends.  The call
 * itself allocates nothing (no hipMalloc, no allocating library routine).
 *   - Every plan on a device of up to 256 compute units fits the array.  A
 *     plan whose partial sums exceed it (tf_workspace_bytes(4, 1, M, K, N,
 *     G) > 64 MiB, possible on larger devices) is refused with
 *     TF_ERR_UNSUPPORTED before any HIP work; other errors as
 *     tf_gemm_w4a16.
 *   - Every call on a GPU shares that GPU's array, which keeps the last
 *     call's contents (each call writes every partial it reads, so nothing
 *     needs clearing).  Calls that overlap on one GPU -- on different streams,
 *     or from several threads without ordering -- race on the array and may
 *     return wrong results; order them on one stream.
 *   - TF_ERR_HIP if the array's address cannot be obtained on the device. */
int tf_gemm_w4a16_noalloc(const uint16_t *x, const void *packed, size_t packed_bytes, uint16_t *y,
                          int64_t M, int64_t K, int64_t N, int64_t G, void *stream);

/* Test hooks, not on the hot path: the dequantized weights w[K][N] as fp32
 * ((q - z) * s is exact in fp32), decoded from a packed buffer by the
 * kernels' own operand builders, so that comparing w with the plain
 * definition bit for bit checks the code the kernels run:
 *   tf_dequant_w4_f32 / _w8_f32: the GEMM's -- the exact bf16 values q - z it
 *     stores in its LDS weight tile -- times s;
 *   tf_dequant_gemv_w4_f32 / _w8_f32: the GEMV kernels' -- bf16 128 + q and
 *     the zero-point operand 128 + z (W8: q and z) -- their difference times
 *     s.
 * w is 4-byte aligned; other arguments and errors as tf_gemv_*. */
int tf_dequant_w4_f32(const void *packed, size_t packed_bytes, float *w,
                      int64_t K, int64_t N, int64_t G, void *stream);
int tf_dequant_w8_f32(const void *packed, size_t packed_bytes, float *w,
                      int64_t K, int64_t N, int64_t G, void *stream);
int tf_dequant_gemv_w4_f32(const void *packed, size_t packed_bytes, float *w,
                           int64_t K, int64_t N, int64_t G, void *stream);
int tf_dequant_gemv_w8_f32(const void *packed, size_t packed_bytes, float *w,
                           int64_t K, int64_t N, int64_t G, void *stream);

/* ------------------------------------------------------------------------ */
/* Test hooks with explicit plan inputs.  A product call plans its launches */
/* for the current device's compute units and picks its kernel by M (the    */
/* GEMV kernels up to 64 rows).  These hooks take both as arguments, per    */
/* call; the library keeps no setting between calls (its only process-wide */
/* state is the per-device compute-unit count, queried once).               */
/*                                                                          */
/*   op     TF_OP_GEMV (tf_gemv_*), TF_OP_GEMM (tf_gemm_*),                 */
/*          TF_OP_GEMV_SILU_MUL, TF_OP_GEMM_SILU_MUL (the *_silu_mul calls), */
/*          TF_OP_GEMV_F16, TF_OP_GEMM_F16 (the *_f16 calls)                 */
/*   cus    compute units to plan for, 1 .. 2^20                            */
/*   route  TF_ROUTE_AUTO (the product calls' choice), TF_ROUTE_TILED (GEMM */
/*          calls run the tiled GEMM at any M, with 256 x 256 tiles wherever */
/*          they apply; AUTO drops them where a K split of theirs would     */
/*          fill less than 85 % of the compute units or leave ranges under  */
/*          8 k-tiles, and for W8 wherever K is split), TF_ROUTE_GEMV        */
/*          (the GEMV kernels up to 64 rows, as AUTO), TF_ROUTE_TILED128    */
/*          (the tiled GEMM at any M with 256 x 128 tiles only)             */
/* Other values: TF_ERR_UNSUPPORTED (the size query returns 0).             */
/* ------------------------------------------------------------------------ */
enum { TF_OP_GEMV = 0, TF_OP_GEMM = 1, TF_OP_GEMV_SILU_MUL = 2, TF_OP_GEMM_SILU_MUL = 3,
       TF_OP_GEMV_F16 = 4, TF_OP_GEMM_F16 = 5 };
enum { TF_ROUTE_AUTO = 0, TF_ROUTE_TILED = 1, TF_ROUTE_GEMV = 2, TF_ROUTE_TILED128 = 3 };

/* The call `op` on (bits, M, K, N, G) as planned for (cus, route): the same
 * validation, kernels and results as the product entry point it names when
 * cus is the device's count and route is TF_ROUTE_AUTO.  The workspace is
 * the one tf_workspace_bytes_planned reports for the same inputs. */
int tf_linear_planned(int bits, int op, const uint16_t *x, const void *packed, size_t packed_bytes,
                      uint16_t *y, int64_t M, int64_t K, int64_t N, int64_t G,
                      void *workspace, size_t ws_bytes, int cus, int route, void *stream);
size_t tf_workspace_bytes_planned(int bits, int op, int64_t M, int64_t K, int64_t N, int64_t G,
                                  int cus, int route);

/* Launch plan of a GEMM call (host only, no GPU work).
 * Above 128 rows, weights whose groups are whole 128-row k-tiles (G a
 * multiple of 128, or G == K) run on 256 x 256 output tiles, unless K has to
 * be split and the split would leave the chip under-filled or its ranges
 * short (W4), or K has to be split at all (W8).  Otherwise the
 * GEMM covers y with 256-row x 128-column tiles (128 x 128 up to 128 rows);
 * when those 256-row tiles are not a whole number of rounds over the compute
 * units, it runs the columns of the last partial round as 256 x 64 tiles in
 * a second launch.  When the tiles fill less than half the compute units
 * (small M), either kernel splits K into ranges that run in the same launch,
 * each writing fp32 partial sums to the workspace, and a second kernel adds
 * them in range order.  Within one kernel the plan never changes the
 * result's bits except through that split (the order of the split sums).
 * Writes eight values: out[5] = 1 when the call runs the GEMV kernels (then
 * out[0..2] = out[6] = out[7] = 0 and out[3], out[4] are their K split), 0
 * for the tiled GEMM; out[0] = row tiles of out[6] rows (256 or 128),
 * out[1] = wide column tiles of out[7] columns (256 or 128), out[2] =
 * 64-column tiles, out[3] = K ranges, out[4] = k-tiles of 128 rows per
 * range.  TF_ERR_NULL / TF_ERR_SHAPE / TF_ERR_GROUP / TF_ERR_UNSUPPORTED on
 * bad input. */
int tf_gemm_plan(int bits, int64_t M, int64_t K, int64_t N, int64_t G, int cus, int route, int64_t *out);

/* Launch plan of the GEMV kernels for M <= 64 rows (host only), for checks of
 * the limits the kernels rely on.  Writes fourteen values: out[0] kernel (0:
 * the kernel for up to 16 rows, 1: the 16-row-chunk kernel), out[1] waves
 * per workgroup, out[2] 16-column blocks per workgroup, out[3] K ranges over
 * workgroups, out[4] k-tiles per range, out[5] k-tiles per staged chunk,
 * out[6] k-tiles of codes in flight per wave, out[7] 16-row chunks per wave,
 * out[8] LDS bytes per workgroup, out[9] the launcher's LDS limit, out[10]
 * 16-byte activation units one staging pass holds (kernel 1; 0: staged by a
 * loop), out[11] 8-byte record words one staging pass holds over all blocks
 * (kernel 1; 0: a loop), out[12] record bytes reserved per block per chunk,
 * out[13] bf16 elements per staged activation row.  Errors as tf_gemm_plan;
 * M outside 1..64 is TF_ERR_SHAPE. */
int tf_gemv_plan(int bits, int64_t M, int64_t K, int64_t N, int64_t G, int cus, int64_t *out);

/* Measurement probes (not on the hot path): the practical roofs the fused
 * kernels are measured against, on the same machine and launch pattern.
 *   tf_probe_stream_read: one launch of a plain kernel that reads `bytes`
 *     (a multiple of 16, buf 16-byte aligned) once with 16-byte non-temporal
 *     loads and discards them; sink is a device uint32 it may write.
 *   tf_probe_mfma: one launch of `workgroups` workgroups of 8 waves, each wave
 *     issuing `iters` x 4 independent bf16 32x32x16 MFMAs; *flops (host) gets
 *     the launch's flop count.  sink is a device float it may write.
 *   tf_probe_block_read: the GEMV's code stream over a packed buffer of
 *     (bits, K, N, G) (layout as tf_packed_bytes_*; device pointer, 16-byte
 *     aligned, `nbytes` at least the packed size, else
 *     TF_ERR_BUFFER_TOO_SMALL) without its arithmetic: one workgroup per 16-column block,
 *     `waves` waves (1..16, at most ceil(K / 128)) splitting the block's
 *     k-tiles into contiguous ranges, `depth` (2, 4 or 8) 16-byte
 *     non-temporal tile loads in flight per wave, and a closing exchange
 *     through LDS with two barriers.  Pass the waves and depth tf_gemv_plan
 *     reports to mirror a GEMV launch.  Reads only the code tiles, never the
 *     records; K < 2^25.  sink is a device uint32 it may write.
 * All return TF_ERR_NULL / TF_ERR_SHAPE / TF_ERR_GROUP / TF_ERR_ALIGN on bad
 * arguments (TF_ERR_UNSUPPORTED for bits other than 4 and 8), TF_ERR_HIP on
 * a launch error. */
int tf_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);
int tf_probe_mfma(int workgroups, int iters, float *sink, int64_t *flops, void *stream);
int tf_probe_block_read(int bits, const void *packed, size_t nbytes, int64_t K, int64_t N, int64_t G, int waves,
                        int depth, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TILEFUSE_H */
