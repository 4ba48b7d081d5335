/*
 * CPU oracle for the fused W4A16 / W8A16 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or constant with the HIP
 * library: every constant below is written out here on its own.
 *
 * What it computes (TileFuse technical summary, Methodology section 1,
 * "Fused mixed-precision microkernels"): unpack the INT4/INT8 weights,
 * dequantize them with per-group or per-channel scales and zero points, then
 * run the matrix product.  Contribution 1 of the same summary says the
 * weights are AWQ-style W4A16/W8A16 checkpoints.  Written out:
 *
 *   q[k][n]  = code of row k, column n              (unpack)
 *   w[k][n]  = (q[k][n] - z[g][n]) * s[g][n],  g = floor(k / G)  (dequant)
 *   y[m][n]  = sum_k x[m][k] * w[k][n]              (GEMM / GEMV)
 *
 * Precision: dequant in fp32 (exact: |q - z| <= 255 has at most 8 significant
 * bits and a bf16 scale has 8, so the product has at most 16 < 24), products
 * and the k-ascending sum in fp64, one rounding to bf16 at the end, straight
 * from fp64 (round to nearest, ties to even).
 *
 * Half-precision variant: many AWQ checkpoints store fp16 scales and run on
 * fp16 activations.  With fmt = 1 the scales and x are IEEE binary16 and the
 * output is rounded once to binary16 (nearest, ties to even, overflow to
 * infinity).  The dequant stays exact in fp32: 8 bits of (q - z) times 11
 * significant bits of an fp16 scale is at most 19 < 24 bits.
 *
 * The repack/unrepack routines implement the interleaved pre-tiled layout
 * (TileFuse summary, Methodology section 2, "Interleaved pre-tiling":
 * scales and zero points packed into the weight tiles, tiles one consumer
 * reads laid out contiguously).  The layout itself is this library's own
 * (the pages fix no geometry); it is spelled out next to oracle_repack.
 *
 * oracle_silu_mul adds the SiLU product of a fused [gate | up] layer
 * (a decode epilogue; see that function).
 *
 * Pins: every function here is checked against something other than itself
 * by the host-only tests (exact rationals, integer GEMM special case,
 * exhaustive dequant exactness, library fp64 matmul, golden word fixtures,
 * round trips).  No function here is "parity unpinned".
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* AWQ 4-bit word layout: word (r, c) holds columns 8c..8c+7 of row r; */
/* column 8c+j sits in nibble NIBBLE_OF_COLUMN[j] (bits 4p..4p+3).     */
/* ------------------------------------------------------------------ */
static const int NIBBLE_OF_COLUMN[8] = {0, 4, 1, 5, 2, 6, 3, 7};

static inline unsigned awq_code(const uint32_t *words, int64_t C, int64_t r, int64_t c)
{
    uint32_t wd = words[r * (C / 8) + c / 8];
    return (wd >> (4 * NIBBLE_OF_COLUMN[c % 8])) & 0xFu;
}

void oracle_unpack_w4(const uint32_t *words, int64_t R, int64_t C, uint8_t *codes)
{
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c)
            codes[r * C + c] = (uint8_t)awq_code(words, C, r, c);
}

void oracle_pack_w4(const uint8_t *codes, int64_t R, int64_t C, uint32_t *words)
{
    for (int64_t r = 0; r < R; ++r)
        for (int64_t cw = 0; cw < C / 8; ++cw) {
            uint32_t wd = 0;
            for (int j = 0; j < 8; ++j)
                wd |= (uint32_t)(codes[r * C + 8 * cw + j] & 0xF) << (4 * NIBBLE_OF_COLUMN[j]);
            words[r * (C / 8) + cw] = wd;
        }
}

/* ------------------------------------------------------------------ */
/* bf16 <-> binary floating point                                      */
/* ------------------------------------------------------------------ */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a double to the nearest bf16 value, ties to even, in one step.
 * bf16 has 8 significant bits, exponents -126..127, subnormal quantum 2^-133. */
uint16_t oracle_f64_to_bf16(double v)
{
    if (isnan(v))
        return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a))
        return sign | 0x7F80;
    if (a == 0.0)
        return sign;
    int e;
    (void)frexp(a, &e);              /* a = f * 2^e, f in [0.5, 1): 2^(e-1) <= a < 2^e */
    int quantum_exp = (e - 1) - 7;   /* spacing of 8-significant-bit values in that binade */
    if (quantum_exp < -133)
        quantum_exp = -133;          /* subnormal range */
    double n = nearbyint(ldexp(a, -quantum_exp)); /* default mode: nearest, ties to even */
    double r = ldexp(n, quantum_exp);
    if (r >= 0x1p128)
        return sign | 0x7F80;        /* rounds past the largest finite bf16 */
    float rf = (float)r;             /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &rf, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

void oracle_round_bf16(const double *y, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f64_to_bf16(y[i]);
}

/* ------------------------------------------------------------------ */
/* IEEE binary16 (fp16) <-> binary floating point                      */
/* Sign bit, 5 exponent bits (bias 15), 10 fraction bits: 11           */
/* significant bits, normal exponents -14..15, subnormal quantum 2^-24, */
/* largest finite value 65504.                                         */
/* ------------------------------------------------------------------ */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 0x1F, f = h & 0x3FF;
    double v;
    if (e == 0x1F)
        v = f ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)f, -24);            /* subnormal: f * 2^-24 */
    else
        v = ldexp((double)(f | 0x400), e - 25); /* (1024 + f) * 2^(e - 15 - 10) */
    return (float)(sign ? -v : v);
}

/* Round a double to the nearest fp16 value, ties to even, in one step;
 * magnitudes that round past 65504 become infinity. */
uint16_t oracle_f64_to_f16(double v)
{
    if (isnan(v))
        return 0x7E00;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a))
        return sign | 0x7C00;
    if (a == 0.0)
        return sign;
    int e;
    (void)frexp(a, &e);             /* 2^(e-1) <= a < 2^e */
    int quantum_exp = (e - 1) - 10; /* spacing of 11-significant-bit values in that binade */
    if (quantum_exp < -24)
        quantum_exp = -24;          /* subnormal range */
    double r = ldexp(nearbyint(ldexp(a, -quantum_exp)), quantum_exp);
    if (r >= 65536.0)
        return sign | 0x7C00;
    if (r < 0x1p-14)                /* subnormal (or the smallest normal, reached below) */
        return sign | (uint16_t)ldexp(r, 24);
    int e2;
    double f2 = frexp(r, &e2);      /* r = f2 * 2^e2, f2 in [0.5, 1) */
    uint16_t frac = (uint16_t)ldexp(f2 * 2.0 - 1.0, 10); /* exact: r has <= 11 significant bits */
    return sign | (uint16_t)((e2 - 1 + 15) << 10) | frac;
}

void oracle_round_f16(const double *y, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f64_to_f16(y[i]);
}

/* A 16-bit scale or activation in format fmt: 0 = bf16, 1 = fp16. */
static inline float half_to_f32(uint16_t b, int fmt) { return fmt ? oracle_f16_to_f32(b) : oracle_bf16_to_f32(b); }

/* ------------------------------------------------------------------ */
/* Dequantization: w[k][j] = (q - z) * s for output column cols[j]     */
/* (all columns when cols == NULL).  fp32, exact.  Scales in format    */
/* fmt (0 = bf16, 1 = fp16).                                          */
/* ------------------------------------------------------------------ */
static inline int64_t col_of(const int64_t *cols, int64_t j) { return cols ? cols[j] : j; }

void oracle_dequant_w4(const uint32_t *qweight, const uint32_t *qzeros, const uint16_t *scales, int fmt,
                       int64_t K, int64_t N, int64_t G, const int64_t *cols, int64_t ncols, float *w)
{
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k) {
        int64_t g = k / G;
        for (int64_t j = 0; j < ncols; ++j) {
            int64_t n = col_of(cols, j);
            int q = (int)awq_code(qweight, N, k, n);
            int z = (int)awq_code(qzeros, N, g, n);
            float s = half_to_f32(scales[g * N + n], fmt);
            w[k * ncols + j] = (float)(q - z) * s;
        }
    }
}

void oracle_dequant_w8(const uint8_t *qweight, const uint8_t *zeros, const uint16_t *scales, int fmt,
                       int64_t K, int64_t N, int64_t G, const int64_t *cols, int64_t ncols, float *w)
{
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k) {
        int64_t g = k / G;
        for (int64_t j = 0; j < ncols; ++j) {
            int64_t n = col_of(cols, j);
            int q = qweight[k * N + n];
            int z = zeros[g * N + n];
            float s = half_to_f32(scales[g * N + n], fmt);
            w[k * ncols + j] = (float)(q - z) * s;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Linear: y[m][n] = sum_{k ascending} x[m][k] * w[k][n], in fp64;    */
/* x in format fmt (0 = bf16, 1 = fp16).                              */
/* Each thread owns a (row, column range) block and walks k outermost, */
/* so every output element still sums in k order.                     */
/* ------------------------------------------------------------------ */
#define ORACLE_COL_CHUNK 512

void oracle_linear(const uint16_t *x, int fmt, int64_t M, int64_t K, const float *w, int64_t N, double *y)
{
    int64_t nchunks = (N + ORACLE_COL_CHUNK - 1) / ORACLE_COL_CHUNK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t job = 0; job < M * nchunks; ++job) {
        int64_t m = job / nchunks;
        int64_t n0 = (job % nchunks) * ORACLE_COL_CHUNK;
        int64_t n1 = n0 + ORACLE_COL_CHUNK < N ? n0 + ORACLE_COL_CHUNK : N;
        double *yr = y + m * N;
        for (int64_t n = n0; n < n1; ++n)
            yr[n] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double xv = (double)half_to_f32(x[m * K + k], fmt);
            const float *wr = w + k * N;
            for (int64_t n = n0; n < n1; ++n)
                yr[n] += xv * (double)wr[n];
        }
    }
}

/* ------------------------------------------------------------------ */
/* SiLU product of a fused [gate | up] layer: out = silu(g) * u with   */
/* silu(v) = v * sigmoid(v) = v / (1 + e^-v), all in fp64.  The pages  */
/* name no activation; this is the Llama-style MLP's, applied to the   */
/* unrounded sums of the gate and up columns (the summary's Results    */
/* section: token generation pays per-kernel dispatch, so the product   */
/* runs in the GEMV's epilogue rather than a launch of its own).       */
/* ------------------------------------------------------------------ */
void oracle_silu_mul(const double *g, const double *u, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads later parallel loops use (the CPU baseline's per-core figure). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------ */
/* Interleaved pre-tiled layout (format version 2).                    */
/*                                                                    */
/*   Column blocks of 16 output columns, block-major; ceil(N/16)       */
/*   blocks, columns past N are padding (code 0, zero 0, scale 0).     */
/*   A block is its metadata followed by its codes:                    */
/*     metadata: one record per group in ascending k, W4 40 bytes      */
/*       (16 bf16 scales, then 16 zero nibbles), W8 48 bytes (16       */
/*       scales, 16 zero bytes); the region is zero-padded to a        */
/*       multiple of 16 bytes.  Column c of the block:                 */
/*         scale bits at 2c; W4 zero in byte 32 + c/2 (low nibble for  */
/*         even c); W8 zero at byte 32 + c.                            */
/*     codes: ceil(K/128) k-tiles of 128 rows (W4 1024 bytes, W8      */
/*       2048); rows past K are padding (code 0).  Row 32u + 8o + i    */
/*       of a k-tile (u, o < 4, i < 8), column r:                      */
/*         W4  word at 16*(16o + r) + 4u; row i in nibble i/2 + 4*(i%2)*/
/*         W8  byte at 1024*(u/2) + 16*(16o + r) + 8*(u%2) + i         */
/*   Group sizes: multiples of 32 dividing K that divide 128, are a    */
/*   multiple of 128, or equal K -- so a k-tile either lies inside one */
/*   group or holds whole groups.                                      */
/* ------------------------------------------------------------------ */
#define BLK_COLS 16
#define TILE_ROWS 128

static int layout_ok(int bits, int64_t K, int64_t N, int64_t G)
{
    if (bits != 4 && bits != 8)
        return 0;
    if (K <= 0 || N <= 0 || G <= 0)
        return 0;
    if (K % 32 || G % 32 || K % G)
        return 0;
    if (!(TILE_ROWS % G == 0 || G % TILE_ROWS == 0 || G == K))
        return 0;
    if (bits == 4 && N % 8)
        return 0;
    return 1;
}

static int64_t tile_bytes(int bits) { return bits == 4 ? 1024 : 2048; }
static int64_t record_bytes(int bits) { return bits == 4 ? 40 : 48; }
static int64_t meta_bytes(int bits, int64_t K, int64_t G)
{
    int64_t m = (K / G) * record_bytes(bits);
    return (m + 15) / 16 * 16;
}
static int64_t ktiles(int64_t K) { return (K + TILE_ROWS - 1) / TILE_ROWS; }
static int64_t block_bytes(int bits, int64_t K, int64_t G) { return meta_bytes(bits, K, G) + ktiles(K) * tile_bytes(bits); }

size_t oracle_packed_bytes(int bits, int64_t K, int64_t N, int64_t G)
{
    if (!layout_ok(bits, K, N, G))
        return 0;
    int64_t nblk = (N + BLK_COLS - 1) / BLK_COLS;
    return (size_t)(nblk * block_bytes(bits, K, G));
}

/* byte offset of the metadata record of (block j, group g) */
static int64_t record_at(int bits, int64_t K, int64_t G, int64_t j, int64_t g)
{
    return j * block_bytes(bits, K, G) + g * record_bytes(bits);
}

/* byte offset of (row k, block column r) inside the code region of block j;  */
/* for W4 also the bit shift inside the little-endian 32-bit word there.      */
static int64_t code_at(int bits, int64_t K, int64_t G, int64_t j, int64_t k, int r, int *shift)
{
    int64_t t = k / TILE_ROWS;
    int kr = (int)(k % TILE_ROWS);
    int u = kr / 32, o = (kr % 32) / 8, i = kr % 8;
    int64_t base = j * block_bytes(bits, K, G) + meta_bytes(bits, K, G) + t * tile_bytes(bits);
    if (bits == 4) {
        *shift = 4 * (i / 2 + 4 * (i % 2));
        return base + 16 * (16 * o + r) + 4 * u;
    }
    *shift = 0;
    return base + 1024 * (u / 2) + 16 * (16 * o + r) + 8 * (u % 2) + i;
}

static void put_u32(uint8_t *p, uint32_t v) { p[0] = v; p[1] = v >> 8; p[2] = v >> 16; p[3] = v >> 24; }
static uint32_t get_u32(const uint8_t *p) { return p[0] | (p[1] << 8) | (p[2] << 16) | ((uint32_t)p[3] << 24); }

/* Codes and zeros are read through this accessor so one repack serves both  */
/* widths.                                                                   */
static unsigned ckpt_code(int bits, const void *qweight, int64_t N, int64_t k, int64_t n)
{
    return bits == 4 ? awq_code((const uint32_t *)qweight, N, k, n) : ((const uint8_t *)qweight)[k * N + n];
}

int oracle_repack(int bits, const void *qweight, const void *qzeros, const uint16_t *scales,
                  int64_t K, int64_t N, int64_t G, uint8_t *packed)
{
    if (!layout_ok(bits, K, N, G))
        return -1;
    memset(packed, 0, oracle_packed_bytes(bits, K, N, G));
    int64_t nblk = (N + BLK_COLS - 1) / BLK_COLS;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < nblk; ++j) {
        for (int r = 0; r < BLK_COLS; ++r) {
            int64_t n = j * BLK_COLS + r;
            if (n >= N)
                continue;
            for (int64_t g = 0; g < K / G; ++g) {
                uint8_t *rec = packed + record_at(bits, K, G, j, g);
                uint16_t sb = scales[g * N + n];
                rec[2 * r] = sb & 0xFF;
                rec[2 * r + 1] = sb >> 8;
                unsigned z = ckpt_code(bits, qzeros, N, g, n);
                if (bits == 4)
                    rec[32 + r / 2] |= (uint8_t)(z << (4 * (r % 2)));
                else
                    rec[32 + r] = (uint8_t)z;
            }
            for (int64_t k = 0; k < K; ++k) {
                int shift;
                int64_t at = code_at(bits, K, G, j, k, r, &shift);
                unsigned q = ckpt_code(bits, qweight, N, k, n);
                if (bits == 4)
                    put_u32(packed + at, get_u32(packed + at) | ((uint32_t)q << shift));
                else
                    packed[at] = (uint8_t)q;
            }
        }
    }
    return 0;
}

/* Inverse of oracle_repack: recover the codes [K][N], zeros [K/G][N] (one  */
/* byte per value, unpacked) and the scale bits [K/G][N].  W4 callers can   */
/* rebuild checkpoint words with oracle_pack_w4.                            */
int oracle_unrepack(int bits, const uint8_t *packed, int64_t K, int64_t N, int64_t G,
                    uint8_t *codes, uint8_t *zeros, uint16_t *scales)
{
    if (!layout_ok(bits, K, N, G))
        return -1;
    int64_t nblk = (N + BLK_COLS - 1) / BLK_COLS;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < nblk; ++j) {
        for (int r = 0; r < BLK_COLS; ++r) {
            int64_t n = j * BLK_COLS + r;
            if (n >= N)
                continue;
            for (int64_t g = 0; g < K / G; ++g) {
                const uint8_t *rec = packed + record_at(bits, K, G, j, g);
                scales[g * N + n] = (uint16_t)(rec[2 * r] | (rec[2 * r + 1] << 8));
                zeros[g * N + n] = bits == 4 ? (rec[32 + r / 2] >> (4 * (r % 2))) & 0xF : rec[32 + r];
            }
            for (int64_t k = 0; k < K; ++k) {
                int shift;
                int64_t at = code_at(bits, K, G, j, k, r, &shift);
                codes[k * N + n] = bits == 4 ? (get_u32(packed + at) >> shift) & 0xF : packed[at];
            }
        }
    }
    return 0;
}
