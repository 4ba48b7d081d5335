/*
 * Host driver that runs every routine of oracle/oracle.c on one case inside
 * an AddressSanitizer + UndefinedBehaviorSanitizer build (test
 * infrastructure: built and run only by tests/test_oracle_sanitized.py).
 *
 * Every buffer is a heap allocation of exactly the size the routine's
 * contract gives, so a read or write one element past an end aborts the
 * run; undefined behaviour (a shift past the width, a signed overflow, a
 * misaligned load) aborts it too.  The driver also checks the round trips
 * the routines promise (pack after unpack, unrepack after repack, a column
 * subset of the dequant) and writes the numeric outputs, so the calling test
 * can compare them with the ordinary build bit for bit.
 *
 * Usage: oracle_sanitized_driver DIR
 *   DIR/spec.txt   "bits M K N G fmt ncols"
 *   DIR/qweight.bin, qzeros.bin (W4: AWQ words; W8: one byte per value),
 *   DIR/scales.bin (K/G x N half bits), x.bin (M x K half bits),
 *   DIR/cols.bin (ncols int64 column indices)
 * Writes DIR/y.bin (M x N fp64), out.bin (M x N half bits), packed.bin,
 * silu.bin (silu of the first half of row 0 times its second half).
 * Exit status 0 and "OK" on stdout when every check holds.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_unpack_w4(const uint32_t *words, int64_t R, int64_t C, uint8_t *codes);
void oracle_pack_w4(const uint8_t *codes, int64_t R, int64_t C, uint32_t *words);
float oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_f64_to_bf16(double v);
void oracle_round_bf16(const double *y, int64_t n, uint16_t *out);
float oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f64_to_f16(double v);
void oracle_round_f16(const double *y, int64_t n, uint16_t *out);
void oracle_dequant_w4(const uint32_t *qweight, const uint32_t *qzeros, const uint16_t *scales, int fmt,
                       int64_t K, int64_t N, int64_t G, const int64_t *cols, int64_t ncols, float *w);
void oracle_dequant_w8(const uint8_t *qweight, const uint8_t *zeros, const uint16_t *scales, int fmt,
                       int64_t K, int64_t N, int64_t G, const int64_t *cols, int64_t ncols, float *w);
void oracle_linear(const uint16_t *x, int fmt, int64_t M, int64_t K, const float *w, int64_t N, double *y);
void oracle_silu_mul(const double *g, const double *u, int64_t n, double *out);
int oracle_num_threads(void);
void oracle_set_num_threads(int n);
size_t oracle_packed_bytes(int bits, int64_t K, int64_t N, int64_t G);
int oracle_repack(int bits, const void *qweight, const void *qzeros, const uint16_t *scales,
                  int64_t K, int64_t N, int64_t G, uint8_t *packed);
int oracle_unrepack(int bits, const uint8_t *packed, int64_t K, int64_t N, int64_t G,
                    uint8_t *codes, uint8_t *zeros, uint16_t *scales);

static const char *g_dir;

static void fail(const char *what)
{
    fprintf(stderr, "FAIL: %s\n", what);
    exit(3);
}

static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p)
        fail("out of memory");
    return p;
}

/* Read DIR/name, which must hold exactly n bytes, into a fresh n-byte buffer. */
static void *read_exact(const char *name, size_t n)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", g_dir, name);
    FILE *f = fopen(path, "rb");
    if (!f)
        fail(path);
    void *p = xmalloc(n);
    size_t got = fread(p, 1, n, f);
    int extra = fgetc(f);
    fclose(f);
    if (got != n || extra != EOF)
        fail(path);
    return p;
}

static void write_all(const char *name, const void *p, size_t n)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", g_dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(p, 1, n, f) != n)
        fail(path);
    fclose(f);
}

/* Every finite half pattern survives widening and rounding back unchanged. */
static void check_conversions(void)
{
    for (uint32_t b = 0; b < 65536; ++b) {
        int bf_nan = (b & 0x7F80) == 0x7F80 && (b & 0x7F);
        int h_nan = (b & 0x7C00) == 0x7C00 && (b & 0x3FF);
        if (!bf_nan && oracle_f64_to_bf16((double)oracle_bf16_to_f32((uint16_t)b)) != b)
            fail("bf16 round trip");
        if (!h_nan && oracle_f64_to_f16((double)oracle_f16_to_f32((uint16_t)b)) != b)
            fail("fp16 round trip");
    }
}

int main(int argc, char **argv)
{
    if (argc != 2)
        fail("usage: oracle_sanitized_driver DIR");
    g_dir = argv[1];
    char path[4096];
    snprintf(path, sizeof path, "%s/spec.txt", g_dir);
    FILE *f = fopen(path, "r");
    if (!f)
        fail(path);
    int bits, fmt;
    long long M, K, N, G, ncols;
    if (fscanf(f, "%d %lld %lld %lld %lld %d %lld", &bits, &M, &K, &N, &G, &fmt, &ncols) != 7)
        fail("spec.txt");
    fclose(f);
    if ((bits != 4 && bits != 8) || M < 1 || K < 1 || N < 1 || G < 1 || K % G || ncols < 0 || (bits == 4 && N % 8))
        fail("spec values");
    const int64_t ng = K / G;
    const size_t wbytes = bits == 4 ? (size_t)(K * N / 2) : (size_t)(K * N);
    const size_t zbytes = bits == 4 ? (size_t)(ng * N / 2) : (size_t)(ng * N);
    void *qweight = read_exact("qweight.bin", wbytes);
    void *qzeros = read_exact("qzeros.bin", zbytes);
    uint16_t *scales = read_exact("scales.bin", (size_t)(ng * N) * 2);
    uint16_t *x = read_exact("x.bin", (size_t)(M * K) * 2);
    int64_t *cols = read_exact("cols.bin", (size_t)ncols * 8);

    check_conversions();
    oracle_set_num_threads(oracle_num_threads());

    /* codes and zeros one byte per value, from either width */
    uint8_t *codes = xmalloc((size_t)(K * N));
    uint8_t *zeros = xmalloc((size_t)(ng * N));
    if (bits == 4) {
        oracle_unpack_w4(qweight, K, N, codes);
        oracle_unpack_w4(qzeros, ng, N, zeros);
        uint32_t *words = xmalloc(wbytes);
        oracle_pack_w4(codes, K, N, words);
        if (memcmp(words, qweight, wbytes))
            fail("pack_w4 after unpack_w4");
        free(words);
    } else {
        memcpy(codes, qweight, wbytes);
        memcpy(zeros, qzeros, zbytes);
    }

    float *w = xmalloc((size_t)(K * N) * sizeof(float));
    float *wc = xmalloc((size_t)(K * ncols) * sizeof(float));
    if (bits == 4) {
        oracle_dequant_w4(qweight, qzeros, scales, fmt, K, N, G, NULL, N, w);
        oracle_dequant_w4(qweight, qzeros, scales, fmt, K, N, G, cols, ncols, wc);
    } else {
        oracle_dequant_w8(qweight, qzeros, scales, fmt, K, N, G, NULL, N, w);
        oracle_dequant_w8(qweight, qzeros, scales, fmt, K, N, G, cols, ncols, wc);
    }
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < ncols; ++j)
            if (memcmp(&wc[k * ncols + j], &w[k * N + cols[j]], sizeof(float)))
                fail("dequant of a column subset");

    double *y = xmalloc((size_t)(M * N) * sizeof(double));
    oracle_linear(x, fmt, M, K, w, N, y);
    uint16_t *out = xmalloc((size_t)(M * N) * 2);
    if (fmt)
        oracle_round_f16(y, M * N, out);
    else
        oracle_round_bf16(y, M * N, out);
    write_all("y.bin", y, (size_t)(M * N) * sizeof(double));
    write_all("out.bin", out, (size_t)(M * N) * 2);

    if (N % 2 == 0) {
        double *s = xmalloc((size_t)(N / 2) * sizeof(double));
        oracle_silu_mul(y, y + N / 2, N / 2, s);
        write_all("silu.bin", s, (size_t)(N / 2) * sizeof(double));
        free(s);
    }

    const size_t pbytes = oracle_packed_bytes(bits, K, N, G);
    if (pbytes) {
        uint8_t *packed = xmalloc(pbytes);
        if (oracle_repack(bits, qweight, qzeros, scales, K, N, G, packed))
            fail("repack rejected a shape packed_bytes accepted");
        write_all("packed.bin", packed, pbytes);
        uint8_t *codes2 = xmalloc((size_t)(K * N));
        uint8_t *zeros2 = xmalloc((size_t)(ng * N));
        uint16_t *scales2 = xmalloc((size_t)(ng * N) * 2);
        if (oracle_unrepack(bits, packed, K, N, G, codes2, zeros2, scales2))
            fail("unrepack rejected a shape packed_bytes accepted");
        if (memcmp(codes2, codes, (size_t)(K * N)) || memcmp(zeros2, zeros, (size_t)(ng * N)) ||
            memcmp(scales2, scales, (size_t)(ng * N) * 2))
            fail("unrepack after repack");
        free(codes2);
        free(zeros2);
        free(scales2);
        free(packed);
    }

    free(qweight);
    free(qzeros);
    free(scales);
    free(x);
    free(cols);
    free(codes);
    free(zeros);
    free(w);
    free(wc);
    free(y);
    free(out);
    printf("OK\n");
    return 0;
}
