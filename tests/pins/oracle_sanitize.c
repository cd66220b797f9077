/*
 * oracle_sanitize.c -- drives every entry point of the CPU oracle
 * (oracle/puro_oracle.c) over small and edge-case inputs, to be built with
 * -fsanitize=address,undefined and run by tests/test_oracle_sanitize.py.
 * Any out-of-bounds access, use of uninitialised heap memory through ASan's
 * checks, or undefined behaviour (shifts, overflow, misaligned access) aborts
 * the program.  A few values are also checked, so that a harness that stopped
 * calling the code would not pass silently.
 *
 * Cases: ragged row counts (1, 129, 300), tiles that are all zero, tiles whose
 * amax is below 2^-64 (the 2^64 pre-scale), weights with and without the
 * transposed copy, the three GEMM modes with sampled and full outputs, the
 * unquantized reference, bf16 rounding, and the neighbour ops with and
 * without a tolerance band.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "puro_oracle.h"

static uint32_t lcg = 12345u;
static uint32_t next_u32(void)
{
    lcg = lcg * 1664525u + 1013904223u;
    return lcg;
}

/* bf16 bit pattern of a value in [-scale, scale) (truncation is enough here) */
static uint16_t rand_bf16(float scale)
{
    const float v = ((float)(next_u32() >> 8) / 16777216.0f * 2.0f - 1.0f) * scale;
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    return (uint16_t)(u >> 16);
}

static int fails = 0;
#define CHECK(cond)                                                                   \
    do {                                                                              \
        if (!(cond)) {                                                                \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);        \
            ++fails;                                                                  \
        }                                                                             \
    } while (0)

static void quantizers(int64_t rows, int64_t cols)
{
    const int64_t rp = (rows + 127) / 128 * 128;
    uint16_t* x = malloc(sizeof(uint16_t) * rows * cols);
    for (int64_t i = 0; i < rows * cols; ++i)
        x[i] = rand_bf16(4.0f);
    /* an all-zero tile (row 0, first 128 columns) and a tiny tile (row 1) */
    for (int64_t c = 0; c < 128; ++c) {
        x[c] = (c & 1) ? 0x8000 : 0x0000;
        if (rows > 1)
            x[cols + c] = (uint16_t)(0x0100 + c);            /* ~1e-38: amax < 2^-64 */
    }
    uint8_t* q = malloc(rows * cols);
    float* s = malloc(sizeof(float) * (cols / 128) * rows);
    uint8_t* qt = malloc(cols * rp);
    float* st = malloc(sizeof(float) * (rp / 128) * cols);
    CHECK(orc_quant_rowwise(x, rows, cols, q, s) == 0);
    CHECK(orc_quant_colwise(x, rows, cols, qt, st) == 0);
    CHECK(s[0] == 0.0f);                                    /* the zero tile */
    CHECK(q[1] == 0x80 && q[0] == 0x00);                    /* signed zeros */
    if (rows > 1)
        CHECK(s[1] > 0.0f && s[1] < 1e-36f);
    for (int64_t c = 0; c < cols; ++c)                      /* pad rows of the copy */
        for (int64_t r = rows; r < rp; ++r)
            CHECK(qt[c * rp + r] == 0);
    CHECK(orc_quant_rowwise(x, rows, 100, q, s) == -1);     /* cols % 128 */
    free(x); free(q); free(s); free(qt); free(st);
}

static void weights(int64_t n, int64_t k)
{
    uint16_t* w = malloc(sizeof(uint16_t) * n * k);
    for (int64_t i = 0; i < n * k; ++i)
        w[i] = rand_bf16(0.05f);
    uint8_t* q = malloc(n * k);
    uint8_t* qt = malloc(n * k);
    float* s = malloc(sizeof(float) * (n / 128) * (k / 128));
    CHECK(orc_quant_weight(w, n, k, q, qt, s) == 0);
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < k; ++j)
            CHECK(qt[j * n + i] == q[i * k + j]);
    CHECK(orc_quant_weight(w, n, k, q, NULL, s) == 0);
    free(w); free(q); free(qt); free(s);
}

static void gemm(int mode, int64_t M, int64_t N, int64_t K)
{
    uint8_t* a = malloc(M * K);
    uint8_t* b = malloc(N * K);
    for (int64_t i = 0; i < M * K; ++i)
        a[i] = (uint8_t)(next_u32() % 0x7F);                /* no NaN codes */
    for (int64_t i = 0; i < N * K; ++i)
        b[i] = (uint8_t)(next_u32() % 0x7F);
    float* sa = malloc(sizeof(float) * (K / 128) * M);
    for (int64_t i = 0; i < (K / 128) * M; ++i)
        sa[i] = 1e-3f * (float)(1 + next_u32() % 100);
    const int64_t nsb = mode == 2 ? (K / 128) * N : (K / 128) * (N / 128);
    float* sb = malloc(sizeof(float) * nsb);
    for (int64_t i = 0; i < nsb; ++i)
        sb[i] = 1e-3f * (float)(1 + next_u32() % 100);
    float* c = malloc(sizeof(float) * M * N);
    double* c64 = malloc(sizeof(double) * M * N);
    CHECK(orc_gemm_blockscaled(mode, M, N, K, a, sa, b, sb, c, c64, 0, M) == 0);
    for (int64_t i = 0; i < M * N; ++i)
        CHECK(fabs((double)c[i] - c64[i]) <= 1e-5 * fabs(c64[i]) + 1e-30);
    int64_t ii[3] = {0, M - 1, M / 2}, jj[3] = {N - 1, 0, N / 2};
    float at[3];
    CHECK(orc_gemm_blockscaled_at(mode, M, N, K, a, sa, b, sb, ii, jj, 3, at) == 0);
    for (int t = 0; t < 3; ++t)
        CHECK(at[t] == c[ii[t] * N + jj[t]]);
    CHECK(orc_gemm_blockscaled(mode, M, N, 100, a, sa, b, sb, c, NULL, 0, M) == -1);
    free(a); free(b); free(sa); free(sb); free(c); free(c64);
}

static void reference(int64_t M, int64_t N, int64_t K)
{
    uint16_t* x = malloc(sizeof(uint16_t) * M * K);
    uint16_t* y = malloc(sizeof(uint16_t) * N * K);
    for (int64_t i = 0; i < M * K; ++i)
        x[i] = rand_bf16(1.0f);
    for (int64_t i = 0; i < N * K; ++i)
        y[i] = rand_bf16(1.0f);
    double* r = malloc(sizeof(double) * M * N);
    CHECK(orc_matmul_ref(M, N, K, x, K, 1, y, K, 1, r, 0, M) == 0);
    CHECK(orc_matmul_ref(M, N, K, x, 1, M, y, 1, N, r, 0, M) == 0);  /* transposed strides */
    free(x); free(y); free(r);
}

static void neighbours(int64_t rows, int64_t f)
{
    uint16_t* gu = malloc(sizeof(uint16_t) * rows * 2 * f);
    uint16_t* dh = malloc(sizeof(uint16_t) * rows * f);
    for (int64_t i = 0; i < rows * 2 * f; ++i)
        gu[i] = rand_bf16(8.0f);
    for (int64_t i = 0; i < rows * f; ++i)
        dh[i] = rand_bf16(1e-3f);
    uint16_t* y = malloc(sizeof(uint16_t) * rows * 2 * f);
    uint16_t* lo = malloc(sizeof(uint16_t) * rows * 2 * f);
    uint16_t* hi = malloc(sizeof(uint16_t) * rows * 2 * f);
    CHECK(orc_swiglu_fwd(gu, rows, f, 0x1p-18, y, lo, hi) == 0);
    CHECK(orc_swiglu_bwd(dh, gu, rows, f, 0x1p-18, y, lo, hi) == 0);
    CHECK(orc_swiglu_bwd(dh, gu, rows, f, 0.0, y, lo, hi) == 0);
    for (int64_t i = 0; i < rows * 2 * f; ++i)
        CHECK(lo[i] == y[i] && hi[i] == y[i]);              /* no band: one result */
    double* rstd = malloc(sizeof(double) * rows);
    uint16_t* gamma = malloc(sizeof(uint16_t) * 2 * f);
    for (int64_t i = 0; i < 2 * f; ++i)
        gamma[i] = rand_bf16(2.0f);
    CHECK(orc_rmsnorm_fwd(gu, gamma, rows, 2 * f, 1e-6, 0x1p-18, y, lo, hi, rstd) == 0);
    CHECK(orc_rmsnorm_fwd(gu, gamma, rows, 2 * f, -1.0, 0x1p-18, y, lo, hi, rstd) == -1);
    double out4[4];
    orc_swiglu_point(-1.5, 0.5, 2.0, out4);
    uint16_t band[3];
    orc_bf16_band(1.0 + 0x1p-8, 1e-9, band);
    CHECK(band[0] == 0x3F80 && band[2] == 0x3F81);
    free(gu); free(dh); free(y); free(lo); free(hi); free(rstd); free(gamma);
}

int main(void)
{
    orc_set_threads(4);
    CHECK(orc_e4m3_encode(448.0f) == 0x7E && orc_e4m3_encode(1.0f) == 0x38);
    CHECK(orc_e4m3_encode(-1e9f) == 0xFE && orc_e4m3_encode(0x1p-10f) == 0x00);
    for (int c = 0; c < 256; ++c)
        (void)orc_e4m3_decode((uint8_t)c);
    uint8_t codes[4096];
    orc_e4m3_encode_range(0xFFFFF800u, 4096, codes);         /* wraps past 2^32 */
    CHECK(orc_quant_elem(1.0f, 0.0f) == 0x00);
    CHECK(orc_f32_to_bf16(1.0f) == 0x3F80 && orc_f64_to_bf16(-0.0) == 0x8000);
    float v[5] = {1.0f, -2.5f, 3.4e38f, 1e-40f, NAN};
    uint16_t h[5];
    orc_f32_to_bf16_array(v, 5, h);
    CHECK(h[0] == 0x3F80 && h[4] == 0x7FC0);
    const int64_t shapes[][2] = {{1, 128}, {129, 256}, {300, 384}};
    for (int i = 0; i < 3; ++i)
        quantizers(shapes[i][0], shapes[i][1]);
    weights(128, 128);
    weights(256, 384);
    for (int mode = 0; mode < 3; ++mode) {
        gemm(mode, 37, 256, 384);
        gemm(mode, 1, 128, 128);
    }
    reference(19, 23, 129);
    neighbours(33, 128);
    neighbours(1, 256);
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("oracle sanitize: ok\n");
    return 0;
}
