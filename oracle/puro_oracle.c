/*
 * puro_oracle.c -- plain CPU oracle (TEST INFRASTRUCTURE ONLY; see
 * puro_oracle.h for what it follows and who may use it).
 *
 * Built with gcc -O2 -ffp-contract=off -fno-fast-math: every FP32 operation
 * below is a single IEEE binary32 operation with round-to-nearest-even, so the
 * scale and code arithmetic is exactly the one written.  Threads only split
 * independent outputs; they never change the arithmetic of any output.
 */
#define _GNU_SOURCE
#include "puro_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------------ */
/* E4M3 codec.  OCP OFP8 E4M3: 1 sign bit, 4 exponent bits (bias 7), 3
 * mantissa bits.  Exponent field 0 holds subnormals m * 2^-9; otherwise the
 * value is (1 + m/8) * 2^(e-7).  S.1111.111 is NaN; there is no infinity, so
 * the largest finite magnitude is S.1111.110 = 1.75 * 2^8 = 448. */

uint8_t orc_e4m3_encode(float v)
{
    uint32_t bits;
    memcpy(&bits, &v, sizeof bits);
    const uint8_t sign = (bits >> 31) ? 0x80 : 0x00;
    const double a = fabs((double)v);

    if (isnan(v))
        return sign | 0x7F;               /* undefined input; keep it NaN */
    if (a > 448.0)
        return sign | 0x7E;               /* saturate (infinity included) */
    if (a < 0x1p-6) {
        /* subnormal range: the code is the nearest multiple of 2^-9; rint()
         * rounds half to even.  A result of 8 is exponent field 1, mantissa 0,
         * i.e. the smallest normal 2^-6, so the bit pattern stays right. */
        const double m = rint(a * 512.0);
        return sign | (uint8_t)m;
    }
    int e2;
    const double f = frexp(a, &e2);       /* a = f * 2^e2, f in [0.5, 1) */
    const double g = 2.0 * f;             /* a = g * 2^E,  g in [1, 2)   */
    int E = e2 - 1;
    double m = rint((g - 1.0) * 8.0);     /* 3-bit mantissa, half to even */
    if (m == 8.0) {                       /* rounded up into the next binade */
        m = 0.0;
        E += 1;
    }
    return sign | (uint8_t)(((E + 7) << 3) | (int)m);
}

double orc_e4m3_decode(uint8_t code)
{
    const int s = code >> 7;
    const int e = (code >> 3) & 0xF;
    const int m = code & 0x7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp((double)(8 + m), e - 10);   /* (1 + m/8) * 2^(e-7) */
    return s ? -mag : mag;
}

/* ------------------------------------------------------------------------ */
/* Tile scale and per-element scaling. */

static inline float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static inline uint16_t bf16_mag(uint16_t h) { return (uint16_t)(h & 0x7FFF); }

float orc_tile_scale(float amax)
{
    return amax / 448.0f;                 /* one IEEE binary32 division */
}

float orc_scaled_value(float x, float amax)
{
    if (amax == 0.0f)
        return x * 0.0f;                  /* signed zero; codes 0x00 / 0x80 */
    if (amax < 0x1p-64f) {
        /* unbounded-exponent reading: scale both by 2^64 (exact) */
        x = x * 0x1p64f;
        amax = amax * 0x1p64f;
    }
    const float r = 448.0f / amax;        /* RN32(448 / amax) */
    return x * r;                         /* RN32(x * r)      */
}

uint8_t orc_quant_elem(float x, float amax)
{
    return orc_e4m3_encode(orc_scaled_value(x, amax));
}

void orc_quant_elems(const float* x, const float* amax, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_quant_elem(x[i], amax[i]);
}

/* ------------------------------------------------------------------------ */
/* A tiny parallel-for over [0, n). */

static int g_threads = 0;

void orc_set_threads(int n) { g_threads = n; }

int orc_get_threads(void)
{
    if (g_threads > 0)
        return g_threads;
    long c = sysconf(_SC_NPROCESSORS_ONLN);
    return c > 0 ? (int)c : 1;
}

typedef void (*range_fn)(void* ctx, int64_t begin, int64_t end);

typedef struct {
    range_fn fn;
    void* ctx;
    int64_t begin, end;
} range_job;

static void* range_thread(void* p)
{
    range_job* j = (range_job*)p;
    j->fn(j->ctx, j->begin, j->end);
    return NULL;
}

static void parallel_for(int64_t n, range_fn fn, void* ctx)
{
    int nt = orc_get_threads();
    if (nt > 256)
        nt = 256;
    if (n <= 0)
        return;
    if ((int64_t)nt > n)
        nt = (int)n;
    if (nt <= 1) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t th[256];
    range_job jobs[256];
    int started[256];
    for (int t = 0; t < nt; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].begin = n * t / nt;
        jobs[t].end = n * (t + 1) / nt;
        started[t] = pthread_create(&th[t], NULL, range_thread, &jobs[t]) == 0;
        if (!started[t])
            range_thread(&jobs[t]);       /* run inline if no thread */
    }
    for (int t = 0; t < nt; ++t)
        if (started[t])
            pthread_join(th[t], NULL);
}

typedef struct {
    uint32_t first;
    uint8_t* out;
} enc_ctx;

static void enc_range(void* p, int64_t b, int64_t e)
{
    const enc_ctx* c = (const enc_ctx*)p;
    for (int64_t i = b; i < e; ++i) {
        const uint32_t u = c->first + (uint32_t)i;
        float v;
        memcpy(&v, &u, sizeof v);
        c->out[i] = orc_e4m3_encode(v);
    }
}

void orc_e4m3_encode_range(uint32_t first_bits, int64_t n, uint8_t* out)
{
    enc_ctx c = {first_bits, out};
    parallel_for(n, enc_range, &c);
}

/* ------------------------------------------------------------------------ */
/* Quantizers. */

typedef struct {
    const uint16_t* x;
    int64_t rows, cols, rows_pad;
    uint8_t* q;
    float* s;
} quant_ctx;

/* 1x128 tiles along cols: tile (r, cb) = x[r][128cb .. 128cb+127]. */
static void rowwise_range(void* p, int64_t r0, int64_t r1)
{
    const quant_ctx* c = (const quant_ctx*)p;
    const int64_t nb = c->cols / 128;
    for (int64_t r = r0; r < r1; ++r) {
        for (int64_t cb = 0; cb < nb; ++cb) {
            const uint16_t* t = c->x + r * c->cols + cb * 128;
            uint16_t m = 0;
            for (int i = 0; i < 128; ++i)
                if (bf16_mag(t[i]) > m)
                    m = bf16_mag(t[i]);
            const float amax = bf16_to_f32(m);
            c->s[cb * c->rows + r] = orc_tile_scale(amax);
            for (int i = 0; i < 128; ++i)
                c->q[r * c->cols + cb * 128 + i] =
                    orc_quant_elem(bf16_to_f32(t[i]), amax);
        }
    }
}

int orc_quant_rowwise(const uint16_t* x, int64_t rows, int64_t cols,
                      uint8_t* q, float* s)
{
    if (rows < 0 || cols <= 0 || cols % 128 != 0)
        return -1;
    if (rows == 0)
        return 0;
    if (!x || !q || !s)
        return -1;
    quant_ctx c = {x, rows, cols, 0, q, s};
    parallel_for(rows, rowwise_range, &c);
    return 0;
}

/* 128x1 tiles along rows: tile (rb, col) = x[128rb .. 128rb+127][col]; the
 * codes are written transposed, qt[col][row]. */
static void colwise_range(void* p, int64_t c0, int64_t c1)
{
    const quant_ctx* c = (const quant_ctx*)p;
    const int64_t nrb = c->rows_pad / 128;
    for (int64_t col = c0; col < c1; ++col) {
        for (int64_t rb = 0; rb < nrb; ++rb) {
            const int64_t rend = (rb * 128 + 128 < c->rows) ? rb * 128 + 128 : c->rows;
            uint16_t m = 0;
            for (int64_t r = rb * 128; r < rend; ++r) {
                const uint16_t h = c->x[r * c->cols + col];
                if (bf16_mag(h) > m)
                    m = bf16_mag(h);
            }
            const float amax = bf16_to_f32(m);
            c->s[rb * c->cols + col] = orc_tile_scale(amax);
            for (int64_t r = rb * 128; r < rb * 128 + 128; ++r) {
                uint8_t code = 0x00;      /* padding rows: zero codes */
                if (r < c->rows)
                    code = orc_quant_elem(bf16_to_f32(c->x[r * c->cols + col]), amax);
                c->q[col * c->rows_pad + r] = code;
            }
        }
    }
}

int orc_quant_colwise(const uint16_t* x, int64_t rows, int64_t cols,
                      uint8_t* qt, float* st)
{
    if (rows < 0 || cols <= 0 || cols % 128 != 0)
        return -1;
    if (rows == 0)
        return 0;
    if (!x || !qt || !st)
        return -1;
    quant_ctx c = {x, rows, cols, (rows + 127) / 128 * 128, qt, st};
    parallel_for(cols, colwise_range, &c);
    return 0;
}

typedef struct {
    const uint16_t* w;
    int64_t n, k;
    uint8_t* q;
    uint8_t* qt;
    float* s;
} wquant_ctx;

/* 128x128 blocks (nb, kb) = w[128nb .. +127][128kb .. +127]. */
static void weight_range(void* p, int64_t nb0, int64_t nb1)
{
    const wquant_ctx* c = (const wquant_ctx*)p;
    const int64_t nkb = c->k / 128;
    for (int64_t nb = nb0; nb < nb1; ++nb) {
        for (int64_t kb = 0; kb < nkb; ++kb) {
            uint16_t m = 0;
            for (int64_t i = nb * 128; i < nb * 128 + 128; ++i)
                for (int64_t j = kb * 128; j < kb * 128 + 128; ++j)
                    if (bf16_mag(c->w[i * c->k + j]) > m)
                        m = bf16_mag(c->w[i * c->k + j]);
            const float amax = bf16_to_f32(m);
            c->s[nb * nkb + kb] = orc_tile_scale(amax);
            for (int64_t i = nb * 128; i < nb * 128 + 128; ++i)
                for (int64_t j = kb * 128; j < kb * 128 + 128; ++j) {
                    const uint8_t code = orc_quant_elem(bf16_to_f32(c->w[i * c->k + j]), amax);
                    c->q[i * c->k + j] = code;
                    if (c->qt)
                        c->qt[j * c->n + i] = code;
                }
        }
    }
}

int orc_quant_weight(const uint16_t* w, int64_t n, int64_t k,
                     uint8_t* q, uint8_t* qt, float* s)
{
    if (n <= 0 || k <= 0 || n % 128 != 0 || k % 128 != 0 || !w || !q || !s)
        return -1;
    wquant_ctx c = {w, n, k, q, qt, s};
    parallel_for(n / 128, weight_range, &c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Block-scaled GEMM. */

typedef struct {
    int mode;
    int64_t M, N, K;
    const uint8_t* a;
    const float* sa;
    const uint8_t* b;
    const float* sb;
    float* c;
    double* c64;
    int64_t row_begin;
    const int64_t* ii;
    const int64_t* jj;
    float* out;
    double dec[256];
} gemm_ctx;

static float scale_b(const gemm_ctx* g, int64_t j, int64_t kb)
{
    const int64_t nkb = g->K / 128;
    switch (g->mode) {
    case 0:  return g->sb[(j / 128) * nkb + kb];        /* [N/128][K/128] */
    case 1:  return g->sb[kb * (g->N / 128) + j / 128]; /* [K/128][N/128] */
    default: return g->sb[kb * g->N + j];               /* [K/128][N]     */
    }
}

static float gemm_elem(const gemm_ctx* g, int64_t i, int64_t j, double* acc64)
{
    const int64_t nkb = g->K / 128;
    const uint8_t* ar = g->a + i * g->K;
    const uint8_t* br = g->b + j * g->K;
    float acc = 0.0f;
    double a64 = 0.0;
    for (int64_t kb = 0; kb < nkb; ++kb) {
        double p = 0.0;                    /* exact: see header */
        for (int64_t k = kb * 128; k < kb * 128 + 128; ++k)
            p += g->dec[ar[k]] * g->dec[br[k]];
        const float sab = g->sa[kb * g->M + i] * scale_b(g, j, kb);
        const float pf = (float)p;         /* RN32(P_kb) */
        const float term = pf * sab;
        acc = acc + term;
        a64 += p * (double)g->sa[kb * g->M + i] * (double)scale_b(g, j, kb);
    }
    if (acc64)
        *acc64 = a64;
    return acc;
}

static void gemm_rows(void* p, int64_t r0, int64_t r1)
{
    const gemm_ctx* g = (const gemm_ctx*)p;
    for (int64_t r = r0; r < r1; ++r) {
        const int64_t i = g->row_begin + r;
        for (int64_t j = 0; j < g->N; ++j) {
            double d;
            const float v = gemm_elem(g, i, j, &d);
            g->c[r * g->N + j] = v;
            if (g->c64)
                g->c64[r * g->N + j] = d;
        }
    }
}

static void gemm_points(void* p, int64_t t0, int64_t t1)
{
    const gemm_ctx* g = (const gemm_ctx*)p;
    for (int64_t t = t0; t < t1; ++t)
        g->out[t] = gemm_elem(g, g->ii[t], g->jj[t], NULL);
}

static int gemm_args_ok(int mode, int64_t M, int64_t N, int64_t K,
                        const void* a, const void* sa, const void* b, const void* sb)
{
    if (mode < 0 || mode > 2 || M < 0 || N <= 0 || K <= 0 || K % 128 != 0)
        return 0;
    if (mode != 2 && N % 128 != 0)
        return 0;
    return a && sa && b && sb;
}

static void fill_dec(double* dec)
{
    for (int c = 0; c < 256; ++c)
        dec[c] = orc_e4m3_decode((uint8_t)c);
}

int orc_gemm_blockscaled(int mode, int64_t M, int64_t N, int64_t K,
                         const uint8_t* a, const float* sa,
                         const uint8_t* b, const float* sb,
                         float* c, double* c64,
                         int64_t row_begin, int64_t row_end)
{
    if (!gemm_args_ok(mode, M, N, K, a, sa, b, sb) || !c)
        return -1;
    if (row_begin < 0 || row_end > M || row_begin > row_end)
        return -1;
    gemm_ctx* g = (gemm_ctx*)calloc(1, sizeof(gemm_ctx));
    if (!g)
        return -1;
    g->mode = mode; g->M = M; g->N = N; g->K = K;
    g->a = a; g->sa = sa; g->b = b; g->sb = sb;
    g->c = c; g->c64 = c64; g->row_begin = row_begin;
    fill_dec(g->dec);
    parallel_for(row_end - row_begin, gemm_rows, g);
    free(g);
    return 0;
}

int orc_gemm_blockscaled_at(int mode, int64_t M, int64_t N, int64_t K,
                            const uint8_t* a, const float* sa,
                            const uint8_t* b, const float* sb,
                            const int64_t* ii, const int64_t* jj, int64_t count,
                            float* out)
{
    if (!gemm_args_ok(mode, M, N, K, a, sa, b, sb) || count < 0)
        return -1;
    if (count == 0)
        return 0;
    if (!ii || !jj || !out)
        return -1;
    for (int64_t t = 0; t < count; ++t)
        if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N)
            return -1;
    gemm_ctx* g = (gemm_ctx*)calloc(1, sizeof(gemm_ctx));
    if (!g)
        return -1;
    g->mode = mode; g->M = M; g->N = N; g->K = K;
    g->a = a; g->sa = sa; g->b = b; g->sb = sb;
    g->ii = ii; g->jj = jj; g->out = out;
    fill_dec(g->dec);
    parallel_for(count, gemm_points, g);
    free(g);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Unquantized reference. */

typedef struct {
    int64_t N, K;
    const uint16_t* x;
    int64_t xs_i, xs_k;
    const uint16_t* y;
    int64_t ys_j, ys_k;
    double* r;
    int64_t row_begin;
} ref_ctx;

static void ref_rows(void* p, int64_t r0, int64_t r1)
{
    const ref_ctx* c = (const ref_ctx*)p;
    for (int64_t r = r0; r < r1; ++r) {
        const int64_t i = c->row_begin + r;
        for (int64_t j = 0; j < c->N; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < c->K; ++k)
                acc += (double)bf16_to_f32(c->x[i * c->xs_i + k * c->xs_k]) *
                       (double)bf16_to_f32(c->y[j * c->ys_j + k * c->ys_k]);
            c->r[r * c->N + j] = acc;
        }
    }
}

int orc_matmul_ref(int64_t M, int64_t N, int64_t K,
                   const uint16_t* x, int64_t xs_i, int64_t xs_k,
                   const uint16_t* y, int64_t ys_j, int64_t ys_k,
                   double* r, int64_t row_begin, int64_t row_end)
{
    if (M < 0 || N <= 0 || K <= 0 || !x || !y || !r)
        return -1;
    if (row_begin < 0 || row_end > M || row_begin > row_end)
        return -1;
    ref_ctx c = {N, K, x, xs_i, xs_k, y, ys_j, ys_k, r, row_begin};
    parallel_for(row_end - row_begin, ref_rows, &c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* FP32 -> bf16 with round-to-nearest-even: keep the top 16 bits of the value
 * rounded at bit 16, halfway cases to the even result. */

uint16_t orc_f64_to_bf16(double d)
{
    if (isnan(d))
        return 0x7FC0;
    const uint16_t sign = signbit(d) ? 0x8000 : 0x0000;
    if (d == 0.0)
        return sign;
    if (isinf(d))
        return sign | 0x7F80;
    int e2;
    frexp(fabs(d), &e2);                  /* |d| = f * 2^e2, f in [0.5,1) */
    /* bf16 keeps 8 significant bits; below 2^-126 the spacing is fixed at
     * 2^-133 (subnormals). */
    int lsb_exp = e2 - 8;
    if (lsb_exp < -133)
        lsb_exp = -133;
    const double units = rint(ldexp(fabs(d), -lsb_exp));   /* half to even */
    const double mag = ldexp(units, lsb_exp);
    const float out = (float)mag;         /* exact, or +inf past the largest bf16 */
    uint32_t u;
    memcpy(&u, &out, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

uint16_t orc_f32_to_bf16(float v)
{
    return orc_f64_to_bf16((double)v);    /* exact widening */
}

typedef struct {
    const float* v;
    uint16_t* out;
} cvt_ctx;

static void cvt_range(void* p, int64_t b, int64_t e)
{
    const cvt_ctx* c = (const cvt_ctx*)p;
    for (int64_t i = b; i < e; ++i)
        c->out[i] = orc_f32_to_bf16(c->v[i]);
}

void orc_f32_to_bf16_array(const float* v, int64_t n, uint16_t* out)
{
    cvt_ctx c = {v, out};
    parallel_for(n, cvt_range, &c);
}

/* ------------------------------------------------------------------------ */
/* Neighbour ops that produce the path's operands (quantize-on-produce).
 *
 * Each op is evaluated in double straight from its definition and rounded
 * once to bf16 (y).  The band: with M the op's magnitude scale at that
 * element, a device that evaluates the op in FP32 returns some value in
 * [v - tol*M, v + tol*M]; rounding is monotonic, so its bf16 result lies
 * between the roundings of the two ends (lo, hi), both included.  lo == hi
 * (== y) marks an element with one correct result. */

/* A positive band is widened by 2^-149: below the normal range an FP32
 * result carries an absolute rounding error of up to half of 2^-149 (the
 * subnormal spacing) whatever its relative bound, so a device result there
 * is correct up to that much more. */
static void round_band(double v, double band, uint16_t* y, uint16_t* lo, uint16_t* hi)
{
    *y = orc_f64_to_bf16(v);
    if (!(band > 0.0)) {
        *lo = *y;                         /* exact: one result (keeps the sign of a zero) */
        *hi = *y;
        return;
    }
    band += 0x1p-149;
    *lo = orc_f64_to_bf16(v - band);
    *hi = orc_f64_to_bf16(v + band);
}

static double bf16_to_f64(uint16_t h) { return (double)bf16_to_f32(h); }

/* logistic function 1 / (1 + e^-g) */
static double sigmoid64(double g) { return 1.0 / (1.0 + exp(-g)); }

/* SwiGLU at one element, in double: h = silu(g) * u with silu(g) = g *
 * sigmoid(g); for the upstream gradient dh,
 *   d gate = dh * u * silu'(g),  silu'(g) = sigmoid(g) * (1 + g * (1 - sigmoid(g)))
 *   d up   = dh * silu(g)
 * m_gate = |dh * u * sigmoid(g)| * (1 + |g|) is the magnitude M of d gate: the
 * sum inside silu' can cancel, and an error in sigmoid(g) enters it
 * multiplied by g.  For h and d up, M is the magnitude of the result. */
static void swiglu_point(double g, double u, double dh, double* h, double* dgate, double* dup,
                         double* m_gate)
{
    const double sg = sigmoid64(g);
    const double silu = g * sg;
    *h = silu * u;
    *dgate = dh * u * (sg * (1.0 + g * (1.0 - sg)));
    *dup = dh * silu;
    *m_gate = fabs(dh * u * sg) * (1.0 + fabs(g));
}

void orc_swiglu_point(double g, double u, double dh, double* out4)
{
    swiglu_point(g, u, dh, &out4[0], &out4[1], &out4[2], &out4[3]);
}

void orc_bf16_band(double v, double band, uint16_t* out3)
{
    round_band(v, band, &out3[0], &out3[1], &out3[2]);
}

typedef struct {
    const uint16_t *a, *b, *gamma;
    int64_t rows, f, cols;
    double tol, eps;
    uint16_t *y, *lo, *hi;
    double* rstd;
} nb_ctx;

/* SwiGLU forward: gate = gu[r][c], up = gu[r][f + c] -> h[r][c]. */
static void swiglu_fwd_rows(void* p, int64_t r0, int64_t r1)
{
    nb_ctx* x = (nb_ctx*)p;
    const int64_t f = x->f;
    for (int64_t r = r0; r < r1; ++r) {
        for (int64_t c = 0; c < f; ++c) {
            const double g = bf16_to_f64(x->a[r * 2 * f + c]);
            const double u = bf16_to_f64(x->a[r * 2 * f + f + c]);
            double h, dg, du, mg;
            swiglu_point(g, u, 0.0, &h, &dg, &du, &mg);
            const int64_t i = r * f + c;
            round_band(h, x->tol * fabs(h), &x->y[i], &x->lo[i], &x->hi[i]);
        }
    }
}

/* SwiGLU backward: dh[r][c], gate, up -> d gate at dgu[r][c], d up at
 * dgu[r][f + c]. */
static void swiglu_bwd_rows(void* p, int64_t r0, int64_t r1)
{
    nb_ctx* x = (nb_ctx*)p;
    const int64_t f = x->f;
    for (int64_t r = r0; r < r1; ++r) {
        for (int64_t c = 0; c < f; ++c) {
            const double dh = bf16_to_f64(x->b[r * f + c]);
            const double g = bf16_to_f64(x->a[r * 2 * f + c]);
            const double u = bf16_to_f64(x->a[r * 2 * f + f + c]);
            double h, dg, du, mg;
            swiglu_point(g, u, dh, &h, &dg, &du, &mg);
            const int64_t ig = r * 2 * f + c, iu = r * 2 * f + f + c;
            round_band(dg, x->tol * mg, &x->y[ig], &x->lo[ig], &x->hi[ig]);
            round_band(du, x->tol * fabs(du), &x->y[iu], &x->lo[iu], &x->hi[iu]);
        }
    }
}

/* RMSNorm forward: y[r][c] = x[r][c] * rstd[r] * gamma[c] with
 * rstd[r] = 1 / sqrt(mean over c of x[r][c]^2 + eps).  M = |y|. */
static void rmsnorm_fwd_rows(void* p, int64_t r0, int64_t r1)
{
    nb_ctx* x = (nb_ctx*)p;
    const int64_t n = x->cols;
    for (int64_t r = r0; r < r1; ++r) {
        double ss = 0.0;
        for (int64_t c = 0; c < n; ++c) {
            const double v = bf16_to_f64(x->a[r * n + c]);
            ss += v * v;
        }
        const double rs = 1.0 / sqrt(ss / (double)n + x->eps);
        if (x->rstd)
            x->rstd[r] = rs;
        for (int64_t c = 0; c < n; ++c) {
            const double y = bf16_to_f64(x->a[r * n + c]) * rs * bf16_to_f64(x->gamma[c]);
            round_band(y, x->tol * fabs(y), &x->y[r * n + c], &x->lo[r * n + c], &x->hi[r * n + c]);
        }
    }
}

/* RMSNorm backward fused with the residual add.  The forward is
 * y_j = x_j * rstd * gamma_j with rstd = (mean over i of x_i^2 + eps)^(-1/2),
 * so d rstd / d x_i = -rstd^3 x_i / cols and the gradient reaching x through
 * the norm is
 *   rstd * gamma_j * dy_j - x_j * rstd^3 * c,   c = (1/cols) sum_i gamma_i dy_i x_i.
 * The residual-stream gradient gin (the branch's skip path; NULL = 0) adds to
 * it: out_j = gin_j + that.  rstd is the forward's FP32 value, taken as
 * given.  M_j = |gin_j| + |rstd gamma_j dy_j| + |x_j| rstd^3 (1/cols)
 * sum_i |gamma_i dy_i x_i| (the terms can cancel, and an error in c enters
 * multiplied by x_j rstd^3). */
typedef struct {
    const uint16_t *dy, *x, *gamma, *gin;
    const float* rstd;
    int64_t cols;
    double tol;
    uint16_t *y, *lo, *hi;
} nbb_ctx;

static void rmsnorm_bwd_rows(void* p, int64_t r0, int64_t r1)
{
    nbb_ctx* a = (nbb_ctx*)p;
    const int64_t n = a->cols;
    for (int64_t r = r0; r < r1; ++r) {
        const double rs = (double)a->rstd[r];
        double c = 0.0, cabs = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            const double t = bf16_to_f64(a->gamma[i]) * bf16_to_f64(a->dy[r * n + i]) *
                             bf16_to_f64(a->x[r * n + i]);
            c += t;
            cabs += fabs(t);
        }
        c /= (double)n;
        cabs /= (double)n;
        const double rs3 = rs * rs * rs;
        for (int64_t j = 0; j < n; ++j) {
            const int64_t e = r * n + j;
            const double gin = a->gin ? bf16_to_f64(a->gin[e]) : 0.0;
            const double xj = bf16_to_f64(a->x[e]);
            const double t1 = rs * bf16_to_f64(a->gamma[j]) * bf16_to_f64(a->dy[e]);
            const double t2 = xj * rs3 * c;
            const double v = gin + t1 - t2;
            const double m = fabs(gin) + fabs(t1) + fabs(xj) * rs3 * cabs;
            round_band(v, a->tol * m, &a->y[e], &a->lo[e], &a->hi[e]);
        }
    }
}

int orc_rmsnorm_bwd(const uint16_t* dy, const uint16_t* x, const uint16_t* gamma,
                    const float* rstd, const uint16_t* gin, int64_t rows, int64_t cols,
                    double tol, uint16_t* y, uint16_t* lo, uint16_t* hi)
{
    if (rows < 0 || cols <= 0 || !dy || !x || !gamma || !rstd || !y || !lo || !hi ||
        !(tol >= 0.0))
        return -1;
    nbb_ctx c = {.dy = dy, .x = x, .gamma = gamma, .gin = gin, .rstd = rstd, .cols = cols,
                 .tol = tol, .y = y, .lo = lo, .hi = hi};
    parallel_for(rows, rmsnorm_bwd_rows, &c);
    return 0;
}

int orc_residual_add(const uint16_t* a, const uint16_t* b, int64_t n, uint16_t* h)
{
    if (n < 0 || !a || !b || !h)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        h[i] = orc_f64_to_bf16(bf16_to_f64(a[i]) + bf16_to_f64(b[i]));
    return 0;
}

int orc_swiglu_fwd(const uint16_t* gu, int64_t rows, int64_t f, double tol, uint16_t* y,
                   uint16_t* lo, uint16_t* hi)
{
    if (rows < 0 || f <= 0 || !gu || !y || !lo || !hi || !(tol >= 0.0))
        return -1;
    nb_ctx c = {.a = gu, .rows = rows, .f = f, .tol = tol, .y = y, .lo = lo, .hi = hi};
    parallel_for(rows, swiglu_fwd_rows, &c);
    return 0;
}

int orc_swiglu_bwd(const uint16_t* dh, const uint16_t* gu, int64_t rows, int64_t f, double tol,
                   uint16_t* y, uint16_t* lo, uint16_t* hi)
{
    if (rows < 0 || f <= 0 || !dh || !gu || !y || !lo || !hi || !(tol >= 0.0))
        return -1;
    nb_ctx c = {.a = gu, .b = dh, .rows = rows, .f = f, .tol = tol, .y = y, .lo = lo, .hi = hi};
    parallel_for(rows, swiglu_bwd_rows, &c);
    return 0;
}

int orc_rmsnorm_fwd(const uint16_t* x, const uint16_t* gamma, int64_t rows, int64_t cols,
                    double eps, double tol, uint16_t* y, uint16_t* lo, uint16_t* hi, double* rstd)
{
    if (rows < 0 || cols <= 0 || !x || !gamma || !y || !lo || !hi || !(tol >= 0.0) ||
        !(eps >= 0.0))
        return -1;
    nb_ctx c = {.a = x, .gamma = gamma, .rows = rows, .cols = cols, .tol = tol, .eps = eps,
                .y = y, .lo = lo, .hi = hi, .rstd = rstd};
    parallel_for(rows, rmsnorm_fwd_rows, &c);
    return 0;
}
