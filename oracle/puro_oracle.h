/*
 * puro_oracle.h -- plain CPU oracle for the fine-grained block-quantized FP8
 * linear layer (tile-wise FP8 quantization of GEMM operands followed by a
 * block-scaled GEMM).
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the ground truth the GPU path is
 * checked against.  It shares no code, header, table or helper with the HIP
 * library and must never be linked into, called from or imported by the
 * product path.  Only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.
 *
 * What it follows:
 *   - "Puro-2B" arXiv report, section 2.1 (Pipeline at a Glance) and the
 *     training.farm blog, FP8 section: the main Transformer linear-layer GEMMs
 *     run in blockwise FP8 in the fine-grained block quantization style of
 *     DeepSeek-V3; sensitive ops and training state stay in BF16/FP32.
 *   - the pages fix no tile shape, format or rounding; the oracle takes the
 *     plainest reading: 1x128 activation tiles along the contraction
 *     dimension, 128x1 tiles along tokens for the weight-gradient operands,
 *     128x128 weight blocks, OCP FP8 E4M3 codes, one FP32 scale per tile equal
 *     to amax/448, round-to-nearest-even with saturation at 448.
 *   - the E4M3 format itself is the public OCP 8-bit floating point
 *     specification (bias 7, max normal 448, S.1111.111 = NaN, no infinity).
 *
 * Every floating-point step is written out in the order the definition gives;
 * no blocking, fusion or reordering beyond it.
 */
#ifndef PURO_ORACLE_H
#define PURO_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- E4M3 codec (OCP OFP8 E4M3) ---------------------------------------- */
uint8_t orc_e4m3_encode(float v);          /* RNE, saturate |v|>448 to +-448 */
double  orc_e4m3_decode(uint8_t code);     /* exact value; NaN for 0x7F/0xFF */
/* out[i] = orc_e4m3_encode(binary32 with bit pattern first_bits + i), the bit
 * pattern wrapping modulo 2^32; i < n. */
void    orc_e4m3_encode_range(uint32_t first_bits, int64_t n, uint8_t* out);

/* ---- tile scale ---------------------------------------------------------- */
/* For a tile with absolute maximum amax (a bf16 value widened to float):
 *   s = RN32(amax / 448)                       -- the stored FP32 scale
 *   v = RN32(x * RN32(448 / amax))             -- the scaled element
 * evaluated with an unbounded exponent range: when amax < 2^-64 both amax and
 * x are multiplied by 2^64 first (exact), so 448/amax never overflows.
 * amax == 0 gives s = 0 and v = x * 0 (a signed zero). */
float   orc_tile_scale(float amax);
float   orc_scaled_value(float x, float amax);
uint8_t orc_quant_elem(float x, float amax);  /* E(scaled value) */
/* out[i] = orc_quant_elem(x[i], amax[i]) for i < n */
void    orc_quant_elems(const float* x, const float* amax, int64_t n, uint8_t* out);

/* ---- quantizers (bf16 inputs as raw uint16 bit patterns) ----------------
 * row-wise, 1x128 tiles along cols:   q[rows][cols], s[cols/128][rows]
 * col-wise, 128x1 tiles along rows:   qt[cols][rows_pad], st[rows_pad/128][cols]
 *   rows_pad = ceil(rows/128)*128; rows beyond `rows` are zero codes and do not
 *   enter the tile amax.
 * weight, 128x128 blocks:             q[n][k], s[n/128][k/128], qt[k][n] (opt.)
 * cols, n and k must be multiples of 128.  Return 0 on success, -1 on a bad
 * argument. */
int orc_quant_rowwise(const uint16_t* x, int64_t rows, int64_t cols,
                      uint8_t* q, float* s);
int orc_quant_colwise(const uint16_t* x, int64_t rows, int64_t cols,
                      uint8_t* qt, float* st);
int orc_quant_weight(const uint16_t* w, int64_t n, int64_t k,
                     uint8_t* q, uint8_t* qt /* may be NULL */, float* s);

/* ---- block-scaled GEMM ---------------------------------------------------
 * C[i][j] = sum over K-blocks kb of  RN32(P_kb) * RN32(sA * sB), accumulated
 * in FP32 (mul, then add), with P_kb = sum_{k in kb} dec(A[i][k]) * dec(B[j][k])
 * computed exactly (in double; every term is a multiple of 2^-18 and the sum
 * of 128 terms stays below 2^25, so no rounding occurs).
 *   A: u8 [M][K], B: u8 [N][K] (both K-contiguous), sa: f32 [K/128][M]
 *   sb: mode 0 (fwd)   [N/128][K/128]
 *       mode 1 (dgrad) [K/128][N/128]
 *       mode 2 (wgrad) [K/128][N]
 * Rows [row_begin, row_end) of C are written (C is indexed [i][j] with row
 * stride N).  c64 (optional) receives the same sum accumulated in double, to
 * report how far FP32 accumulation moves the result. */
int orc_gemm_blockscaled(int mode, int64_t M, int64_t N, int64_t K,
                         const uint8_t* a, const float* sa,
                         const uint8_t* b, const float* sb,
                         float* c, double* c64,
                         int64_t row_begin, int64_t row_end);

/* Same sum for an explicit list of output elements (i[t], j[t]). */
int orc_gemm_blockscaled_at(int mode, int64_t M, int64_t N, int64_t K,
                            const uint8_t* a, const float* sa,
                            const uint8_t* b, const float* sb,
                            const int64_t* ii, const int64_t* jj, int64_t count,
                            float* out);

/* Unquantized reference in double over bf16 inputs:
 *   R[i][j] = sum_k X[i*xs_i + k*xs_k] * Y[j*ys_j + k*ys_k]
 * for rows [row_begin, row_end), R row stride N. */
int orc_matmul_ref(int64_t M, int64_t N, int64_t K,
                   const uint16_t* x, int64_t xs_i, int64_t xs_k,
                   const uint16_t* y, int64_t ys_j, int64_t ys_k,
                   double* r, int64_t row_begin, int64_t row_end);

/* FP32 -> bf16, round to nearest even (the epilogue's output rounding). */
uint16_t orc_f32_to_bf16(float v);
/* Any double -> bf16, rounded once to nearest even (subnormals kept, +-inf
 * past the largest finite bf16, NaN -> 0x7FC0). */
uint16_t orc_f64_to_bf16(double v);
void     orc_f32_to_bf16_array(const float* v, int64_t n, uint16_t* out);

/* ---- neighbour ops that produce the path's operands ----------------------
 * (quantize-on-produce).  The pages keep the ops around the FP8 GEMMs in
 * BF16 ("Puro-2B" arXiv report, section 2.1; training.farm blog, FP8
 * section): each produces a bf16 tensor, which the path quantizes exactly as
 * orc_quant_rowwise / orc_quant_colwise do.  The pages do not define the ops;
 * these are the standard RMSNorm and SwiGLU of a pre-norm Transformer block,
 * with gate and up concatenated as gu[rows][2f] (gate first), the layout the
 * fused up+gate projection produces.
 *
 * Each op is evaluated in double and rounded once to bf16 (y).  A device
 * that evaluates the op in FP32 with an error of at most tol * M (M: the op's
 * magnitude at that element, stated per op in the source) returns a bf16
 * value between lo and hi, both included: the roundings of the two ends of
 * that band, widened by 2^-149 (an FP32 result below the normal range is
 * rounded to that spacing whatever its relative bound; tol = 0 keeps the band
 * empty).  lo == hi (== y) where only one result is correct.  Return 0, or
 * -1 on a bad argument.
 *   swiglu_fwd: gu [rows][2f] -> [rows][f],  h = silu(gate) * up
 *   swiglu_bwd: dh [rows][f], gu [rows][2f] -> [rows][2f] = (d gate | d up)
 *   rmsnorm_fwd: x [rows][cols], gamma [cols] -> [rows][cols],
 *                y = x * rstd * gamma, rstd[r] = 1/sqrt(mean(x^2) + eps)
 *                (rstd, optional, receives rstd in double) */
int orc_swiglu_fwd(const uint16_t* gu, int64_t rows, int64_t f, double tol, uint16_t* y,
                   uint16_t* lo, uint16_t* hi);
int orc_swiglu_bwd(const uint16_t* dh, const uint16_t* gu, int64_t rows, int64_t f, double tol,
                   uint16_t* y, uint16_t* lo, uint16_t* hi);
int orc_rmsnorm_fwd(const uint16_t* x, const uint16_t* gamma, int64_t rows, int64_t cols,
                    double eps, double tol, uint16_t* y, uint16_t* lo, uint16_t* hi,
                    double* rstd);
/* RMSNorm backward fused with the residual add (the output gradient of the
 * projection that writes the residual stream: out-proj, down): with the
 * forward's FP32 rstd taken as given,
 *   out[r][j] = gin[r][j] + rstd[r] * gamma[j] * dy[r][j]
 *               - x[r][j] * rstd[r]^3 * (1/cols) sum_i gamma[i] dy[r][i] x[r][i]
 * in double, rounded once to bf16 with its band (gin NULL = 0).  The
 * derivative of y = x * rstd * gamma (rstd = (mean x^2 + eps)^(-1/2)) by the
 * chain rule, plus the skip path. */
int orc_rmsnorm_bwd(const uint16_t* dy, const uint16_t* x, const uint16_t* gamma,
                    const float* rstd, const uint16_t* gin, int64_t rows, int64_t cols,
                    double tol, uint16_t* y, uint16_t* lo, uint16_t* hi);
/* The residual add that forms an RMSNorm's input: h[i] = a[i] + b[i], the
 * exact sum of the two bf16 values rounded once to bf16 (nearest even).  The
 * norm's statistic of h is orc_rmsnorm_fwd's rstd.  Return 0, or -1 on a bad
 * argument. */
int orc_residual_add(const uint16_t* a, const uint16_t* b, int64_t n, uint16_t* h);
/* The SwiGLU arithmetic above at one point, unrounded: out4 = {h, d gate,
 * d up, M of d gate} for gate g, up u and upstream gradient dh. */
void orc_swiglu_point(double g, double u, double dh, double* out4);
/* The rounding above for one value: out3 = {y, lo, hi} of v with band
 * half-width `band` (+ 2^-149 when band > 0). */
void orc_bf16_band(double v, double band, uint16_t* out3);

/* Worker threads used by the array functions (default: all online cores). */
void orc_set_threads(int n);
int  orc_get_threads(void);

#ifdef __cplusplus
}
#endif
#endif /* PURO_ORACLE_H */
