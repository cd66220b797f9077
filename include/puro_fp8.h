/*
 * puro_fp8.h -- C ABI of the fine-grained block-quantized FP8 linear layer
 * for AMD Instinct MI355X (CDNA4, gfx950).
 *
 * What is computed.  The Puro-2B pretraining recipe puts the main Transformer
 * linear-layer GEMMs on an FP8 path using DeepSeek-V3-style fine-grained
 * block quantization, while numerically sensitive operations and training
 * state stay in BF16/FP32 (arXiv report "Puro-2B", section 2.1 "Pipeline at a
 * Glance"; training.farm blog, section "FP8"; bit.fan article, section "FP8
 * training and its trade-off").  The pages give no tile shape, format or
 * rounding; this library fixes them as follows:
 *   - codes: OCP FP8 E4M3 (bias 7, max 448, no infinity), one byte each;
 *   - one FP32 scale per tile: s = RN32(amax / 448), amax = max |x| over the
 *     tile; each element is v = RN32(x * RN32(448 / amax)) and its code is
 *     E4M3 round-to-nearest-even of v with saturation at 448.  When
 *     amax < 2^-64, x and amax are first multiplied by 2^64 (exact) so the
 *     reciprocal cannot overflow; amax == 0 gives s = 0 and signed-zero codes;
 *   - tiles: 1x128 along the contraction dimension for activations and
 *     output gradients, 128x1 along tokens for the weight-gradient operands,
 *     128x128 for weights;
 *   - GEMM: C = sum over 128-deep K-blocks of (A_kb . B_kb^T) * sA * sB,
 *     with the per-block partial product in FP32 and the scale applied to
 *     every K-block before FP32 accumulation across blocks.
 *
 * Conventions for every entry point:
 *   - Every pointer argument except `stream` is a DEVICE pointer; `stream` is
 *     a hipStream_t (NULL = the null stream).  The caller owns every buffer;
 *     the library never allocates, frees or synchronizes, keeps no mutable
 *     global state, and is safe to call from several host threads.
 *   - Calls are asynchronous: they validate arguments, enqueue kernels on
 *     `stream` and return.  Argument errors return synchronously before any
 *     work is enqueued and have no side effects.  A launch failure returns
 *     PURO_ERR_HIP; the status is that of this call's own launches, so an
 *     earlier, unread error of another HIP call on the thread is neither
 *     reported nor cleared.  A device fault surfaces at the caller's next
 *     synchronization.  No C++ exception crosses this boundary.
 *   - Tensors are dense and row-major.  Every base pointer must be 16-byte
 *     aligned.  Outputs must not alias inputs.  NaN / Inf inputs give
 *     undefined codes (not checked).
 *   - Sizes are int64_t element counts.  A dimension of 0 where allowed
 *     makes the call a no-op that returns PURO_OK.
 */
#ifndef PURO_FP8_H
#define PURO_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PURO_FP8_ABI_VERSION 1

typedef enum {
    PURO_OK = 0,
    PURO_ERR_NULL_POINTER = 1,  /* a required pointer is NULL                 */
    PURO_ERR_BAD_SHAPE = 2,     /* negative size, or not a multiple of 128    */
    PURO_ERR_MISALIGNED = 3,    /* a base pointer is not 16-byte aligned      */
    PURO_ERR_BAD_ENUM = 4,      /* unknown mode / dtype, or a bad combination */
    PURO_ERR_WORKSPACE = 5,     /* workspace smaller than required            */
    PURO_ERR_UNIMPLEMENTED = 6, /* valid request this version does not serve  */
    PURO_ERR_HIP = 7,           /* the HIP runtime rejected a launch          */
    PURO_ERR_INTERNAL = 8,      /* unexpected failure inside the library      */
    PURO_ERR_BAD_VALUE = 9      /* a scalar argument out of range (e.g. eps)  */
} puro_status_t;

typedef enum {
    PURO_GEMM_FWD = 0,    /* Y  = X . W^T   : M = tokens, N = out, K = in     */
    PURO_GEMM_DGRAD = 1,  /* dX = dY . W    : M = tokens, N = in,  K = out    */
    PURO_GEMM_WGRAD = 2,  /* dW = dY^T . X  : M = out,    N = in,  K = tokens */
    PURO_GEMM_DGRAD_W = 3, /* dX = dY . W as DGRAD, with b the weight's own
                              codes W [out][in] = [K][N] (no transposed copy) */
    PURO_GEMM_FWD_T = 4    /* Y = X . W^T as FWD, with b the transposed codes
                              W^T [in][out] = [K][N] (no untransposed copy)   */
} puro_gemm_mode_t;

typedef enum {
    PURO_OUT_BF16 = 0,   /* FP32 result rounded to bf16, nearest-even        */
    PURO_OUT_FP32 = 1
} puro_out_dtype_t;

/*
 * Activation / gradient quantizer (1x128 and 128x1 tiles).
 *
 *   x   bf16 [rows][cols]                       input (raw bf16 bits)
 *   q   u8   [rows][cols]                       1x128 codes (tiles along cols)
 *   s   f32  [cols/128][rows]                   one scale per 1x128 tile,
 *                                               block-major so a GEMM reads
 *                                               the scales of one K-block for
 *                                               consecutive rows contiguously
 *   qt  u8   [cols][rows_pad]                   128x1 codes, TRANSPOSED
 *                                               (tiles along rows)
 *   st  f32  [rows_pad/128][cols]               one scale per 128x1 tile
 *
 * rows_pad = ceil(rows / 128) * 128.  In the transposed copy, rows beyond
 * `rows` hold zero codes and do not enter the tile amax, so a WGRAD GEMM can
 * use K = rows_pad.  Either pair (q, s) or (qt, st) may be NULL (skipped);
 * not both.  Requires cols > 0, cols % 128 == 0, rows >= 0.
 * Defined by: the fine-grained block quantization of linear-layer GEMM
 * operands (arXiv report section 2.1; blog section "FP8").
 */
puro_status_t puro_fp8_quant_act(const void* x, int64_t rows, int64_t cols,
                                 uint8_t* q, float* s, uint8_t* qt, float* st,
                                 void* stream);

/*
 * Weight quantizer (128x128 blocks).
 *
 *   w   bf16 [n][k]          input weight (out features n, in features k)
 *   q   u8   [n][k]          codes (NULL = skip: a layer whose GEMMs are
 *                            FWD_T and DGRAD reads only qt)
 *   qt  u8   [k][n]          the same codes transposed (NULL = skip); DGRAD
 *                            and FWD_T read it
 *   s   f32  [n/128][k/128]  one scale per block
 *
 * Requires n, k > 0 and multiples of 128; s and at least one of q, qt.
 * Defined by: the same passages as puro_fp8_quant_act.
 */
puro_status_t puro_fp8_quant_weight(const void* w, int64_t n, int64_t k,
                                    uint8_t* q, uint8_t* qt, float* s,
                                    void* stream);

/*
 * Several weights quantized in ONE launch (one block's QKV, out-proj,
 * up/gate and down): each descriptor is exactly the arguments of one
 * puro_fp8_quant_weight call, with the same layouts, requirements and
 * results bit for bit.  The small weights of a block do not fill the 256
 * compute units one at a time (a 2048x2048 weight is 256 blocks of 128x128);
 * together they do, and one launch replaces four.
 *   descs  HOST array of `count` descriptors, read during the call only
 *   count  0 .. PURO_FP8_MAX_GROUPED_WEIGHTS (0 enqueues nothing)
 * A descriptor that fails puro_fp8_quant_weight's checks fails the call with
 * that status, and nothing is enqueued.  The outputs of different
 * descriptors must not overlap.
 * Defined by: the same passages as puro_fp8_quant_act.
 */
#define PURO_FP8_MAX_GROUPED_WEIGHTS 16
typedef struct puro_fp8_weight_desc {
    const void* w;    /* bf16 [n][k] */
    int64_t n, k;
    uint8_t* q;       /* u8 [n][k] or NULL */
    uint8_t* qt;      /* u8 [k][n] or NULL */
    float* s;         /* f32 [n/128][k/128] */
} puro_fp8_weight_desc;

puro_status_t puro_fp8_quant_weight_grouped(const puro_fp8_weight_desc* descs, int count,
                                            void* stream);

/*
 * Block-scaled FP8 GEMM.
 *
 *   C[m][n] (+)= sum over kb < K/128 of
 *                  sA(kb, m) * sB(kb, n) * sum_{k in kb} dec(a[m][k]) * dec(b[n][k])
 *
 *   a   u8  [M][K]   E4M3 codes, K-contiguous
 *   sa  f32 [K/128][M]
 *   b   u8  [N][K]   E4M3 codes, K-contiguous (DGRAD_W, FWD_T: [K][N],
 *                    N-contiguous)
 *   sb  f32 FWD     [N/128][K/128] (the weight's block scales; FWD_T too)
 *           DGRAD   [K/128][N/128] (the weight's block scales as stored for
 *                                   W [K][N]; b is the transposed code copy)
 *           DGRAD_W [K/128][N/128] (the same scales; b is W's codes as the
 *                                   weight quantizer writes them)
 *           WGRAD   [K/128][N]     (per-column 128x1 scales)
 *   c   bf16 or f32 [M][N] according to c_dtype
 *
 * How a linear layer with W [out][in] and T tokens maps onto the modes:
 *   FWD:   a = q(X) [T][in],   sa = s(X),  b = q(W) [out][in],  sb = s(W)
 *   DGRAD: a = q(dY) [T][out], sa = s(dY), b = qt(W) [in][out], sb = s(W)
 *   DGRAD_W: a = q(dY), sa = s(dY), b = q(W) [out][in], sb = s(W); the
 *          weight quantizer's transposed copy is then not needed (qt = NULL).
 *          The result equals DGRAD's (the same products); requires
 *          N <= 2^29 (N = in).
 *   FWD_T: a = q(X), sa = s(X), b = qt(W) [in][out], sb = s(W); the result
 *          equals FWD's; requires N <= 2^29 (N = out).  A layer that runs
 *          FWD_T and DGRAD needs only the transposed weight codes.
 * The two [K][N] modes read B with LDS transpose reads; which layout runs
 * faster depends on the shape (the FWD and DGRAD kernels are the same
 * otherwise).
 *   WGRAD: a = qt(dY) [out][T_pad], sa = st(dY), b = qt(X) [in][T_pad],
 *          sb = st(X)
 *
 * Requires M >= 0, N > 0 and K > 0 with N % 128 == 0 and K % 128 == 0, and
 * K <= 2^24 (16,777,216; PURO_ERR_BAD_SHAPE otherwise).
 * accumulate != 0 adds into the existing contents of c and needs
 * c_dtype == PURO_OUT_FP32.  workspace must hold at least
 * puro_fp8_gemm_workspace_bytes(mode, M, N, K) bytes (it may be NULL when
 * that is 0); its contents are scratch.
 * Defined by: the FP8 GEMMs of the main linear layers (arXiv report section
 * 2.1; blog section "FP8"), forward and the two backward products.
 */
puro_status_t puro_fp8_gemm_blockscaled(puro_gemm_mode_t mode, int64_t M, int64_t N,
                                        int64_t K, const uint8_t* a, const float* sa,
                                        const uint8_t* b, const float* sb, void* c,
                                        puro_out_dtype_t c_dtype, int accumulate,
                                        void* workspace, size_t workspace_bytes,
                                        void* stream);

/* Workspace bytes puro_fp8_gemm_blockscaled needs for this problem (0 if
 * none, or if the arguments are invalid). */
size_t puro_fp8_gemm_workspace_bytes(puro_gemm_mode_t mode, int64_t M, int64_t N,
                                     int64_t K);

/*
 * Block-scaled FP8 GEMM that allocates nothing, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, layouts, results and
 * errors as puro_fp8_gemm_blockscaled, without the workspace: when the
 * problem splits K across work-groups, the FP32 partials go to a static
 * device array of PURO_FP8_NOALLOC_SCRATCH_BYTES that each GPU the library
 * runs on holds until the process ends.  Problems whose
 * puro_fp8_gemm_workspace_bytes exceeds that size return PURO_ERR_WORKSPACE
 * before anything is enqueued.  The first call on a device looks up the
 * array's address on that device (hipGetSymbolAddress); no call allocates or
 * frees memory.  Every call on one GPU shares the array: calls that overlap
 * on one GPU (on other streams or from other threads) race and must be
 * serialized by the caller.
 */
#define PURO_FP8_NOALLOC_SCRATCH_BYTES (64u << 20)
puro_status_t puro_fp8_gemm_blockscaled_noalloc(puro_gemm_mode_t mode, int64_t M, int64_t N,
                                                int64_t K, const uint8_t* a, const float* sa,
                                                const uint8_t* b, const float* sb, void* c,
                                                puro_out_dtype_t c_dtype, int accumulate,
                                                void* stream);

/* Static, NUL-terminated description of a status code. */
const char* puro_fp8_status_string(puro_status_t status);

/* PURO_FP8_ABI_VERSION of the built library. */
int puro_fp8_abi_version(void);

/*
 * Diagnostic: the device E4M3 encoder the quantizers use, applied to the
 * binary32 values whose bit patterns are first_bits, first_bits + 1, ...,
 * first_bits + n - 1 (wrapping modulo 2^32).  out: u8 [n] device buffer.
 * Lets a test compare the hardware conversion against a reference over whole
 * ranges of inputs.  Requires n >= 0.
 */
puro_status_t puro_fp8_probe_encode(uint32_t first_bits, int64_t n, uint8_t* out,
                                    void* stream);

/*
 * Diagnostic: the FP32 sigmoid 1 / (1 + e^-g) that the SwiGLU producers
 * evaluate (puro_fp8_swiglu_quant, puro_fp8_swiglu_bwd_quant), applied to the
 * binary32 values whose bit patterns are first_bits, first_bits + 1, ...,
 * first_bits + n - 1 (wrapping modulo 2^32).  The producers use one of two
 * forms per wave of 64 lanes: the plain form when every gate of the wave is
 * >= -64, else the deep form (scaled by 2^64 below -64, so results heading
 * for the subnormal range are not flushed; the probe returns it scaled
 * back).  form 0: chosen per wave of 64 consecutive inputs as the producers
 * do; 1: the plain form; 2: the deep form (PURO_ERR_BAD_ENUM otherwise).
 * out: f32 [n] device buffer, 4-byte aligned.  Lets a test hold each form to
 * its error bound over whole ranges of inputs.  Requires n >= 0.
 */
puro_status_t puro_fp8_probe_sigmoid(uint32_t first_bits, int64_t n, int form, float* out,
                                     void* stream);

/*
 * Diagnostic: one matrix-core instruction on raw per-lane operand bytes, so
 * a test can see how each form adds its products (the GEMM's accuracy
 * depends on it).  One wave of 64 lanes; the accumulator input is zero.
 *   a, b  u8  [64][32]  lane l's operand bytes at offset 32*l (the 8-byte
 *                       forms use the first 8 of them, the bf16 form 16)
 *   d     f32 [64][16]  lane l's result registers at offset 16*l; unused
 *                       slots are written as 0
 *   form  0  v_mfma_f32_16x16x128_f8f6f4, E4M3 x E4M3 (the GEMM's form)
 *         1  v_mfma_f32_32x32x64_f8f6f4,  E4M3 x E4M3
 *         2  v_mfma_f32_16x16x32_fp8_fp8
 *         3  v_mfma_f32_32x32x16_fp8_fp8
 *         4  v_mfma_f32_16x16x32_bf16
 *         5  v_mfma_scale_f32_16x16x128_f8f6f4 with E8M0 scale bytes scale_a,
 *            scale_b passed at run time (0 .. 255)
 * PURO_ERR_BAD_ENUM for another form, PURO_ERR_BAD_VALUE for a scale byte
 * out of range; pointers 16-byte aligned.
 */
puro_status_t puro_fp8_probe_mfma(int form, const uint8_t* a, const uint8_t* b, int scale_a,
                                  int scale_b, float* d, void* stream);

/*
 * Quantize-on-produce: the BF16 ops next to the FP8 GEMMs, each writing its
 * result straight as FP8 operands (and, optionally, as bf16).
 *
 * The pages run only the main linear-layer GEMMs in FP8 and keep the other
 * ops in BF16 (arXiv report section 2.1; blog section "FP8").  These entry
 * points compute such an op in FP32, round the result to bf16 (nearest even)
 * and quantize that bf16 tensor in the same kernel, so the outputs equal
 * what the op followed by puro_fp8_quant_act on its [rows][out_cols] bf16
 * result gives, without the bf16 round trip through HBM.  Output layouts and
 * the ragged-row rule are those of puro_fp8_quant_act:
 *   q  u8  [rows][out_cols]       s  f32 [out_cols/128][rows]
 *   qt u8  [out_cols][rows_pad]   st f32 [rows_pad/128][out_cols]
 *   y  bf16 [rows][out_cols]      the op's bf16 result (NULL = not written)
 * Each of the pairs (q, s) and (qt, st) may be NULL, and y may be NULL, but
 * not all three.  Requires rows >= 0 and the column counts below to be > 0
 * multiples of 128.
 *
 * FP32 evaluation.  The result may differ from the exactly rounded bf16 of
 * the op where the exact value lies within the FP32 evaluation error of a
 * bf16 rounding boundary; it is then the other neighbour.  That error stays
 * below 2^-18 of the op's magnitude (|result|; for d gate,
 * |dh * up * sigmoid(gate)| * (1 + |gate|)) plus 2^-150 (half the FP32
 * subnormal spacing, for results below the normal range), for every gate
 * value (deep negative gates, where sigmoid heads for the subnormal range,
 * are evaluated with the exponential scaled by 2^64 and the result scaled
 * back in one last rounding) and, for RMSNorm, rows up to 2^15 columns.
 */

/*
 * SwiGLU forward.  gu bf16 [rows][2f] holds gate (columns 0 .. f-1) and up
 * (columns f .. 2f-1), as the fused up+gate projection writes them; the
 * output (out_cols = f) is h = silu(gate) * up, silu(g) = g / (1 + e^-g):
 * the input X of the down projection.
 */
puro_status_t puro_fp8_swiglu_quant(const void* gu, int64_t rows, int64_t f,
                                    uint8_t* q, float* s, uint8_t* qt, float* st,
                                    void* y, void* stream);

/*
 * SwiGLU backward.  dh bf16 [rows][f] is the gradient of h, gu as above; the
 * output (out_cols = 2f) is (d gate | d up) with
 *   d gate = dh * up * sigmoid(gate) * (1 + gate * (1 - sigmoid(gate)))
 *   d up   = dh * silu(gate)
 * the output gradient dY of the up+gate projection.
 */
puro_status_t puro_fp8_swiglu_bwd_quant(const void* dh, const void* gu, int64_t rows,
                                        int64_t f, uint8_t* q, float* s, uint8_t* qt,
                                        float* st, void* y, void* stream);

/*
 * RMSNorm forward.  x bf16 [rows][cols], gamma bf16 [cols]; the output
 * (out_cols = cols) is y = x * rstd * gamma with
 * rstd[r] = 1 / sqrt(mean over c of x[r][c]^2 + eps), the input X of the
 * projection after the norm.  rstd f32 [rows] is written too (the norm's
 * backward needs it) and is required.  eps must be finite and >= 0
 * (PURO_ERR_BAD_VALUE otherwise).  Two kernels: the row statistics, then
 * the fused normalize-and-quantize pass.
 */
puro_status_t puro_fp8_rmsnorm_quant(const void* x, const void* gamma, int64_t rows,
                                     int64_t cols, float eps, float* rstd, uint8_t* q,
                                     float* s, uint8_t* qt, float* st, void* y,
                                     void* stream);

/*
 * RMSNorm forward with the row statistic handed over: as
 * puro_fp8_rmsnorm_quant, but rstd f32 [rows] is an INPUT (as
 * puro_bf16_residual_add_rstd writes it for the norm's input), so the call is one
 * pass over x: the normalize-and-quantize kernel alone.  Arguments, layouts
 * and errors as for puro_fp8_rmsnorm_quant (no eps: it is in rstd).
 */
puro_status_t puro_fp8_rmsnorm_quant_rstd(const void* x, const void* gamma, const float* rstd,
                                          int64_t rows, int64_t cols, uint8_t* q, float* s,
                                          uint8_t* qt, float* st, void* y, void* stream);

/*
 * RMSNorm backward fused with the residual add: the output gradient dY of the
 * projection that writes the residual stream (the out-projection, and the
 * previous block's down projection), as FP8 operands.
 *   dy   bf16 [rows][cols]  gradient of the norm's output y (the next
 *                           projection's DGRAD result)
 *   x    bf16 [rows][cols]  the norm's input (the residual stream)
 *   gamma bf16 [cols], rstd f32 [rows] as the forward used them
 *   gin  bf16 [rows][cols]  gradient arriving along the skip path (NULL = 0)
 *   coef f32 [rows]         written: rstd^3 * (1/cols) sum_i gamma_i dy_i x_i
 * out (out_cols = cols) = gin + rstd * gamma * dy - x * coef, the derivative
 * of y = x * rstd * gamma by the chain rule plus the skip path; the bf16
 * result y (optional) is the gradient that continues down the residual
 * stream.  Two kernels: the per-row coefficient, then the fused pass.  The
 * FP32 error before the bf16 rounding is below (cols/512 + 18) * 2^-24 of
 * M = |gin| + |rstd gamma dy| + |x| rstd^3 (1/cols) sum_i |gamma_i dy_i x_i|
 * (under 2^-18 M for rows of up to 16384 columns); the bf16 value is one of
 * the two neighbours of the exact result whenever that band allows both.
 * rows, cols and outputs as for puro_fp8_rmsnorm_quant; rstd, coef and gin
 * 16-byte aligned.
 */
puro_status_t puro_fp8_rmsnorm_bwd_quant(const void* dy, const void* x, const void* gamma,
                                         const float* rstd, const void* gin, int64_t rows,
                                         int64_t cols, float* coef, uint8_t* q, float* s,
                                         uint8_t* qt, float* st, void* y, void* stream);

/*
 * The residual add that produces an RMSNorm's input, with the norm's row
 * statistic: h bf16 [rows][cols] = a + b (the FP32 sum of the two bf16
 * values, rounded to nearest even) and rstd f32 [rows] =
 * 1 / sqrt(mean over the row of h^2 + eps), for puro_fp8_rmsnorm_quant_rstd.
 * a, b, h bf16 [rows][cols]; cols a positive multiple of 128; eps finite and
 * >= 0 (PURO_ERR_BAD_VALUE otherwise).  Every pointer is required
 * (PURO_ERR_NULL_POINTER) and 16-byte aligned (PURO_ERR_MISALIGNED); rows = 0
 * enqueues nothing.  The caller owns all buffers; h must not alias a or b.
 */
puro_status_t puro_bf16_residual_add_rstd(const void* a, const void* b, int64_t rows, int64_t cols,
                                     float eps, void* h, float* rstd, void* stream);

/*
 * BF16 comparator (measurement only, not part of the FP8 path).
 *
 * The BF16 linear-layer GEMM the FP8 path replaces, on this library's own
 * tiling, staging and schedule (bf16 matrix cores, no block scales), so the
 * FP8 / BF16 speedup can be measured kernel for kernel:
 *
 *   c  bf16 [M][N]  = a . b^T, FP32 accumulation, rounded to nearest even
 *   a  bf16 [M][K]  K-contiguous
 *   b  bf16 [N][K]  K-contiguous (for DGRAD / WGRAD pass the transposed
 *                   operands, as the FP8 path's transposed code copies do)
 *
 * Requires M >= 0, N > 0 and a multiple of 128, K > 0 and a multiple of 64,
 * K <= 2^23; pointers 16-byte aligned.  Few output tiles with a long K split
 * the contraction: the FP32 partials need a workspace of
 * puro_bf16_gemm_nt_workspace_bytes(M, N, K) bytes (0 when not split).
 * Errors and streams as for puro_fp8_gemm_blockscaled.
 * Defined by: the BF16 matmul the FP8 path replaces (arXiv report section
 * 2.1; blog section "FP8").
 */
size_t puro_bf16_gemm_nt_workspace_bytes(int64_t M, int64_t N, int64_t K);
puro_status_t puro_bf16_gemm_nt(int64_t M, int64_t N, int64_t K, const void* a, const void* b,
                                void* c, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PURO_FP8_H */
