// produce.hip -- quantize-on-produce for gfx950: the BF16 neighbour ops of
// the FP8 GEMMs compute their bf16 output in registers and quantize it there,
// so the operand never makes a bf16 round trip through HBM.
//
// The pages put only the main linear-layer GEMMs on FP8 and keep the other
// ops in BF16 (arXiv report "Puro-2B" section 2.1; training.farm blog section
// "FP8").  Each kernel here therefore rounds the op's FP32 result to bf16
// (nearest even) first and quantizes that bf16 value, so its codes and scales
// are those of quant_act applied to the op's bf16 output:
//   - SwiGLU forward: h = silu(gate) * up, gate | up concatenated as the
//     fused up+gate projection writes them (gu [rows][2f], gate first); h is
//     the down projection's input X.
//   - SwiGLU backward: d gate = dh * up * silu'(gate), d up = dh * silu(gate),
//     written as dgu [rows][2f] (d gate first): the up+gate projection's
//     output gradient dY.
//   - RMSNorm forward: y = x * rstd * gamma, rstd = 1/sqrt(mean(x^2) + eps):
//     the input X of the projection after the norm.
// Each can also write the bf16 result itself (what the unfused op writes).
//
// Work decomposition, block walk and code layout are those of the plain
// activation quantizer (quant_block.hpp): one 256-thread work-group per
// 128x128 output block.  SwiGLU backward takes one 128x128 block of h
// columns and quantizes the two output blocks it yields (d gate and d up), so
// dh, gate and up are read once.
#include "launch.hpp"
#include "quant_block.hpp"

namespace puro {

// e^t in FP32 with Cody and Waite's split-constant argument reduction
// (Software Manual for the Elementary Functions, 1980): log2(e) is held as
// LOG2E_HI + LOG2E_LO (the FP32 rounding of log2 e and the FP32 rounding of
// the rest), t * log2(e) is formed as the unevaluated sum y_hi + y_lo (the
// rounding error of t * LOG2E_HI recovered exactly by an FMA), and
// e^t = 2^y_hi * 2^y_lo with the hardware 2^x (v_exp_f32) for 2^y_hi and
// 1 + y_lo * ln 2 for 2^y_lo (|y_lo| < 2^-17 for |t| < 128, so dropping the
// quadratic term costs less than 2^-34).  The last step multiplies by
// (1 + y_lo * ln 2) rather than adding r * y_lo * ln 2, so that r = inf (t
// above ~88.7) stays inf instead of becoming inf - inf.  Measured on the
// device over every FP32 t in [-104, 88.7] with a normal result: within
// 3.3 * 2^-24 of e^t.  It costs 6 instructions where the math library's
// expf costs about 13; the bare 2^(t * log2 e) would cost 2, but rounding
// t * log2 e carries |t| * 2^-24 into the exponent.
__device__ __forceinline__ float exp_f32(float t)
{
    constexpr float kLog2eHi = 0x1.715476p+0f;      // RN32(log2 e)
    constexpr float kLog2eLo = 0x1.4ae0cp-26f;      // RN32(log2 e - kLog2eHi)
    constexpr float kLn2 = 0x1.62e430p-1f;          // RN32(ln 2)
    const float y_hi = t * kLog2eHi;
    const float y_lo = fmaf(t, kLog2eLo, fmaf(t, kLog2eHi, -y_hi));
    const float r = __builtin_amdgcn_exp2f(y_hi);
    return r * (1.0f + y_lo * kLn2);
}

// sigmoid(g) = 1 / (1 + e^-g) in FP32: exp_f32, then the hardware
// reciprocal (within 1 ulp).  A relative error of e^-g reaches sigmoid damped
// by e^-g / (1 + e^-g), so sigmoid stays within about 5 units of 2^-24 for
// every g (measured over every FP32 g in [-88, 88] with a normal result:
// 4.1 * 2^-24); for g below about -88.7 the exponential overflows and the
// result is 0.
__device__ __forceinline__ float sigmoid_f32(float g)
{
    return __builtin_amdgcn_rcpf(1.0f + exp_f32(-g));
}

// The sigmoid on consecutive FP32 bit patterns (puro_fp8_probe_sigmoid).
__global__ __launch_bounds__(256) void probe_sigmoid_kernel(uint32_t first, int64_t n, float* out)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
        out[i] = sigmoid_f32(__uint_as_float(first + (uint32_t)i));
}

__device__ __forceinline__ uint4 load16(const uint16_t* p)
{
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ void store16(uint16_t* p, const uint4& v)
{
    *reinterpret_cast<uint4*>(p) = v;
}

// Eight bf16 words of an op applied lane-wise to one, two or three inputs of
// eight bf16 values each; `fn(a, b, c)` returns the FP32 result.
template <typename Fn>
__device__ __forceinline__ uint4 map8(const uint4& a, const uint4& b, const uint4& c, Fn fn)
{
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
    const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = pack_bf16(fn(bf16_lo(aw[i]), bf16_lo(bw[i]), bf16_lo(cw[i])),
                         fn(bf16_hi(aw[i]), bf16_hi(bw[i]), bf16_hi(cw[i])));
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// h = silu(g) * u = (g * sigmoid(g)) * u.
struct SwigluH {
    __device__ float operator()(float g, float u, float) const
    {
        return (g * sigmoid_f32(g)) * u;
    }
};

// d gate = ((dh * u) * sigmoid(g)) * (1 + g * (1 - sigmoid(g))).
struct SwigluDGate {
    __device__ float operator()(float g, float u, float dh) const
    {
        const float sg = sigmoid_f32(g);
        return ((dh * u) * sg) * __builtin_fmaf(g, 1.0f - sg, 1.0f);
    }
};

// d up = dh * (g * sigmoid(g)).
struct SwigluDUp {
    __device__ float operator()(float g, float, float dh) const
    {
        return dh * (g * sigmoid_f32(g));
    }
};

constexpr uint4 kZero4 = {0u, 0u, 0u, 0u};

// ---- SwiGLU forward ---------------------------------------------------------

template <bool ROW, bool COL, bool STORE_Y>
__global__ __launch_bounds__(256) void swiglu_quant_kernel(
    const uint16_t* __restrict__ gu, int64_t rows, int64_t f, int64_t ld_t,
    uint8_t* __restrict__ q, float* __restrict__ s, uint8_t* __restrict__ qt,
    float* __restrict__ st, uint16_t* __restrict__ h, int group_rows)
{
    __shared__ QuantLds<ROW, COL, false, false> lds;
    const int t = threadIdx.x;
    const BlockRC b = block_of(blockIdx.x, ld_t / 128, f / 128, group_rows);
    const int64_t row0 = b.rb * 128 + 8 * (t >> 4);
    const int64_t col0 = b.cb * 128 + 8 * (t & 15);

    uint4 gv[8], uv[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int64_t r = row0 + p;
        gv[p] = r < rows ? load16(gu + r * 2 * f + col0) : kZero4;
        uv[p] = r < rows ? load16(gu + r * 2 * f + f + col0) : kZero4;
    }
    uint4 v[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        // rows past the end hold zeros (silu(0) * 0 = +0), as the body requires
        v[p] = row0 + p < rows ? map8(gv[p], uv[p], kZero4, SwigluH{}) : kZero4;
        if (STORE_Y && row0 + p < rows)
            store16(h + (row0 + p) * f + col0, v[p]);
    }
    if constexpr (ROW || COL)
        quant_block_body<ROW, COL, false, false>(v, rows, f, ld_t, b.rb, b.cb, q, s, qt, st, lds);
}

// ---- SwiGLU backward --------------------------------------------------------

template <bool ROW, bool COL, bool STORE_Y>
__global__ __launch_bounds__(256) void swiglu_bwd_quant_kernel(
    const uint16_t* __restrict__ dh, const uint16_t* __restrict__ gu, int64_t rows, int64_t f,
    int64_t ld_t, uint8_t* __restrict__ q, float* __restrict__ s, uint8_t* __restrict__ qt,
    float* __restrict__ st, uint16_t* __restrict__ dgu, int group_rows)
{
    __shared__ QuantLds<ROW, COL, false, false> lds;
    const int t = threadIdx.x;
    const BlockRC b = block_of(blockIdx.x, ld_t / 128, f / 128, group_rows);
    const int64_t row0 = b.rb * 128 + 8 * (t >> 4);
    const int64_t col0 = b.cb * 128 + 8 * (t & 15);

    uint4 dg[8], du[8];
    {
        uint4 dv[8], gv[8], uv[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int64_t r = row0 + p;
            dv[p] = r < rows ? load16(dh + r * f + col0) : kZero4;
            gv[p] = r < rows ? load16(gu + r * 2 * f + col0) : kZero4;
            uv[p] = r < rows ? load16(gu + r * 2 * f + f + col0) : kZero4;
        }
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const bool in = row0 + p < rows;
            dg[p] = in ? map8(gv[p], uv[p], dv[p], SwigluDGate{}) : kZero4;
            du[p] = in ? map8(gv[p], uv[p], dv[p], SwigluDUp{}) : kZero4;
            if (STORE_Y && in) {
                store16(dgu + (row0 + p) * 2 * f + col0, dg[p]);
                store16(dgu + (row0 + p) * 2 * f + f + col0, du[p]);
            }
        }
    }
    if constexpr (ROW || COL) {
        quant_block_body<ROW, COL, false, false>(dg, rows, 2 * f, ld_t, b.rb, b.cb, q, s, qt, st,
                                                 lds);
        __syncthreads();   // the second block reuses the LDS
        quant_block_body<ROW, COL, false, false>(du, rows, 2 * f, ld_t, b.rb, b.cb + f / 128, q, s,
                                                 qt, st, lds);
    }
}

// ---- RMSNorm forward --------------------------------------------------------

// rstd[r] = 1 / sqrt(mean over c of x[r][c]^2 + eps), one wave per row.  Each
// lane keeps eight partial sums (one per element of its 16-byte loads) that
// are added pairwise and then across the wave, so no sum runs over more than
// cols/512 sequential terms.  The square root and division are IEEE
// correctly rounded (the library is built without fast-math).
__global__ __launch_bounds__(256) void rmsnorm_rstd_kernel(const uint16_t* __restrict__ x,
                                                           int64_t rows, int64_t cols, float eps,
                                                           float* __restrict__ rstd)
{
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows)
        return;
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t c = 8 * lane; c < cols; c += 512) {
        const uint4 v = load16(x + r * cols + c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = bf16_lo(w[i]), hi = bf16_hi(w[i]);
            acc[2 * i] = __builtin_fmaf(lo, lo, acc[2 * i]);
            acc[2 * i + 1] = __builtin_fmaf(hi, hi, acc[2 * i + 1]);
        }
    }
    float sum = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        sum += __shfl_xor(sum, off, 64);
    if (lane == 0)
        rstd[r] = 1.0f / sqrtf(sum / (float)cols + eps);
}

template <bool ROW, bool COL, bool STORE_Y>
__global__ __launch_bounds__(256) void rmsnorm_quant_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma,
    const float* __restrict__ rstd, int64_t rows, int64_t cols, int64_t ld_t,
    uint8_t* __restrict__ q, float* __restrict__ s, uint8_t* __restrict__ qt,
    float* __restrict__ st, uint16_t* __restrict__ y, int group_rows)
{
    __shared__ QuantLds<ROW, COL, false, false> lds;
    const int t = threadIdx.x;
    const BlockRC b = block_of(blockIdx.x, ld_t / 128, cols / 128, group_rows);
    const int64_t row0 = b.rb * 128 + 8 * (t >> 4);
    const int64_t col0 = b.cb * 128 + 8 * (t & 15);

    uint4 xv[8];
    float rs[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int64_t r = row0 + p;
        xv[p] = r < rows ? load16(x + r * cols + col0) : kZero4;
        rs[p] = r < rows ? rstd[r] : 0.0f;
    }
    const uint4 gv = load16(gamma + col0);
    uint4 v[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const float rp = rs[p];
        v[p] = row0 + p < rows
                   ? map8(xv[p], gv, kZero4, [rp](float xe, float ge, float) { return (xe * rp) * ge; })
                   : kZero4;
        if (STORE_Y && row0 + p < rows)
            store16(y + (row0 + p) * cols + col0, v[p]);
    }
    if constexpr (ROW || COL)
        quant_block_body<ROW, COL, false, false>(v, rows, cols, ld_t, b.rb, b.cb, q, s, qt, st,
                                                 lds);
}

// ---- launchers --------------------------------------------------------------

// Launches KERNEL<ROW, COL, STORE_Y> for the requested outputs (q, qt and
// yout are the launcher's output pointers; at least one is non-null) and
// evaluates to the launch's status.  ARGS is the parenthesized argument list.
#define PURO_EXPAND(...) __VA_ARGS__
#define PURO_DISPATCH_OUTPUTS(KERNEL, GRID, ARGS)                                              \
    [&]() -> hipError_t {                                                                      \
        const bool r_ = q != nullptr, c_ = qt != nullptr, y_ = yout != nullptr;                \
        const dim3 b_(256);                                                                    \
        if (r_ && c_ && y_)                                                                    \
            return launch_kernel(KERNEL<true, true, true>, GRID, b_, stream, PURO_EXPAND ARGS);  \
        if (r_ && c_)                                                                          \
            return launch_kernel(KERNEL<true, true, false>, GRID, b_, stream, PURO_EXPAND ARGS); \
        if (r_ && y_)                                                                          \
            return launch_kernel(KERNEL<true, false, true>, GRID, b_, stream, PURO_EXPAND ARGS); \
        if (r_)                                                                                \
            return launch_kernel(KERNEL<true, false, false>, GRID, b_, stream, PURO_EXPAND ARGS); \
        if (c_ && y_)                                                                          \
            return launch_kernel(KERNEL<false, true, true>, GRID, b_, stream, PURO_EXPAND ARGS); \
        if (c_)                                                                                \
            return launch_kernel(KERNEL<false, true, false>, GRID, b_, stream, PURO_EXPAND ARGS); \
        return launch_kernel(KERNEL<false, false, true>, GRID, b_, stream, PURO_EXPAND ARGS);    \
    }()

hipError_t launch_swiglu_quant(const void* gu, int64_t rows, int64_t f, uint8_t* q, float* s,
                               uint8_t* qt, float* st, void* yout, hipStream_t stream)
{
    const int64_t rows_pad = (rows + 127) / 128 * 128;
    const dim3 grid((unsigned)((rows_pad / 128) * (f / 128)));
    const uint16_t* g = static_cast<const uint16_t*>(gu);
    uint16_t* h = static_cast<uint16_t*>(yout);
    const int gr = quant_group_rows(false, f);
    return PURO_DISPATCH_OUTPUTS(swiglu_quant_kernel, grid,
                                 (g, rows, f, rows_pad, q, s, qt, st, h, gr));
}

hipError_t launch_swiglu_bwd_quant(const void* dh, const void* gu, int64_t rows, int64_t f,
                                   uint8_t* q, float* s, uint8_t* qt, float* st, void* yout,
                                   hipStream_t stream)
{
    const int64_t rows_pad = (rows + 127) / 128 * 128;
    const dim3 grid((unsigned)((rows_pad / 128) * (f / 128)));
    const uint16_t* d = static_cast<const uint16_t*>(dh);
    const uint16_t* g = static_cast<const uint16_t*>(gu);
    uint16_t* dgu = static_cast<uint16_t*>(yout);
    const int gr = quant_group_rows(false, 2 * f);
    return PURO_DISPATCH_OUTPUTS(swiglu_bwd_quant_kernel, grid,
                                 (d, g, rows, f, rows_pad, q, s, qt, st, dgu, gr));
}

hipError_t launch_rmsnorm_quant(const void* x, const void* gamma, int64_t rows, int64_t cols,
                                float eps, float* rstd, uint8_t* q, float* s, uint8_t* qt,
                                float* st, void* yout, hipStream_t stream)
{
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint16_t* gb = static_cast<const uint16_t*>(gamma);
    uint16_t* y = static_cast<uint16_t*>(yout);
    const hipError_t e = launch_kernel(rmsnorm_rstd_kernel, dim3((unsigned)((rows + 3) / 4)),
                                       dim3(256), stream, xb, rows, cols, eps, rstd);
    if (e != hipSuccess)
        return e;
    const int64_t rows_pad = (rows + 127) / 128 * 128;
    const dim3 grid((unsigned)((rows_pad / 128) * (cols / 128)));
    const int gr = quant_group_rows(false, cols);
    return PURO_DISPATCH_OUTPUTS(rmsnorm_quant_kernel, grid,
                                 (xb, gb, rstd, rows, cols, rows_pad, q, s, qt, st, y, gr));
}

hipError_t launch_probe_sigmoid(uint32_t first, int64_t n, float* out, hipStream_t stream)
{
    const int64_t blocks = (n + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
    return launch_kernel(probe_sigmoid_kernel, dim3(grid), dim3(256), stream, first, n, out);
}

#undef PURO_DISPATCH_OUTPUTS
#undef PURO_EXPAND

}  // namespace puro
