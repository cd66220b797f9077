// abi.hip -- the extern "C" entry points declared in include/puro_fp8.h:
// argument validation (synchronous, before any enqueue), then the launch on
// the caller's stream.  No exception crosses the boundary.
#include "puro_fp8.h"

#include <hip/hip_runtime.h>

#include <limits>

#include "launch.hpp"

namespace {

constexpr int64_t kMaxDim = std::numeric_limits<int32_t>::max();
// The GEMM addresses a row of a 256-row tile with a 32-bit offset
// row * K + k from the tile's 64-bit base, so K is limited to 2^24.
constexpr int64_t kMaxGemmK = int64_t(1) << 24;
// DGRAD_W and FWD_T stage four B rows per copy with a 32-bit lane offset
// (row * N + column < 4 N).
constexpr int64_t kMaxDgradWN = int64_t(1) << 29;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

puro_status_t from_hip(hipError_t e) { return e == hipSuccess ? PURO_OK : PURO_ERR_HIP; }

template <typename F>
puro_status_t guarded(F&& f)
{
    try {
        return f();
    } catch (...) {
        return PURO_ERR_INTERNAL;
    }
}

puro_status_t check_act(const void* x, int64_t rows, int64_t cols, const uint8_t* q,
                        const float* s, const uint8_t* qt, const float* st)
{
    if (rows < 0 || cols <= 0 || cols % 128 != 0 || cols > kMaxDim)
        return PURO_ERR_BAD_SHAPE;
    // grid limit: one work-group per 128x128 block, a 1-D grid (each factor
    // is bounded first so the product cannot overflow)
    if (rows > kMaxDim * 128 || ((rows + 127) / 128) * (cols / 128) > kMaxDim)
        return PURO_ERR_BAD_SHAPE;
    if (rows == 0)
        return PURO_OK;                      // empty input: nothing to do
    if (!x)
        return PURO_ERR_NULL_POINTER;
    const bool row = q || s, col = qt || st;
    if (!row && !col)
        return PURO_ERR_NULL_POINTER;
    if ((q == nullptr) != (s == nullptr) || (qt == nullptr) != (st == nullptr))
        return PURO_ERR_NULL_POINTER;
    if (!aligned16(x) || (q && !aligned16(q)) || (s && !aligned16(s)) || (qt && !aligned16(qt)) ||
        (st && !aligned16(st)))
        return PURO_ERR_MISALIGNED;
    return PURO_OK;
}

puro_status_t check_weight(const void* w, int64_t n, int64_t k, const uint8_t* q,
                           const uint8_t* qt, const float* s)
{
    if (n <= 0 || k <= 0 || n % 128 != 0 || k % 128 != 0 || n > kMaxDim || k > kMaxDim ||
        (n / 128) * (k / 128) > kMaxDim)
        return PURO_ERR_BAD_SHAPE;
    if (!w || !s || (!q && !qt))
        return PURO_ERR_NULL_POINTER;
    if (!aligned16(w) || (q && !aligned16(q)) || !aligned16(s) || (qt && !aligned16(qt)))
        return PURO_ERR_MISALIGNED;
    return PURO_OK;
}

// Quantize-on-produce outputs: rows x out_cols, the layouts of check_act.
// `in_ok` is false when a required input pointer is NULL.
puro_status_t check_produce(bool in_ok, bool in_aligned, int64_t rows, int64_t out_cols,
                            const uint8_t* q, const float* s, const uint8_t* qt, const float* st,
                            const void* y)
{
    if (rows < 0 || out_cols <= 0 || out_cols % 128 != 0 || out_cols > kMaxDim)
        return PURO_ERR_BAD_SHAPE;
    if (rows > kMaxDim * 128 || ((rows + 127) / 128) * (out_cols / 128) > kMaxDim)
        return PURO_ERR_BAD_SHAPE;
    if (rows == 0)
        return PURO_OK;
    if (!in_ok)
        return PURO_ERR_NULL_POINTER;
    if ((q == nullptr) != (s == nullptr) || (qt == nullptr) != (st == nullptr))
        return PURO_ERR_NULL_POINTER;
    if (!q && !qt && !y)
        return PURO_ERR_NULL_POINTER;
    if (!in_aligned || (q && !aligned16(q)) || (s && !aligned16(s)) || (qt && !aligned16(qt)) ||
        (st && !aligned16(st)) || (y && !aligned16(y)))
        return PURO_ERR_MISALIGNED;
    return PURO_OK;
}

bool gemm_shape_ok(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N <= 0 || K <= 0 || N % 128 != 0 || K % 128 != 0)
        return false;
    if (M > kMaxDim || N > kMaxDim || K > kMaxGemmK)
        return false;
    // the launch grid holds tiles_m * tiles_n * splits work-groups (int)
    const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
    return tiles * 8 <= kMaxDim;
}

// BF16 comparator: K counts bf16 elements (2 bytes); the kernel's K-block is
// 128 bytes, i.e. 64 elements.
bool bf16_shape_ok(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N <= 0 || K <= 0 || N % 128 != 0 || K % 64 != 0)
        return false;
    if (M > kMaxDim || N > kMaxDim || 2 * K > kMaxGemmK)
        return false;
    const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
    return tiles * 8 <= kMaxDim;
}

}  // namespace

extern "C" {

puro_status_t puro_fp8_quant_act(const void* x, int64_t rows, int64_t cols, uint8_t* q, float* s,
                                 uint8_t* qt, float* st, void* stream)
{
    return guarded([&]() -> puro_status_t {
        const puro_status_t rc = check_act(x, rows, cols, q, s, qt, st);
        if (rc != PURO_OK || rows == 0)
            return rc;
        return from_hip(puro::launch_quant_act(x, rows, cols, q, s, qt, st,
                                               static_cast<hipStream_t>(stream)));
    });
}

puro_status_t puro_fp8_quant_weight(const void* w, int64_t n, int64_t k, uint8_t* q, uint8_t* qt,
                                    float* s, void* stream)
{
    return guarded([&]() -> puro_status_t {
        const puro_status_t rc = check_weight(w, n, k, q, qt, s);
        if (rc != PURO_OK)
            return rc;
        return from_hip(puro::launch_quant_weight(w, n, k, q, qt, s,
                                                  static_cast<hipStream_t>(stream)));
    });
}

puro_status_t puro_fp8_quant_weight_grouped(const puro_fp8_weight_desc* descs, int count,
                                            void* stream)
{
    return guarded([&]() -> puro_status_t {
        static_assert(PURO_FP8_MAX_GROUPED_WEIGHTS == puro::kMaxGroupedWeights, "group size");
        if (count < 0 || count > PURO_FP8_MAX_GROUPED_WEIGHTS)
            return PURO_ERR_BAD_SHAPE;
        if (count == 0)
            return PURO_OK;
        if (!descs)
            return PURO_ERR_NULL_POINTER;
        puro::WeightJob jobs[puro::kMaxGroupedWeights];
        int64_t blocks = 0;
        for (int i = 0; i < count; ++i) {
            const puro_fp8_weight_desc& d = descs[i];
            const puro_status_t rc = check_weight(d.w, d.n, d.k, d.q, d.qt, d.s);
            if (rc != PURO_OK)
                return rc;
            blocks += (d.n / 128) * (d.k / 128);
            jobs[i] = puro::WeightJob{static_cast<const uint16_t*>(d.w), d.n, d.k, d.q, d.qt, d.s};
        }
        if (blocks > kMaxDim)       // one work-group per block, a 1-D grid
            return PURO_ERR_BAD_SHAPE;
        return from_hip(puro::launch_quant_weight_grouped(jobs, count,
                                                          static_cast<hipStream_t>(stream)));
    });
}

puro_status_t puro_fp8_swiglu_quant(const void* gu, int64_t rows, int64_t f, uint8_t* q,
                                    float* s, uint8_t* qt, float* st, void* y, void* stream)
{
    return guarded([&]() -> puro_status_t {
        if (f > kMaxDim / 2)
            return PURO_ERR_BAD_SHAPE;
        const puro_status_t rc = check_produce(gu != nullptr, aligned16(gu), rows, f, q, s, qt, st, y);
        if (rc != PURO_OK || rows == 0)
            return rc;
        return from_hip(puro::launch_swiglu_quant(gu, rows, f, q, s, qt, st, y,
                                                  static_cast<hipStream_t>(stream)));
    });
}

puro_status_t puro_fp8_swiglu_bwd_quant(const void* dh, const void* gu, int64_t rows, int64_t f,
                                        uint8_t* q, float* s, uint8_t* qt, float* st, void* y,
                                        void* stream)
{
    return guarded([&]() -> puro_status_t {
        if (f <= 0 || f % 128 != 0 || f > kMaxDim / 2)
            return PURO_ERR_BAD_SHAPE;
        const puro_status_t rc = check_produce(dh && gu, aligned16(dh) && aligned16(gu), rows,
                                               2 * f, q, s, qt, st, y);
        if (rc != PURO_OK || rows == 0)
            return rc;
        return from_hip(puro::launch_swiglu_bwd_quant(dh, gu, rows, f, q, s, qt, st, y,
                                                      static_cast<hipStream_t>(stream)));
    });
}

puro_status_t puro_fp8_rmsnorm_quant(const void* x, const void* gamma, int64_t rows, int64_t cols,
                                     float eps, float* rstd, uint8_t* q, float* s, uint8_t* qt,
                                     float* st, void* y, void* stream)
{
    return guarded([&]() -> puro_status_t {
        const puro_status_t rc = check_produce(x && gamma && rstd,
                                               aligned16(x) && aligned16(gamma) && aligned16(rstd),
                                               rows, cols, q, s, qt, st, y);
        if (rc != PURO_OK)
            return rc;
        if ((rows + 3) / 4 > kMaxDim)        // the statistics pass runs 4 rows per work-group
            return PURO_ERR_BAD_SHAPE;
        if (!(eps >= 0.0f) || eps > std::numeric_limits<float>::max())
            return PURO_ERR_BAD_VALUE;
        if (rows == 0)
            return PURO_OK;
        return from_hip(puro::launch_rmsnorm_quant(x, gamma, rows, cols, eps, rstd, q, s, qt, st,
                                                   y, static_cast<hipStream_t>(stream)));
    });
}

size_t puro_fp8_gemm_workspace_bytes(puro_gemm_mode_t mode, int64_t M, int64_t N, int64_t K)
{
    if ((int)mode < 0 || (int)mode > 4 || !gemm_shape_ok(M, N, K) || M == 0)
        return 0;
    return puro::gemm_workspace_bytes((int)mode, M, N, K);
}

puro_status_t puro_fp8_gemm_blockscaled(puro_gemm_mode_t mode, int64_t M, int64_t N, int64_t K,
                                        const uint8_t* a, const float* sa, const uint8_t* b,
                                        const float* sb, void* c, puro_out_dtype_t c_dtype,
                                        int accumulate, void* workspace, size_t workspace_bytes,
                                        void* stream)
{
    return guarded([&]() -> puro_status_t {
        if ((int)mode < 0 || (int)mode > 4)
            return PURO_ERR_BAD_ENUM;
        if ((int)c_dtype != PURO_OUT_BF16 && (int)c_dtype != PURO_OUT_FP32)
            return PURO_ERR_BAD_ENUM;
        if (accumulate && c_dtype != PURO_OUT_FP32)
            return PURO_ERR_BAD_ENUM;
        if (!gemm_shape_ok(M, N, K) || ((mode == PURO_GEMM_DGRAD_W || mode == PURO_GEMM_FWD_T) && N > kMaxDgradWN))
            return PURO_ERR_BAD_SHAPE;
        if (M == 0)
            return PURO_OK;
        if (!a || !sa || !b || !sb || !c)
            return PURO_ERR_NULL_POINTER;
        if (!aligned16(a) || !aligned16(sa) || !aligned16(b) || !aligned16(sb) || !aligned16(c))
            return PURO_ERR_MISALIGNED;
        const size_t need = puro::gemm_workspace_bytes((int)mode, M, N, K);
        if (need > 0) {
            if (!workspace || workspace_bytes < need)
                return PURO_ERR_WORKSPACE;
            if (!aligned16(workspace))
                return PURO_ERR_MISALIGNED;
        }
        return from_hip(puro::launch_gemm((int)mode, M, N, K, a, sa, b, sb, c,
                                          c_dtype == PURO_OUT_FP32, accumulate ? 1 : 0, workspace,
                                          static_cast<hipStream_t>(stream)));
    });
}

puro_status_t puro_fp8_gemm_blockscaled_noalloc(puro_gemm_mode_t mode, int64_t M, int64_t N,
                                                int64_t K, const uint8_t* a, const float* sa,
                                                const uint8_t* b, const float* sb, void* c,
                                                puro_out_dtype_t c_dtype, int accumulate,
                                                void* stream)
{
    return guarded([&]() -> puro_status_t {
        if ((int)mode < 0 || (int)mode > 4)
            return PURO_ERR_BAD_ENUM;
        if ((int)c_dtype != PURO_OUT_BF16 && (int)c_dtype != PURO_OUT_FP32)
            return PURO_ERR_BAD_ENUM;
        if (accumulate && c_dtype != PURO_OUT_FP32)
            return PURO_ERR_BAD_ENUM;
        if (!gemm_shape_ok(M, N, K) || ((mode == PURO_GEMM_DGRAD_W || mode == PURO_GEMM_FWD_T) && N > kMaxDgradWN))
            return PURO_ERR_BAD_SHAPE;
        if (M == 0)
            return PURO_OK;
        if (!a || !sa || !b || !sb || !c)
            return PURO_ERR_NULL_POINTER;
        if (!aligned16(a) || !aligned16(sa) || !aligned16(b) || !aligned16(sb) || !aligned16(c))
            return PURO_ERR_MISALIGNED;
        if (puro::gemm_workspace_bytes((int)mode, M, N, K) > puro::gemm_noalloc_scratch_bytes())
            return PURO_ERR_WORKSPACE;
        return from_hip(puro::launch_gemm_noalloc((int)mode, M, N, K, a, sa, b, sb, c,
                                                  c_dtype == PURO_OUT_FP32, accumulate ? 1 : 0,
                                                  static_cast<hipStream_t>(stream)));
    });
}

size_t puro_bf16_gemm_nt_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (!bf16_shape_ok(M, N, K) || M == 0)
        return 0;
    return puro::gemm_bf16_workspace_bytes(M, N, K);
}

puro_status_t puro_bf16_gemm_nt(int64_t M, int64_t N, int64_t K, const void* a, const void* b,
                                void* c, void* workspace, size_t workspace_bytes, void* stream)
{
    return guarded([&]() -> puro_status_t {
        if (!bf16_shape_ok(M, N, K))
            return PURO_ERR_BAD_SHAPE;
        if (M == 0)
            return PURO_OK;
        if (!a || !b || !c)
            return PURO_ERR_NULL_POINTER;
        if (!aligned16(a) || !aligned16(b) || !aligned16(c))
            return PURO_ERR_MISALIGNED;
        const size_t need = puro::gemm_bf16_workspace_bytes(M, N, K);
        if (need > 0) {
            if (!workspace || workspace_bytes < need)
                return PURO_ERR_WORKSPACE;
            if (!aligned16(workspace))
                return PURO_ERR_MISALIGNED;
        }
        return from_hip(puro::launch_gemm_bf16_nt(M, N, K, a, b, c, workspace,
                                                  static_cast<hipStream_t>(stream)));
    });
}

puro_status_t puro_fp8_rmsnorm_quant_rstd(const void* x, const void* gamma, const float* rstd,
                                          int64_t rows, int64_t cols, uint8_t* q, float* s,
                                          uint8_t* qt, float* st, void* y, void* stream)
{
    return guarded([&]() -> puro_status_t {
        const puro_status_t rc = check_produce(x && gamma && rstd,
                                               aligned16(x) && aligned16(gamma) && aligned16(rstd),
                                               rows, cols, q, s, qt, st, y);
        if (rc != PURO_OK || rows == 0)
            return rc;
        return from_hip(puro::launch_rmsnorm_quant_rstd(x, gamma, rstd, rows, cols, q, s, qt, st,
                                                        y, static_cast<hipStream_t>(stream)));
    });
}

puro_status_t puro_fp8_rmsnorm_bwd_quant(const void* dy, const void* x, const void* gamma,
                                         const float* rstd, const void* gin, int64_t rows,
                                         int64_t cols, float* coef, uint8_t* q, float* s,
                                         uint8_t* qt, float* st, void* y, void* stream)
{
    return guarded([&]() -> puro_status_t {
        const puro_status_t rc =
            check_produce(dy && x && gamma && rstd && coef,
                          aligned16(dy) && aligned16(x) && aligned16(gamma) && aligned16(rstd) &&
                              aligned16(coef) && (!gin || aligned16(gin)),
                          rows, cols, q, s, qt, st, y);
        if (rc != PURO_OK)
            return rc;
        if ((rows + 3) / 4 > kMaxDim)        // the statistics pass runs 4 rows per work-group
            return PURO_ERR_BAD_SHAPE;
        if (rows == 0)
            return PURO_OK;
        return from_hip(puro::launch_rmsnorm_bwd_quant(dy, x, gamma, rstd, gin, rows, cols, coef,
                                                       q, s, qt, st, y,
                                                       static_cast<hipStream_t>(stream)));
    });
}

puro_status_t puro_bf16_residual_add_rstd(const void* a, const void* b, int64_t rows, int64_t cols,
                                     float eps, void* h, float* rstd, void* stream)
{
    return guarded([&]() -> puro_status_t {
        if (rows < 0 || cols <= 0 || cols % 128 != 0 || cols > kMaxDim || (rows + 3) / 4 > kMaxDim)
            return PURO_ERR_BAD_SHAPE;
        if (rows == 0)
            return PURO_OK;
        if (!a || !b || !h || !rstd)
            return PURO_ERR_NULL_POINTER;
        if (!aligned16(a) || !aligned16(b) || !aligned16(h) || !aligned16(rstd))
            return PURO_ERR_MISALIGNED;
        if (!(eps >= 0.0f) || eps > std::numeric_limits<float>::max())
            return PURO_ERR_BAD_VALUE;
        return from_hip(puro::launch_residual_rstd(a, b, rows, cols, eps, h, rstd,
                                                   static_cast<hipStream_t>(stream)));
    });
}

puro_status_t puro_fp8_probe_encode(uint32_t first_bits, int64_t n, uint8_t* out, void* stream)
{
    return guarded([&]() -> puro_status_t {
        if (n < 0)
            return PURO_ERR_BAD_SHAPE;
        if (n == 0)
            return PURO_OK;
        if (!out)
            return PURO_ERR_NULL_POINTER;
        return from_hip(puro::launch_probe_encode(first_bits, n, out,
                                                  static_cast<hipStream_t>(stream)));
    });
}

puro_status_t puro_fp8_probe_sigmoid(uint32_t first_bits, int64_t n, int form, float* out,
                                     void* stream)
{
    return guarded([&]() -> puro_status_t {
        if (form < 0 || form > 2)
            return PURO_ERR_BAD_ENUM;
        if (n < 0)
            return PURO_ERR_BAD_SHAPE;
        if (n == 0)
            return PURO_OK;
        if (!out)
            return PURO_ERR_NULL_POINTER;
        if ((reinterpret_cast<uintptr_t>(out) & 3u) != 0)
            return PURO_ERR_MISALIGNED;
        return from_hip(puro::launch_probe_sigmoid(first_bits, n, form, out,
                                                   static_cast<hipStream_t>(stream)));
    });
}

puro_status_t puro_fp8_probe_mfma(int form, const uint8_t* a, const uint8_t* b, int scale_a,
                                  int scale_b, float* d, void* stream)
{
    return guarded([&]() -> puro_status_t {
        if (form < 0 || form > 5)
            return PURO_ERR_BAD_ENUM;
        if (!a || !b || !d)
            return PURO_ERR_NULL_POINTER;
        if (!aligned16(a) || !aligned16(b) || !aligned16(d))
            return PURO_ERR_MISALIGNED;
        if (scale_a < 0 || scale_a > 255 || scale_b < 0 || scale_b > 255)
            return PURO_ERR_BAD_VALUE;
        return from_hip(puro::launch_probe_mfma(form, a, b, scale_a, scale_b, d,
                                                static_cast<hipStream_t>(stream)));
    });
}

const char* puro_fp8_status_string(puro_status_t status)
{
    switch (status) {
    case PURO_OK:                return "PURO_OK: success";
    case PURO_ERR_NULL_POINTER:  return "PURO_ERR_NULL_POINTER: a required pointer is NULL";
    case PURO_ERR_BAD_SHAPE:     return "PURO_ERR_BAD_SHAPE: size out of range or not a multiple of 128";
    case PURO_ERR_MISALIGNED:    return "PURO_ERR_MISALIGNED: a pointer is not 16-byte aligned";
    case PURO_ERR_BAD_ENUM:      return "PURO_ERR_BAD_ENUM: unknown mode or dtype, or a bad combination";
    case PURO_ERR_WORKSPACE:     return "PURO_ERR_WORKSPACE: workspace smaller than required";
    case PURO_ERR_UNIMPLEMENTED: return "PURO_ERR_UNIMPLEMENTED: not supported by this library version";
    case PURO_ERR_HIP:           return "PURO_ERR_HIP: the HIP runtime rejected a launch";
    case PURO_ERR_INTERNAL:      return "PURO_ERR_INTERNAL: unexpected internal failure";
    case PURO_ERR_BAD_VALUE:     return "PURO_ERR_BAD_VALUE: a scalar argument is out of range";
    }
    return "unknown puro_status_t";
}

int puro_fp8_abi_version(void) { return PURO_FP8_ABI_VERSION; }

}  // extern "C"
