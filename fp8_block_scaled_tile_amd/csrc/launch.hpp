// launch.hpp -- internal host-side launchers (not part of the C ABI).  Each
// expects arguments already validated by the C entry points in abi.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>
#include <utility>

namespace puro {

// Launches `kernel` through hipLaunchKernel and returns that launch's own
// status.  (hipGetLastError after a triple-chevron launch reports the last
// error of any runtime call on the thread: it could blame the launch for an
// earlier, unrelated failure of the caller's, and would clear it.)  The
// arguments are converted to the kernel's parameter types first, as a
// triple-chevron launch converts them.
template <typename... P, typename... A>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream,
                         A&&... args)
{
    static_assert(sizeof...(P) == sizeof...(A) && sizeof...(P) > 0, "kernel argument count");
    std::tuple<std::decay_t<P>...> vals(static_cast<std::decay_t<P>>(std::forward<A>(args))...);
    return std::apply(
        [&](auto&... v) {
            void* ptrs[] = {const_cast<void*>(static_cast<const void*>(&v))...};
            return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0,
                                   stream);
        },
        vals);
}

hipError_t launch_quant_act(const void* x, int64_t rows, int64_t cols, uint8_t* q, float* s,
                            uint8_t* qt, float* st, hipStream_t stream);
hipError_t launch_quant_weight(const void* w, int64_t n, int64_t k, uint8_t* q, uint8_t* qt,
                               float* s, hipStream_t stream);
// One launch over several weights: d[i] = (w, n, k, q, qt, s) of one
// puro_fp8_quant_weight call each, count <= kMaxGroupedWeights.
constexpr int kMaxGroupedWeights = 16;
struct WeightJob {
    const uint16_t* w;
    int64_t n, k;
    uint8_t* q;
    uint8_t* qt;
    float* s;
};
hipError_t launch_quant_weight_grouped(const WeightJob* jobs, int count, hipStream_t stream);
hipError_t launch_swiglu_quant(const void* gu, int64_t rows, int64_t f, uint8_t* q, float* s,
                               uint8_t* qt, float* st, void* h, hipStream_t stream);
hipError_t launch_swiglu_bwd_quant(const void* dh, const void* gu, int64_t rows, int64_t f,
                                   uint8_t* q, float* s, uint8_t* qt, float* st, void* dgu,
                                   hipStream_t stream);
hipError_t launch_rmsnorm_quant(const void* x, const void* gamma, int64_t rows, int64_t cols,
                                float eps, float* rstd, uint8_t* q, float* s, uint8_t* qt,
                                float* st, void* y, hipStream_t stream);
hipError_t launch_rmsnorm_quant_rstd(const void* x, const void* gamma, const float* rstd,
                                     int64_t rows, int64_t cols, uint8_t* q, float* s,
                                     uint8_t* qt, float* st, void* y, hipStream_t stream);
hipError_t launch_rmsnorm_bwd_quant(const void* dy, const void* x, const void* gamma,
                                    const float* rstd, const void* gin, int64_t rows, int64_t cols,
                                    float* coef, uint8_t* q, float* s, uint8_t* qt, float* st,
                                    void* y, hipStream_t stream);
hipError_t launch_residual_rstd(const void* a, const void* b, int64_t rows, int64_t cols, float eps,
                                void* h, float* rstd, hipStream_t stream);
hipError_t launch_probe_encode(uint32_t first, int64_t n, uint8_t* out, hipStream_t stream);
hipError_t launch_probe_sigmoid(uint32_t first, int64_t n, int form, float* out,
                                hipStream_t stream);
hipError_t launch_probe_mfma(int form, const uint8_t* a, const uint8_t* b, int scale_a,
                             int scale_b, float* d, hipStream_t stream);

size_t gemm_workspace_bytes(int mode, int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm(int mode, int64_t M, int64_t N, int64_t K, const uint8_t* a,
                       const float* sa, const uint8_t* b, const float* sb, void* c, int out_fp32,
                       int accumulate, void* ws, hipStream_t stream);

size_t gemm_noalloc_scratch_bytes();
hipError_t launch_gemm_noalloc(int mode, int64_t M, int64_t N, int64_t K, const uint8_t* a,
                               const float* sa, const uint8_t* b, const float* sb, void* c,
                               int out_fp32, int accumulate, hipStream_t stream);

size_t gemm_bf16_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_bf16_nt(int64_t M, int64_t N, int64_t K, const void* a, const void* b,
                               void* c, void* ws, hipStream_t stream);

}  // namespace puro
