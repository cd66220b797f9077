// abi_consumer.cpp -- the C ABI of libpuro_fp8.so used from a plain host
// program: no Python, no PyTorch.  Device memory comes from the HIP runtime
// (hipMalloc); the library is called through include/puro_fp8.h only.
//
// One small linear layer, X [T x K] and W [N x K] in bf16 with a ragged token
// count: quant_act (row + transposed column codes), quant_weight (+ W^T),
// FWD Y = X . W^T with FP32 output, WGRAD dW = dY^T . X with FP32 output and
// DGRAD dX = dY . W with bf16 output, the last on a stream of its own.
// Codes and scales must equal the CPU oracle's bit for bit; the GEMM outputs
// must be within relative Frobenius error 1e-3 of the oracle's.  The oracle
// (oracle/puro_oracle.h) is test infrastructure and is linked here, by a
// test, never by the library.  Inputs come from a counter-based generator
// (splitmix64) defined in this file.
//
// Exit status 0 on success; the last line printed says what was checked.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "puro_fp8.h"
#include "puro_oracle.h"

namespace {

uint64_t splitmix64(uint64_t x)
{
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

// bf16 bit pattern of a value uniform in [-2, 2) (float value truncated to
// bf16; only the bit pattern matters, both sides read the same bytes)
uint16_t random_bf16(uint64_t stream, uint64_t i)
{
    const double u = (double)(splitmix64(stream * 0x100000000ull + i) >> 11) * 0x1p-53;
    const float f = (float)(4.0 * u - 2.0);
    uint32_t b;
    std::memcpy(&b, &f, 4);
    return (uint16_t)(b >> 16);
}

bool ok_hip(hipError_t e, const char* what)
{
    if (e != hipSuccess) {
        std::printf("FAIL %s: %s\n", what, hipGetErrorString(e));
        return false;
    }
    return true;
}

bool ok_puro(puro_status_t s, const char* what)
{
    if (s != PURO_OK) {
        std::printf("FAIL %s: %s\n", what, puro_fp8_status_string(s));
        return false;
    }
    return true;
}

template <typename T>
T* dev_alloc(size_t n)
{
    void* p = nullptr;
    if (hipMalloc(&p, n * sizeof(T) + 16) != hipSuccess)
        return nullptr;
    return static_cast<T*>(p);
}

template <typename T>
std::vector<T> to_host(const T* d, size_t n)
{
    std::vector<T> h(n);
    if (hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost) != hipSuccess)
        h.clear();
    return h;
}

// bf16 value nearest to f (ties to even), as a float; f is finite
float round_bf16(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    float r;
    std::memcpy(&r, &u, 4);
    return r;
}

double rel_fro(const std::vector<float>& got, const std::vector<float>& ref)
{
    double num = 0.0, den = 0.0;
    for (size_t i = 0; i < ref.size(); ++i) {
        const double d = (double)got[i] - (double)ref[i];
        num += d * d;
        den += (double)ref[i] * (double)ref[i];
    }
    return std::sqrt(num / (den > 0.0 ? den : 1.0));
}

}  // namespace

int main()
{
    const int64_t T = 300, K = 512, N = 384;
    const int64_t Tp = (T + 127) / 128 * 128;
    std::printf("abi_consumer: ABI version %d, T=%lld K=%lld N=%lld\n", puro_fp8_abi_version(),
                (long long)T, (long long)K, (long long)N);

    std::vector<uint16_t> x(T * K), w(N * K), dy(T * N);
    for (int64_t i = 0; i < T * K; ++i) x[i] = random_bf16(1, i);
    for (int64_t i = 0; i < N * K; ++i) w[i] = random_bf16(2, i);
    for (int64_t i = 0; i < T * N; ++i) dy[i] = random_bf16(3, i);

    uint16_t *dx = dev_alloc<uint16_t>(T * K), *dw = dev_alloc<uint16_t>(N * K), *ddy = dev_alloc<uint16_t>(T * N);
    uint8_t *qx = dev_alloc<uint8_t>(T * K), *qtx = dev_alloc<uint8_t>(K * Tp);
    uint8_t *qw = dev_alloc<uint8_t>(N * K), *qtw = dev_alloc<uint8_t>(K * N);
    uint8_t *qdy = dev_alloc<uint8_t>(T * N), *qtdy = dev_alloc<uint8_t>(N * Tp);
    float *sx = dev_alloc<float>((K / 128) * T), *stx = dev_alloc<float>((Tp / 128) * K);
    float *sw = dev_alloc<float>((N / 128) * (K / 128));
    float *sdy = dev_alloc<float>((N / 128) * T), *stdy = dev_alloc<float>((Tp / 128) * N);
    float *y = dev_alloc<float>(T * N), *gw = dev_alloc<float>(N * K);
    uint16_t* gx = dev_alloc<uint16_t>(T * K);
    if (!dx || !dw || !ddy || !qx || !qtx || !qw || !qtw || !qdy || !qtdy || !sx || !stx || !sw ||
        !sdy || !stdy || !y || !gw || !gx) {
        std::printf("FAIL hipMalloc\n");
        return 1;
    }
    if (!ok_hip(hipMemcpy(dx, x.data(), x.size() * 2, hipMemcpyHostToDevice), "copy x") ||
        !ok_hip(hipMemcpy(dw, w.data(), w.size() * 2, hipMemcpyHostToDevice), "copy w") ||
        !ok_hip(hipMemcpy(ddy, dy.data(), dy.size() * 2, hipMemcpyHostToDevice), "copy dy"))
        return 1;

    // garbage in the transposed copies: the library must write the padding
    // tokens T .. Tp-1 as zero codes itself (the WGRAD contracts over Tp)
    if (!ok_hip(hipMemset(qtx, 0xAB, K * Tp), "memset qtx") || !ok_hip(hipMemset(qtdy, 0xAB, N * Tp), "memset qtdy"))
        return 1;

    const size_t ws_bytes = puro_fp8_gemm_workspace_bytes(PURO_GEMM_WGRAD, N, K, Tp);
    void* ws = ws_bytes ? dev_alloc<uint8_t>(ws_bytes) : nullptr;
    if (ws_bytes && !ws) {
        std::printf("FAIL hipMalloc workspace\n");
        return 1;
    }
    if (!ok_puro(puro_fp8_quant_act(dx, T, K, qx, sx, qtx, stx, nullptr), "quant_act x") ||
        !ok_puro(puro_fp8_quant_weight(dw, N, K, qw, qtw, sw, nullptr), "quant_weight") ||
        !ok_puro(puro_fp8_quant_act(ddy, T, N, qdy, sdy, qtdy, stdy, nullptr), "quant_act dy") ||
        !ok_puro(puro_fp8_gemm_blockscaled(PURO_GEMM_FWD, T, N, K, qx, sx, qw, sw, y, PURO_OUT_FP32, 0,
                                           nullptr, 0, nullptr), "gemm fwd") ||
        !ok_puro(puro_fp8_gemm_blockscaled(PURO_GEMM_WGRAD, N, K, Tp, qtdy, stdy, qtx, stx, gw,
                                           PURO_OUT_FP32, 0, ws, ws_bytes, nullptr), "gemm wgrad"))
        return 1;
    if (!ok_hip(hipDeviceSynchronize(), "synchronize"))
        return 1;
    // DGRAD on a stream of its own (its inputs are complete after the sync)
    hipStream_t stream = nullptr;
    if (!ok_hip(hipStreamCreate(&stream), "stream create") ||
        !ok_puro(puro_fp8_gemm_blockscaled(PURO_GEMM_DGRAD, T, K, N, qdy, sdy, qtw, sw, gx, PURO_OUT_BF16,
                                           0, nullptr, 0, stream), "gemm dgrad") ||
        !ok_hip(hipStreamSynchronize(stream), "stream synchronize") ||
        !ok_hip(hipStreamDestroy(stream), "stream destroy"))
        return 1;

    // oracle
    std::vector<uint8_t> oqx(T * K), oqtx(K * Tp), oqw(N * K), oqtw(K * N), oqdy(T * N), oqtdy(N * Tp);
    std::vector<float> osx((K / 128) * T), ostx((Tp / 128) * K), osw((N / 128) * (K / 128));
    std::vector<float> osdy((N / 128) * T), ostdy((Tp / 128) * N), oy(T * N), ogw(N * K), ogx(T * K);
    if (orc_quant_rowwise(x.data(), T, K, oqx.data(), osx.data()) ||
        orc_quant_colwise(x.data(), T, K, oqtx.data(), ostx.data()) ||
        orc_quant_weight(w.data(), N, K, oqw.data(), oqtw.data(), osw.data()) ||
        orc_quant_rowwise(dy.data(), T, N, oqdy.data(), osdy.data()) ||
        orc_quant_colwise(dy.data(), T, N, oqtdy.data(), ostdy.data()) ||
        orc_gemm_blockscaled(0, T, N, K, oqx.data(), osx.data(), oqw.data(), osw.data(), oy.data(),
                             nullptr, 0, T) ||
        orc_gemm_blockscaled(2, N, K, Tp, oqtdy.data(), ostdy.data(), oqtx.data(), ostx.data(),
                             ogw.data(), nullptr, 0, N) ||
        orc_gemm_blockscaled(1, T, K, N, oqdy.data(), osdy.data(), oqtw.data(), osw.data(),
                             ogx.data(), nullptr, 0, T)) {
        std::printf("FAIL oracle\n");
        return 1;
    }

    struct Cmp {
        const char* what;
        std::vector<uint8_t> got, ref;
    };
    auto bytes_of = [](const std::vector<float>& v) {
        std::vector<uint8_t> b(v.size() * 4);
        std::memcpy(b.data(), v.data(), b.size());
        return b;
    };
    std::vector<Cmp> cmps = {
        {"q(x)", to_host(qx, T * K), oqx},
        {"qt(x)", to_host(qtx, K * Tp), oqtx},
        {"s(x)", bytes_of(to_host(sx, (K / 128) * T)), bytes_of(osx)},
        {"st(x)", bytes_of(to_host(stx, (Tp / 128) * K)), bytes_of(ostx)},
        {"q(w)", to_host(qw, N * K), oqw},
        {"qt(w)", to_host(qtw, K * N), oqtw},
        {"s(w)", bytes_of(to_host(sw, (N / 128) * (K / 128))), bytes_of(osw)},
        {"q(dy)", to_host(qdy, T * N), oqdy},
        {"qt(dy)", to_host(qtdy, N * Tp), oqtdy},
        {"s(dy)", bytes_of(to_host(sdy, (N / 128) * T)), bytes_of(osdy)},
        {"st(dy)", bytes_of(to_host(stdy, (Tp / 128) * N)), bytes_of(ostdy)},
    };
    for (const Cmp& c : cmps) {
        if (c.got.size() != c.ref.size() || std::memcmp(c.got.data(), c.ref.data(), c.ref.size()) != 0) {
            std::printf("FAIL %s differs from the oracle\n", c.what);
            return 1;
        }
    }
    const double e_fwd = rel_fro(to_host(y, T * N), oy);
    const double e_wgrad = rel_fro(to_host(gw, N * K), ogw);
    std::vector<float> gx32(T * K);
    {
        const std::vector<uint16_t> g = to_host(gx, T * K);
        for (size_t i = 0; i < gx32.size() && i < g.size(); ++i) {
            const uint32_t b = (uint32_t)g[i] << 16;
            std::memcpy(&gx32[i], &b, 4);
        }
    }
    for (float& v : ogx)
        v = round_bf16(v);            // the bf16 output is the RNE of the FP32 result
    const double e_dgrad = rel_fro(gx32, ogx);
    std::printf("rel_fro fwd %.3e wgrad %.3e dgrad(bf16) %.3e\n", e_fwd, e_wgrad, e_dgrad);
    if (!(e_fwd <= 1e-3) || !(e_wgrad <= 1e-3) || !(e_dgrad <= 1e-3)) {
        std::printf("FAIL GEMM error above 1e-3\n");
        return 1;
    }
    for (void* p : {(void*)dx, (void*)dw, (void*)ddy, (void*)qx, (void*)qtx, (void*)qw, (void*)qtw,
                    (void*)qdy, (void*)qtdy, (void*)sx, (void*)stx, (void*)sw, (void*)sdy,
                    (void*)stdy, (void*)y, (void*)gw, (void*)gx, ws})
        if (p)
            (void)hipFree(p);
    std::printf("abi_consumer ok: 11 code/scale buffers bit-exact, FWD and WGRAD (FP32) within 1e-3, "
                "DGRAD (bf16, own stream) within 1e-3 of the oracle rounded to bf16\n");
    return 0;
}
