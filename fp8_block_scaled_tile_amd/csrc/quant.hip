// quant.hip -- tile-wise FP8 (E4M3) quantizers for gfx950: activations and
// gradients (1x128 row tiles and/or 128x1 column tiles with the transposed
// copy) and weights (128x128 blocks), each work-group loading one 128x128
// block of the bf16 input and quantizing it with quant_block_body.
#include "launch.hpp"
#include "quant_block.hpp"

namespace puro {

template <bool ROW, bool COL, bool WEIGHT, bool WT>
__global__ __launch_bounds__(256) void quant_block_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_t,
    uint8_t* __restrict__ q, float* __restrict__ s, uint8_t* __restrict__ qt,
    float* __restrict__ st, BlockWalk walk)
{
    __shared__ QuantLds<ROW, COL, WEIGHT, WT> lds;
    const int t = threadIdx.x;
    const BlockRC b = block_of(blockIdx.x, (WEIGHT ? rows : ld_t) / 128, cols / 128, walk);
    const int64_t row0 = b.rb * 128 + 8 * (t >> 4);
    const int64_t col0 = b.cb * 128 + 8 * (t & 15);

    // Every lane issues its eight 16-byte loads up front.  The input is read
    // from HBM exactly once whatever combination of outputs is requested.
    uint4 v[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int64_t r = row0 + p;
        if (r < rows)
            v[p] = *reinterpret_cast<const uint4*>(x + r * cols + col0);
        else
            v[p] = make_uint4(0u, 0u, 0u, 0u);
    }
    quant_block_body<ROW, COL, WEIGHT, WT>(v, rows, cols, ld_t, b.rb, b.cb, q, s, qt, st, lds);
}

// Several weights in one launch: work-group b takes block b - first[i] of
// weight i, first[i] <= b < first[i + 1] (a uniform scalar search over at
// most 16 entries), and quantizes it exactly as quant_block_kernel does for
// that weight alone (same block walk inside the weight, same body).  With WT,
// a weight whose qt is NULL skips the transposed copy.
struct WeightJobs {
    WeightJob j[kMaxGroupedWeights];
    int64_t first[kMaxGroupedWeights + 1];
    int count;
    int group_rows;
};

template <bool WT>
__global__ __launch_bounds__(256) void quant_weight_grouped_kernel(const WeightJobs jobs)
{
    __shared__ QuantLds<false, false, true, WT> lds;
    const int t = threadIdx.x;
    const int64_t bid = blockIdx.x;
    int i = 0;
    while (i + 1 < jobs.count && bid >= jobs.first[i + 1])
        ++i;
    const WeightJob J = jobs.j[i];
    const BlockRC b = block_of(bid - jobs.first[i], J.n / 128, J.k / 128, grouped_walk(jobs.group_rows));
    const int64_t row0 = b.rb * 128 + 8 * (t >> 4);
    const int64_t col0 = b.cb * 128 + 8 * (t & 15);
    uint4 v[8];
#pragma unroll
    for (int p = 0; p < 8; ++p)
        v[p] = *reinterpret_cast<const uint4*>(J.w + (row0 + p) * J.k + col0);
    quant_block_body<false, false, true, WT>(v, J.n, J.k, J.n, b.rb, b.cb, J.q, J.s, J.qt, nullptr,
                                            lds);
}

// Diagnostic: E4M3 code of every binary32 bit pattern first + i, i < n.
__global__ __launch_bounds__(256) void probe_encode_kernel(uint32_t first, int64_t n,
                                                           uint8_t* __restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * 256 * 4;
    for (int64_t base = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; base < n; base += stride) {
        float f[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            f[j] = __uint_as_float(first + (uint32_t)(base + j));
        int c = cvt2_lo(f[0], f[1], 0);
        c = cvt2_hi(f[2], f[3], c);
        if (base + 4 <= n && ((reinterpret_cast<uintptr_t>(out) + base) & 3) == 0) {
            *reinterpret_cast<uint32_t*>(out + base) = (uint32_t)c;
        } else {
            for (int j = 0; j < 4 && base + j < n; ++j)
                out[base + j] = (uint8_t)((uint32_t)c >> (8 * j));
        }
    }
}

hipError_t launch_quant_act(const void* x, int64_t rows, int64_t cols, uint8_t* q, float* s,
                            uint8_t* qt, float* st, hipStream_t stream)
{
    const int64_t rows_pad = (rows + 127) / 128 * 128;
    const dim3 grid((unsigned)((rows_pad / 128) * (cols / 128)));
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const bool row = q != nullptr, col = qt != nullptr;
    const BlockWalk walk = act_walk(quant_group_rows(false, cols), rows_pad / 128, cols / 128);
    if (row && col)
        return launch_kernel(quant_block_kernel<true, true, false, false>, grid, dim3(256), stream,
                             xb, rows, cols, rows_pad, q, s, qt, st, walk);
    if (row)
        return launch_kernel(quant_block_kernel<true, false, false, false>, grid, dim3(256), stream,
                             xb, rows, cols, rows_pad, q, s, qt, st, walk);
    return launch_kernel(quant_block_kernel<false, true, false, false>, grid, dim3(256), stream,
                         xb, rows, cols, rows_pad, q, s, qt, st, walk);
}

hipError_t launch_quant_weight(const void* w, int64_t n, int64_t k, uint8_t* q, uint8_t* qt,
                               float* s, hipStream_t stream)
{
    const dim3 grid((unsigned)((n / 128) * (k / 128)));
    const uint16_t* wb = static_cast<const uint16_t*>(w);
    const BlockWalk walk = grouped_walk(quant_group_rows(true, k));
    if (qt)
        return launch_kernel(quant_block_kernel<false, false, true, true>, grid, dim3(256), stream,
                             wb, n, k, n, q, s, qt, nullptr, walk);
    return launch_kernel(quant_block_kernel<false, false, true, false>, grid, dim3(256), stream,
                         wb, n, k, n, q, s, nullptr, nullptr, walk);
}

hipError_t launch_quant_weight_grouped(const WeightJob* jobs, int count, hipStream_t stream)
{
    WeightJobs g{};
    bool any_t = false;
    int64_t total = 0;
    for (int i = 0; i < count; ++i) {
        g.j[i] = jobs[i];
        g.first[i] = total;
        total += (jobs[i].n / 128) * (jobs[i].k / 128);
        any_t = any_t || jobs[i].qt != nullptr;
    }
    g.first[count] = total;
    g.count = count;
    g.group_rows = quant_group_rows(true, 0);
    if (count == 0 || total == 0)
        return hipSuccess;
    const dim3 grid((unsigned)total);
    if (any_t)
        return launch_kernel(quant_weight_grouped_kernel<true>, grid, dim3(256), stream, g);
    return launch_kernel(quant_weight_grouped_kernel<false>, grid, dim3(256), stream, g);
}

hipError_t launch_probe_encode(uint32_t first, int64_t n, uint8_t* out, hipStream_t stream)
{
    const int64_t blocks_needed = (n + 1023) / 1024;
    const unsigned grid = (unsigned)(blocks_needed < 65536 ? blocks_needed : 65536);
    return launch_kernel(probe_encode_kernel, dim3(grid), dim3(256), stream, first, n, out);
}

}  // namespace puro
