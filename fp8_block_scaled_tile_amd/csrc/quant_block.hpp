// quant_block.hpp -- quantization of one 128x128 block of a bf16 matrix held
// in registers, shared by the plain quantizers (quant.hip) and the fused
// producers (produce.hip).
//
// Fine-grained block quantization of the linear-layer GEMM operands (arXiv
// report "Puro-2B" section 2.1; training.farm blog section "FP8"): one FP32
// scale per tile, s = amax/448, codes = E4M3(x * 448/amax).  Activations and
// gradients use 1x128 tiles along the contraction dimension (row-wise) and,
// for the weight-gradient GEMM, 128x1 tiles along tokens with the codes
// stored transposed (column-wise); weights use 128x128 blocks.
//
// One 256-thread work-group owns a 128x128 block.  Thread t holds columns
// 8*(t%16) .. +7 and rows 8*(t/16) .. +7 of the block (v[p] = row p of its
// 8, eight bf16 values), so each row of the block lives in one 16-lane DPP
// row: the 1x128 amax is a four-step DPP maximum with no LDS traffic, and each
// of the 8 rows' scale divisions is done by one lane of the DPP row and
// broadcast (row_newbcast) to the other 15.  Row-wise codes are stored
// straight from registers (16 lanes write one 128-byte line); the transposed
// copy goes through an XOR-swizzled 16 KB LDS tile and leaves as 16-byte
// stores.
#pragma once

#include "block_walk.hpp"
#include "device_common.hpp"

namespace puro {

template <bool ROW, bool COL, bool WEIGHT, bool WT>
struct QuantLds {
    int colmax[COL ? 16 : 1][COL ? 128 : 1];
    float col_r[COL ? 128 : 1];
    float col_pre[COL ? 128 : 1];
    __attribute__((aligned(16))) uint8_t tbuf[(COL || WT) ? 128 * 128 : 16];
    int wmax[16];
};

// Codes and scales of block (rb, cb) from v.  Output layouts:
//   row tiles:  q[r][c] (row stride cols), s[c/128][r]
//   col tiles:  qt[c][r] (row stride ld_t), st[r/128][c]
//   weight:     q as above, s[rb][cb] (cols/128 per row), qt[c][r] if WT
// Rows at or past `rows` must hold zeros in v; they are not stored and do not
// raise a tile's amax.  Uses __syncthreads(): every thread of the work-group
// must call it, and a second call must be separated from the first by a
// barrier (the LDS is reused).
template <bool ROW, bool COL, bool WEIGHT, bool WT>
__device__ __forceinline__ void quant_block_body(const uint4 (&v)[8], int64_t rows, int64_t cols,
                                                 int64_t ld_t, int64_t rb, int64_t cb,
                                                 uint8_t* __restrict__ q, float* __restrict__ s,
                                                 uint8_t* __restrict__ qt, float* __restrict__ st,
                                                 QuantLds<ROW, COL, WEIGHT, WT>& L)
{
    constexpr bool TRANS = COL || WT;
    const int t = threadIdx.x;
    const int qd = t & 15;       // column chunk of 8 elements
    const int g = t >> 4;        // row group of 8 rows
    const int64_t row0 = rb * 128 + 8 * g;
    const int64_t col0 = cb * 128 + 8 * qd;

    // ---- 128x128 block scale (weights) ----------------------------------
    TileQ wq = {0.0f, 0.0f, 1.0f};
    if constexpr (WEIGHT) {
        int m = 0;
#pragma unroll
        for (int p = 0; p < 8; ++p)
            m = max(m, mag8(v[p]));
        m = dpp_row_max(m);
        if (qd == 0)
            L.wmax[g] = m;
        __syncthreads();
        int bm = L.wmax[0];
#pragma unroll
        for (int i = 1; i < 16; ++i)
            bm = max(bm, L.wmax[i]);
        wq = tile_params(bm);
        if (t == 0)
            s[rb * (cols / 128) + cb] = wq.s;
    }

    // ---- codes in input orientation (1x128 tiles, or the weight block) --
    // (a weight quantized for the transposed copy only passes q = NULL)
    if (ROW || (WEIGHT && q != nullptr)) {
        // Row tiles: every lane of a DPP row gets the 8 row maxima; lane qd
        // computes the parameters of row qd & 7 only, lanes 0..7 store their
        // row's scale, and r is broadcast from lane p of the DPP row.
        int am[8];
        float rr[8];
        if constexpr (!WEIGHT) {
#pragma unroll
            for (int p = 0; p < 8; ++p)
                am[p] = dpp_row_max(mag8(v[p]));
            int mine = am[0];
#pragma unroll
            for (int p = 1; p < 8; ++p)
                mine = ((qd & 7) == p) ? am[p] : mine;
            const TileQ tm = tile_params(mine);
            if (qd < 8 && row0 + qd < rows)
                s[cb * rows + row0 + qd] = tm.s;
            const int ri = __float_as_int(tm.r);
            rr[0] = __int_as_float(__builtin_amdgcn_update_dpp(0, ri, 0x150, 0xF, 0xF, false));   // row_newbcast:0
            rr[1] = __int_as_float(__builtin_amdgcn_update_dpp(0, ri, 0x151, 0xF, 0xF, false));
            rr[2] = __int_as_float(__builtin_amdgcn_update_dpp(0, ri, 0x152, 0xF, 0xF, false));
            rr[3] = __int_as_float(__builtin_amdgcn_update_dpp(0, ri, 0x153, 0xF, 0xF, false));
            rr[4] = __int_as_float(__builtin_amdgcn_update_dpp(0, ri, 0x154, 0xF, 0xF, false));
            rr[5] = __int_as_float(__builtin_amdgcn_update_dpp(0, ri, 0x155, 0xF, 0xF, false));
            rr[6] = __int_as_float(__builtin_amdgcn_update_dpp(0, ri, 0x156, 0xF, 0xF, false));
            rr[7] = __int_as_float(__builtin_amdgcn_update_dpp(0, ri, 0x157, 0xF, 0xF, false));
        }
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int64_t r = row0 + p;
            TileQ tq = wq;
            if constexpr (!WEIGHT) {
                tq.r = rr[p];
                tq.pre = (am[p] != 0 && am[p] < 0x1F80) ? 0x1p64f : 1.0f;   // amax < 2^-64
            }
            uint2 codes;
            if (__builtin_amdgcn_ballot_w64(tq.pre != 1.0f) != 0)
                codes = encode8(v[p], tq.pre, tq.r);
            else
                codes = encode8_r(v[p], tq.r);
            if (r < rows)
                *reinterpret_cast<uint2*>(q + r * cols + col0) = codes;
        }
    }

    // ---- transposed codes (128x1 tiles, or the weight block transposed) -
    // (a weight of a grouped launch may pass qt = NULL: uniform per block)
    if constexpr (TRANS) {
        if (WEIGHT && qt == nullptr)
            return;
        if constexpr (COL) {
            int cm[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                cm[i] = 0;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                cm[0] = max(cm[0], (int)(v[p].x & 0x7FFFu));
                cm[1] = max(cm[1], (int)((v[p].x >> 16) & 0x7FFFu));
                cm[2] = max(cm[2], (int)(v[p].y & 0x7FFFu));
                cm[3] = max(cm[3], (int)((v[p].y >> 16) & 0x7FFFu));
                cm[4] = max(cm[4], (int)(v[p].z & 0x7FFFu));
                cm[5] = max(cm[5], (int)((v[p].z >> 16) & 0x7FFFu));
                cm[6] = max(cm[6], (int)(v[p].w & 0x7FFFu));
                cm[7] = max(cm[7], (int)((v[p].w >> 16) & 0x7FFFu));
            }
            *reinterpret_cast<int4*>(&L.colmax[g][8 * qd]) = make_int4(cm[0], cm[1], cm[2], cm[3]);
            *reinterpret_cast<int4*>(&L.colmax[g][8 * qd + 4]) = make_int4(cm[4], cm[5], cm[6], cm[7]);
            __syncthreads();
            if (t < 128) {
                int m = L.colmax[0][t];
#pragma unroll
                for (int j = 1; j < 16; ++j)
                    m = max(m, L.colmax[j][t]);
                const TileQ tq = tile_params(m);
                L.col_r[t] = tq.r;
                L.col_pre[t] = tq.pre;
                st[rb * cols + cb * 128 + t] = tq.s;
            }
            __syncthreads();
        }
        // Column i of this thread's 8x8 patch: 8 codes for rows 8g .. 8g+7,
        // stored as one 8-byte chunk of LDS row c = 8*qd + i.  The chunk index
        // is XOR-swizzled with qd so the 16 lanes of a DPP row hit distinct
        // banks.
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float r = wq.r, pre = wq.pre;
            if constexpr (COL) {
                r = L.col_r[8 * qd + i];
                pre = L.col_pre[8 * qd + i];
            }
            float f[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const uint32_t w = (i < 2) ? v[p].x : (i < 4) ? v[p].y : (i < 6) ? v[p].z : v[p].w;
                f[p] = (i & 1) ? bf16_hi(w) : bf16_lo(w);
            }
            if (__builtin_amdgcn_ballot_w64(pre != 1.0f) != 0) {     // a tiny tile in the wave
#pragma unroll
                for (int p = 0; p < 8; ++p)
                    f[p] = f[p] * pre;
            }
            int lo = cvt2_lo(f[0] * r, f[1] * r, 0);
            lo = cvt2_hi(f[2] * r, f[3] * r, lo);
            int hi = cvt2_lo(f[4] * r, f[5] * r, 0);
            hi = cvt2_hi(f[6] * r, f[7] * r, hi);
            const int c = 8 * qd + i;
            *reinterpret_cast<uint2*>(L.tbuf + c * 128 + 8 * (g ^ qd)) = make_uint2((uint32_t)lo, (uint32_t)hi);
        }
        __syncthreads();
        // Read back 16 bytes (two logical chunks 2h, 2h+1) of LDS row c.  They
        // sit in the aligned pair h ^ (qc >> 1), swapped when qc is odd.
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
            const int c = (t >> 3) + 32 * pass;
            const int h = t & 7;
            const int qc = (c >> 3) & 15;
            uint4 w = *reinterpret_cast<const uint4*>(L.tbuf + c * 128 + 16 * (h ^ (qc >> 1)));
            if (qc & 1)
                w = make_uint4(w.z, w.w, w.x, w.y);
            *reinterpret_cast<uint4*>(qt + (cb * 128 + c) * ld_t + rb * 128 + 16 * h) = w;
        }
    }
}

}  // namespace puro
