// device_common.hpp -- small device-side helpers shared by the quantizer and
// GEMM kernels of the block-quantized FP8 library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace puro {

// Maximum over the 16 lanes of each DPP row (lanes 16r .. 16r+15).  After the
// two quad permutations every lane holds its quad's maximum; the half-row
// mirror pairs quad 0 with quad 1 (and 2 with 3); the row mirror pairs the
// two halves.  All four steps stay inside the row, so no lane is out of
// bounds.
__device__ __forceinline__ int dpp_row_max(int v)
{
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));  // row_mirror
    return v;
}

// |bf16| magnitudes of the two halves of a packed word, as integers.  The
// bf16 magnitude order equals the integer order of its low 15 bits, so the
// tile amax is an exact integer maximum.
__device__ __forceinline__ int mag2(uint32_t w)
{
    return max((int)(w & 0x7FFFu), (int)((w >> 16) & 0x7FFFu));
}

__device__ __forceinline__ int mag8(const uint4& v)
{
    return max(max(mag2(v.x), mag2(v.y)), max(mag2(v.z), mag2(v.w)));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Per-tile quantization parameters from the amax bit pattern (bf16 bits,
// sign cleared).  s = RN32(amax/448); an element maps to RN32((x*pre)*r)
// with r = RN32(448/(amax*pre)).  pre is 2^64 when amax < 2^-64 (so the
// reciprocal cannot overflow; x*pre is exact) and 1 otherwise.  amax == 0
// gives r = 0, i.e. signed zeros.  Division is IEEE correctly rounded (the
// library is built without fast-math) and fp32 denormals are kept.
struct TileQ {
    float s, r, pre;
};

__device__ __forceinline__ TileQ tile_params(int amax_bits)
{
    const float amax = __uint_as_float((uint32_t)amax_bits << 16);
    TileQ t;
    t.s = amax / 448.0f;
    if (amax == 0.0f) {
        t.r = 0.0f;
        t.pre = 1.0f;
    } else if (amax < 0x1p-64f) {
        t.pre = 0x1p64f;
        t.r = 448.0f / (amax * 0x1p64f);
    } else {
        t.pre = 1.0f;
        t.r = 448.0f / amax;
    }
    return t;
}

// Two E4M3 codes (OCP, round-to-nearest-even) packed into the low or high
// 16 bits of `old`, via the gfx950 hardware conversion.
__device__ __forceinline__ int cvt2_lo(float a, float b, int old)
{
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
}
__device__ __forceinline__ int cvt2_hi(float a, float b, int old)
{
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, true);
}

// Codes of the 8 bf16 values in `v` for a tile with pre == 1, as 8 bytes:
// the same bytes as encode8(v, 1.0f, r), since a product with 1 is exact.
// Callers take this form when no tile in the wave has amax < 2^-64.
__device__ __forceinline__ uint2 encode8_r(const uint4& v, float r)
{
    uint2 o;
    int lo = cvt2_lo(bf16_lo(v.x) * r, bf16_hi(v.x) * r, 0);
    lo = cvt2_hi(bf16_lo(v.y) * r, bf16_hi(v.y) * r, lo);
    int hi = cvt2_lo(bf16_lo(v.z) * r, bf16_hi(v.z) * r, 0);
    hi = cvt2_hi(bf16_lo(v.w) * r, bf16_hi(v.w) * r, hi);
    o.x = (uint32_t)lo;
    o.y = (uint32_t)hi;
    return o;
}

// Codes of the 8 bf16 values in `v`, scaled by (pre, r), as 8 bytes.
__device__ __forceinline__ uint2 encode8(const uint4& v, float pre, float r)
{
    uint2 o;
    int lo = cvt2_lo((bf16_lo(v.x) * pre) * r, (bf16_hi(v.x) * pre) * r, 0);
    lo = cvt2_hi((bf16_lo(v.y) * pre) * r, (bf16_hi(v.y) * pre) * r, lo);
    int hi = cvt2_lo((bf16_lo(v.z) * pre) * r, (bf16_hi(v.z) * pre) * r, 0);
    hi = cvt2_hi((bf16_lo(v.w) * pre) * r, (bf16_hi(v.w) * pre) * r, hi);
    o.x = (uint32_t)lo;
    o.y = (uint32_t)hi;
    return o;
}

// Two FP32 values -> packed bf16 (a in the low half), round to nearest even,
// denormals kept: one v_cvt_pk_bf16_f32.  For every non-NaN input this is
// the integer rounding u + 0x7FFF + ((u >> 16) & 1), upper half (checked on
// the device over all 2^32 patterns).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    const bf16x2_t h = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

}  // namespace puro
