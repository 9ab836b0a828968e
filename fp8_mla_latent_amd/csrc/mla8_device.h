// Device helpers shared by the attention kernels (mla8_kernels.hip) and the
// indexer kernels (mla8_index.hip): the e4m3 encoder, the per-row quantizer
// arithmetic and wave reductions.
//
// Method source: colibri PR #300 "KV8 long-context CUDA: fp8 device shadow,
// split-T kernels, DSA-aware gather", first commit ("KV8 base"), c/kv_fp8.h
// bullet: RNE e4m3 encoder saturating at +/-448, signed zero kept, NaN stored
// as 0; per-row quantizer with scale amax/448 and a subnormal-amax guard.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla8 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// e4m3 encoder on the f32 bit pattern.  Round-to-nearest-even onto 3 mantissa
// bits, saturation at 448, sign of zero kept, NaN -> 0x00.
__device__ __forceinline__ uint32_t enc_e4m3(float y)
{
    const uint32_t b = __float_as_uint(y);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t a = b & 0x7FFFFFFFu;
    if (a > 0x7F800000u)
        return 0u;                  // NaN of either sign: inert zero
    if (a >= 0x43E00000u)
        return sign | 0x7Eu;        // |y| >= 448, infinity included
    uint32_t code;
    if (a >= 0x3C800000u) {         // |y| >= 2^-6: e4m3 normal range
        // Drop 20 mantissa bits with round-half-even; a carry out of the kept
        // mantissa moves into the exponent field by itself.
        const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
        code = (r >> 20) - (120u << 3);  // re-bias the exponent 127 -> 7
    } else {
        // e4m3 subnormals are the multiples of 2^-9 below 2^-6; the product is
        // exact and v_rndne_f32 rounds half to even.  8 -> 0x08 = 2^-6.
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    }
    return sign | code;
}

// Four values to e4m3 by the hardware conversion (v_cvt_pk_fp8_f32, two per
// instruction: round to nearest even onto OCP e4m3), bytes in argument order.
// It equals enc_e4m3 for finite |y| < 448, the only inputs it is given here;
// it does not saturate, so larger or non-finite inputs give other codes.
__device__ __forceinline__ uint32_t enc_e4m3_pk4(float y0, float y1, float y2, float y3)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true);
    return (uint32_t)w;
}

// Two f32 -> fp16, round to nearest even (v_cvt_pk_f16_f32): a in the low
// half, b in the high half.
__device__ __forceinline__ uint32_t pk_f16(float a, float b)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, h2));
}

// r - f32(h), h the fp16 in the low (H = 0) or high (H = 1) half of x, in one
// v_fma_mix_f32 (the fp16 operand widened exactly, one rounding of the result).
template <int H>
__device__ __forceinline__ float sub_f16(float r, uint32_t x)
{
    float d;
    if constexpr (H == 0)
        asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(x), "v"(r));
    else
        asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(x), "v"(r));
    return d;
}

// f32(h) * m, h the fp16 in the low (H = 0) or high (H = 1) half of x: an
// fma with +0 (so that it stays one v_fma_mix_f32; exact for m a power of 2
// and a product in f32's normal range).
template <int H>
__device__ __forceinline__ float mul_f16(uint32_t x, float m)
{
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 h = __builtin_bit_cast(h2, x);
    return __builtin_fmaf((float)h[H], m, 0.0f);
}

// max(a, |x|, |y|) in one v_max3_f32 (no canonicalising of the operands; a
// NaN operand gives the other operands' maximum or a NaN).
__device__ __forceinline__ float max3_abs(float a, float x, float y)
{
    float d;
    asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(d) : "v"(a), "v"(x), "v"(y));
    return d;
}

// Maximum over the 16 lanes of each row (DPP: quad swaps, then half-row and
// row mirrors), and over the whole wave (permlane swaps across rows).
__device__ __forceinline__ float row16_max(float x)
{
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false)));
    return x;
}
__device__ __forceinline__ float max_xor16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// A row's stored scale amax/448 and the inverse 448/amax its entries are
// multiplied by before encoding: IEEE f32 quotients (the library is built with
// correctly rounded f32 division).  The guard: when 448/amax is not finite the
// row encodes as signed zeros.
__device__ __forceinline__ void row_scale_inv(float amax, float& scale, float& inv)
{
    scale = amax / 448.0f;
    inv = 448.0f / amax;
    if (!(inv <= 3.402823466e38f))
        inv = 0.0f;
}

__device__ __forceinline__ float max_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// bf16 bits of an f32 value: round to nearest even (a finite value that rounds
// past the largest bf16 becomes infinity, infinities stay), NaN -> the quiet
// NaN 0x7FC0 with its sign.
__device__ __forceinline__ uint32_t bf16_rne_bits(float x)
{
    const uint32_t b = __float_as_uint(x);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u)
        return ((b >> 16) & 0x8000u) | 0x7FC0u;
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// One row by one wave: the row (d <= kMaxRowWidth floats, at most three
// float4 per lane) stays in registers between the amax pass and the encode
// pass.
constexpr int kMaxRowWidth = 768;
__device__ __forceinline__ void quantize_row_wave(const float* __restrict__ x, int32_t d,
                                                  uint8_t* __restrict__ codes_row,
                                                  float* __restrict__ scale_out, int lane)
{
    const float4* xr = reinterpret_cast<const float4*>(x);
    const int nv = d >> 2;
    float4 v[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int i = lane + 64 * k;
        v[k] = (i < nv) ? xr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const float e[4] = {fabsf(v[k].x), fabsf(v[k].y), fabsf(v[k].z), fabsf(v[k].w)};
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (e[c] <= 3.402823466e38f)  // finite only: false for NaN and inf
                amax = fmaxf(amax, e[c]);
    }
    amax = max_xor32(max_xor16(row16_max(amax)));
    float scale, inv;
    row_scale_inv(amax, scale, inv);
    uint32_t* cr = reinterpret_cast<uint32_t*>(codes_row);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int i = lane + 64 * k;
        if (i < nv)
            cr[i] = enc_e4m3(v[k].x * inv) | (enc_e4m3(v[k].y * inv) << 8) |
                    (enc_e4m3(v[k].z * inv) << 16) | (enc_e4m3(v[k].w * inv) << 24);
    }
    if (lane == 0)
        *scale_out = scale;
}

// Mixed row (noPE e4m3 + per-row scale, RoPE bf16) by one wave: the lc noPE
// values of x through the row quantizer above (their own amax and scale),
// the rc RoPE values that follow them to bf16 by round-to-nearest-even; the
// stored row is lc code bytes then rc bf16 values (lc + 2 rc bytes).
__device__ __forceinline__ void quantize_row_mx_wave(const float* __restrict__ x, int32_t lc,
                                                     int32_t rc, uint8_t* __restrict__ row,
                                                     float* __restrict__ scale_out, int lane)
{
    quantize_row_wave(x, lc, row, scale_out, lane);
    if (lane < rc / 4) {
        const float4 v = reinterpret_cast<const float4*>(x + lc)[lane];
        const uint32_t b0 = bf16_rne_bits(v.x), b1 = bf16_rne_bits(v.y);
        const uint32_t b2 = bf16_rne_bits(v.z), b3 = bf16_rne_bits(v.w);
        reinterpret_cast<uint2*>(row + lc)[lane] = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    }
}

}  // namespace mla8
