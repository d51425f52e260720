// device.hpp -- gfx950 device helpers shared by the routed-expert kernels.
//
// MXFP4 decode.  A weight is w = v * 2^(s-127) with v the e2m1 value of a 4-bit
// code (bit3 = sign) and s the group's ue8m0 scale byte (colibri PR #684,
// MXFP4-kernel commit).  gfx950's V_CVT_SCALEF32_PK_{F32,BF16}_FP4 converts two
// codes of one byte and scales them by 2^(E-127), E being the exponent field of
// its fp32 scale operand; for every E in 0..254 the result is the closed form
// rounded to the destination type (subnormals kept, overflow to +-inf), which
// was checked on the device for all 16 codes x 255 bytes.  The hardware treats
// E = 255 as NaN, whereas the closed form at s = 255 is v * 2^128 (+-0, +-2^127 or
// +-inf), so s = 255 is decoded with E = 254 and then doubled, which is exact.
// Both fp32 and bf16 hold every decoded value exactly (at most two significant
// bits, magnitude >= 2^-128).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace k3moe {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// fp32 whose exponent field is the scale byte (255 handled by the caller).
__device__ __forceinline__ float scale_operand(uint32_t s) {
    return __uint_as_float((s < 255u ? s : 254u) << 23);
}

// 8 codes (one dword, code j in bits 4j..4j+3 = column j) -> 8 fp32 in column order.
__device__ __forceinline__ void fp4x8_to_f32(uint32_t q, uint32_t s, float out[8]) {
    const float sc = scale_operand(s);
    f32x2 r0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, sc, 0);
    f32x2 r1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, sc, 1);
    f32x2 r2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, sc, 2);
    f32x2 r3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, sc, 3);
    out[0] = r0.x; out[1] = r0.y; out[2] = r1.x; out[3] = r1.y;
    out[4] = r2.x; out[5] = r2.y; out[6] = r3.x; out[7] = r3.y;
    if (__builtin_expect(s == 255u, 0)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) out[j] *= 2.0f;
    }
}

// 8 codes -> 8 bf16 (as four packed dwords, column order) ready for an MFMA operand.
__device__ __forceinline__ u32x4 fp4x8_to_bf16(uint32_t q, uint32_t s) {
    const float sc = scale_operand(s);
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 0));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 1));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 2));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 3));
    if (__builtin_expect(s == 255u, 0)) {
        // double each bf16 through fp32 (exact: the values are exact or +-inf)
        uint32_t* p = reinterpret_cast<uint32_t*>(&r);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float lo = __uint_as_float(p[j] << 16) * 2.0f;
            float hi = __uint_as_float(p[j] & 0xFFFF0000u) * 2.0f;
            p[j] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
        }
    }
    return r;
}

// 8 codes -> 8 bf16 without the s = 255 fix-up (callers guarantee s < 255, e.g.
// after a wave-uniform check).
__device__ __forceinline__ u32x4 fp4x8_to_bf16_nofix(uint32_t q, float sc) {
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 0));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 1));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 2));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc, 3));
    return r;
}

// 8 codes -> 8 fp16 (as four packed dwords, column order), scale 2^(s-127) given as
// an fp32; exact when every decoded value is an fp16 normal (callers check the
// scale bytes: 114 <= s <= 140 keeps 0.5 * 2^(s-127) >= 2^-14 and 6 * 2^(s-127) <=
// 65504).
__device__ __forceinline__ u32x4 fp4x8_to_f16_nofix(uint32_t q, float sc) {
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, sc, 0));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, sc, 1));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, sc, 2));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, sc, 3));
    return r;
}

// 32 codes (a 16-byte chunk = one scale group) -> 32 bf16 as 16 packed dwords,
// out[j] holding columns 8j..8j+7.  One branch for the rare s = 255 fix-up per
// chunk, so the common path is straight-line code.
__device__ __forceinline__ void fp4x32_to_bf16(const uint4& q, uint32_t s, u32x4 (&out)[4]) {
    const float sc = scale_operand(s);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        out[j].x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], sc, 0));
        out[j].y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], sc, 1));
        out[j].z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], sc, 2));
        out[j].w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], sc, 3));
    }
    if (__builtin_expect(s == 255u, 0)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t* p = reinterpret_cast<uint32_t*>(&out[j]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lo = __uint_as_float(p[i] << 16) * 2.0f;
                const float hi = __uint_as_float(p[i] & 0xFFFF0000u) * 2.0f;
                p[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
            }
        }
    }
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// max(v, v moved by one DPP pattern); lanes outside ROW_MASK's rows see 0, the
// identity of the maximum, which lets the compiler fold the move into the max.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false));
}

// Maximum over each row of 16 lanes, returned to every lane of the row: swap
// neighbours, swap pairs, rotate by 4, rotate by 8.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
    v = dpp_max_u32<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_max_u32<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_max_u32<0x124, 0xF>(v);  // row_ror:4
    v = dpp_max_u32<0x128, 0xF>(v);  // row_ror:8
    return v;
}

// Sum over the 64 lanes of a wave; every lane receives the total.  Fixed
// butterfly order, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// SiTU-GLU 4 tanh(g/4) sigmoid(g) * 25 tanh(u/25) (colibri PR #676 summary,
// Stable LatentMoE bullet), with device libm tanh/exp: saturates to the exact
// limits (exp overflow gives sigmoid 0) and propagates NaN.
__device__ __forceinline__ float situ_accurate(float g, float u) {
    float sg = 1.0f / (1.0f + expf(-g));
    return 4.0f * tanhf(0.25f * g) * sg * (25.0f * tanhf(u / 25.0f));
}

// The same function from the hardware exp2 and reciprocal, for the bf16 chunk
// path: tanh(a) = 1 - 2 / (e^{2a} + 1), sigmoid(g) = 1 / (1 + e^{-g}).  Absolute
// error ~1e-7 per factor; +-inf inputs give the exact limits, NaN propagates.
__device__ __forceinline__ float fast_exp(float a) { return __builtin_amdgcn_exp2f(a * 1.4426950408889634f); }
__device__ __forceinline__ float fast_rcp(float a) { return __builtin_amdgcn_rcpf(a); }
__device__ __forceinline__ float fast_tanh(float a) { return 1.0f - 2.0f * fast_rcp(fast_exp(2.0f * a) + 1.0f); }
__device__ __forceinline__ float situ_fast(float g, float u) {
    float sg = fast_rcp(1.0f + fast_exp(-g));
    return 4.0f * fast_tanh(0.25f * g) * sg * (25.0f * fast_tanh(0.04f * u));
}

}  // namespace k3moe
