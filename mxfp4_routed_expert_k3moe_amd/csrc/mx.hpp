// mx.hpp -- OCP MXFP8 encoding on the device: E4M3 elements, one E8M0 scale per
// 32 consecutive values.
//
// The GPU form of the pages' low-precision activations (colibri PR #684,
// int8-activation commit: activations quantized in groups of 32 and multiplied
// with the MXFP4 weights as stored).  gfx950's scaled MFMA takes groups of 32
// with a power-of-two scale, so the group is kept and the element type is FP8
// E4M3 (bias 7, three mantissa bits, subnormals, largest finite 448, S.1111.111
// NaN).  For a group with largest magnitude amax:
//   amax = 0           -> scale byte 0, codes +-0
//   NaN or inf present -> scale byte 255 (the E8M0 NaN), codes 0x7F
//   otherwise          -> s = max(exponent field of amax - 8, 0), i.e.
//                         floor(log2 amax) - 8 + 127 clamped at 0, so the
//                         largest value lands in E4M3's top binade; each value
//                         v * 2^(127-s) is clamped to +-448 and rounded to the
//                         nearest E4M3 value, ties to the even code, sign kept.
// A second part, where used, quantizes the fp32 residual v - value(part 0) the
// same way; the residual is exact in fp32 (part 0 is zero or within a factor two
// of v).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace k3moe {

constexpr uint32_t kMxNaNScale = 255u;
constexpr uint32_t kE4M3NaN = 0x7Fu;

// Scale byte from the largest magnitude's bits (sign cleared).
__device__ __forceinline__ uint32_t mx_scale_of(uint32_t amax_bits) {
    if (amax_bits >= 0x7F800000u) return kMxNaNScale;
    const int ef = (int)(amax_bits >> 23);
    return (uint32_t)max(ef - 8, 0);
}

// E4M3 code of v * 2^(127-s), s < 255 (then s <= 246, so 2^(127-s) is a normal
// fp32 and the scaling is exact wherever it matters: results below 2^-126 round
// to code 0 either way).
__device__ __forceinline__ uint32_t mx_encode(float v, uint32_t s) {
    const float y = v * __uint_as_float((254u - s) << 23);
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fminf(fabsf(y), 448.0f);
    uint32_t code;
    if (a < 0.015625f) {  // below 2^-6: subnormal E4M3, quantum 2^-9
        code = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        // drop 20 of fp32's 23 mantissa bits, round to nearest even; a carry
        // moves into the exponent; exponent bias 127 -> 7
        const uint32_t b = __float_as_uint(a);
        code = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
    }
    return sign | code;
}

// Value of an E4M3 code under scale byte s < 255 (exact in fp32, subnormals kept).
__device__ __forceinline__ float mx_decode(uint32_t code, uint32_t s) {
    const uint32_t e = (code >> 3) & 15u, m = code & 7u;
    const float mag = e == 0 ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
    const float sc = s == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(s << 23);  // 2^(s-127)
    const float v = mag * sc;
    return (code & 0x80u) ? -v : v;
}

}  // namespace k3moe
