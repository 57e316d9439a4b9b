// Device helpers: exact element decoders for the expert-block formats and
// bf16 conversions. Every decoder below is exact (the values are powers of two
// times at most 4 significant bits).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace eo {

__device__ __forceinline__ float bf16_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Upper half of an fp32: the bf16 with the same value when the low 16 bits are 0.
__device__ __forceinline__ uint32_t bf_hi(float v) { return __float_as_uint(v) >> 16; }

__device__ __forceinline__ uint32_t f32_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// e2m1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
__device__ __forceinline__ float e2m1_f32(uint32_t c) {
    uint32_t e = (c >> 1) & 3u, b = c & 1u;
    uint32_t bits = e ? (((e + 126u) << 23) | (b << 22)) : (b ? 0x3F000000u : 0u);
    return __uint_as_float(bits | ((c & 8u) << 28));
}

// e4m3fn: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0;
// exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN.
__device__ __forceinline__ float e4m3_f32(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float v;
    if (e == 15u && m == 7u)
        v = __uint_as_float(0x7FC00000u);
    else if (e == 0u)
        v = (float)m * 0.001953125f;  // 2^-9
    else
        v = __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (c & 0x80u) ? -v : v;
}

// e8m0: 2^(c - 127); 0xFF is NaN.
__device__ __forceinline__ float e8m0_f32(uint32_t c) {
    if (c == 0xFFu) return __uint_as_float(0x7FC00000u);
    if (c == 0u) return __uint_as_float(0x00400000u);  // 2^-127
    return __uint_as_float(c << 23);
}

__device__ __forceinline__ float silu_f32(float u) { return u / (1.0f + __expf(-u)); }

}  // namespace eo
