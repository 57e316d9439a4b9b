// Weight decoders of the expert kernels, shared by the grouped GEMM, the decode
// GEMV and the debug decoder that checks them element by element. Each turns
// packed codes into bf16 pairs with gfx950's scaled converts; all are exact
// (an e2m1 value has at most 2 significant bits, an e4m3 value at most 4, and
// the scales applied inside them are powers of two or e4m3 values). Formats:
// juejin.cn overview, section 5.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/eo.h"
#include "dev_common.h"

namespace eo {

typedef float dec_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 dec_bf16x2 __attribute__((ext_vector_type(2)));

// Four e4m3fn codes (one word, first code in the low byte) as two bf16 pairs:
// the scaled convert at scale 1.
__device__ __forceinline__ void fp8x4_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// Two e4m3fn codes (the low 16 bits of two) as a bf16 pair, through the scalar
// decoder (the decode GEMV's form).
__device__ __forceinline__ uint32_t e4m3x2_bf16(uint32_t two) {
    return bf_hi(e4m3_f32(two & 0xFF)) | (bf_hi(e4m3_f32((two >> 8) & 0xFF)) << 16);
}

// Two fp4 codes (byte B of w, even element in the low nibble) as a bf16 pair,
// scaled inside the convert. The convert applies only the power of two of its
// scale operand: MXFP4's e8m0 scale goes in whole; at 1.0 the codes come out
// unscaled.
template <int B>
__device__ __forceinline__ uint32_t fp4x2_bf16_pow2(uint32_t w, float sc) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, B));
}

// The grouped GEMM's fp4 tile decode: MXFP4 as above; for NVFP4 the pair is
// converted to fp32 at scale 1, multiplied by the e4m3 block scale sc there and
// packed to bf16 (round to nearest even, which changes nothing: the product is
// exact in bf16).
template <int FMT, int B>
__device__ __forceinline__ uint32_t fp4x2_bf16(uint32_t w, float sc) {
    if (FMT == EO_W_MXFP4) return fp4x2_bf16_pow2<B>(w, sc);
    const dec_f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B) * sc;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, dec_bf16x2));
}

}  // namespace eo
