// Debug decoder: one packed expert block to fp32 [W_gate | W_up | W_down], with
// the same element decoders the FFN kernels use. Values (juejin.cn overview,
// section 5 lists the formats): MXFP4 e2m1 * 2^(e8m0-127); NVFP4
// (e2m1 * e4m3) * g with one rounding on the multiply by g; FP8 e4m3 * s_row
// with one rounding; bf16 widened; fp32 as stored.
#include "decode_dev.h"
#include "dev_common.h"
#include "eo_internal.h"

namespace eo {

namespace {

__global__ __launch_bounds__(256) void k_dequant(int fmt, Layout lay, const uint8_t* __restrict__ b,
                                                 int H, int I, float* __restrict__ out) {
    const int64_t n13 = 2ll * I * H, n = n13 + (int64_t)H * I;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const bool top = i < n13;
    const int64_t li = top ? i : i - n13;
    const int K = top ? H : I;
    const int64_t row = li / K, col = li % K;
    const uint8_t* data = b + (top ? lay.d13 : lay.d2);
    const uint8_t* scal = b + (top ? lay.s13 : lay.s2);
    float v;
    switch (fmt) {
    case EO_W_FP32: v = ((const float*)data)[li]; break;
    case EO_W_BF16: v = bf16_f32(((const uint16_t*)data)[li]); break;
    case EO_W_FP8: v = e4m3_f32(data[li]) * ((const float*)scal)[row]; break;
    default: {
        uint32_t byte = data[li >> 1];
        uint32_t code = (li & 1) ? (byte >> 4) : (byte & 0xF);
        float e = e2m1_f32(code);
        if (fmt == EO_W_MXFP4) {
            v = e * e8m0_f32(scal[row * (K / 32) + col / 32]);
        } else {
            float p = e * e4m3_f32(scal[row * (K / 16) + col / 16]);
            int t = top ? (row < I ? 0 : 1) : 2;
            v = p * ((const float*)(b + lay.gl))[t];
        }
    }
    }
    out[i] = v;
}

// The same block decoded element by element through the decoders the expert
// kernels use, each followed by the factors that kernel applies outside the
// decode, multiplied in the same order:
//   dec 1, the grouped GEMM's tile decode: fp8 codes by the scaled convert at
//     scale 1, then the row scale; MXFP4 pairs by the scaled convert with the
//     e8m0 scale inside; NVFP4 pairs converted at scale 1, times the e4m3
//     block scale in fp32, packed to bf16, then times g.
//   dec 2, the decode GEMV's: fp8 codes through the scalar e4m3 decoder to
//     bf16, then the row scale; MXFP4 as dec 1; NVFP4 pairs by the scaled
//     convert at scale 1, then times the e4m3 block scale, then times g.
// bf16 and fp32 weights are read as stored by both.
template <int DEC>
__global__ __launch_bounds__(256) void k_dequant_dec(int fmt, Layout lay,
                                                     const uint8_t* __restrict__ b, int H, int I,
                                                     float* __restrict__ out) {
    const int64_t n13 = 2ll * I * H, n = n13 + (int64_t)H * I;
    // one thread per element pair (the converts take two codes)
    const int64_t i = 2 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
    if (i >= n) return;
    const bool top = i < n13;
    const int64_t li = top ? i : i - n13;
    const int K = top ? H : I;
    const int64_t row = li / K, col = li % K;  // col even: the pair shares its block
    const uint8_t* data = b + (top ? lay.d13 : lay.d2);
    const uint8_t* scal = b + (top ? lay.s13 : lay.s2);
    const int t = top ? (row < I ? 0 : 1) : 2;
    float v0, v1;
    if (fmt == EO_W_FP32) {
        v0 = ((const float*)data)[li];
        v1 = ((const float*)data)[li + 1];
    } else if (fmt == EO_W_BF16) {
        const uint32_t pr = ((const uint32_t*)data)[li >> 1];
        v0 = bf16_f32(pr & 0xFFFF);
        v1 = bf16_f32(pr >> 16);
    } else if (fmt == EO_W_FP8) {
        // the word holding the pair; the pair is its bytes (li & 3) and (li & 3) + 1
        const uint32_t wd = ((const uint32_t*)data)[li >> 2];
        uint32_t pr;
        if (DEC == 1) {
            uint32_t lo, hi;
            fp8x4_bf16(wd, lo, hi);
            pr = (li & 2) ? hi : lo;
        } else {
            pr = e4m3x2_bf16((li & 2) ? wd >> 16 : wd);
        }
        const float rs = ((const float*)scal)[row];
        v0 = bf16_f32(pr & 0xFFFF) * rs;
        v1 = bf16_f32(pr >> 16) * rs;
    } else {
        // the pair is byte (li/2) & 3 of the word holding it
        const uint32_t wd = ((const uint32_t*)data)[li >> 3];
        const int B = (int)((li >> 1) & 3);
        uint32_t pr = 0;
        if (fmt == EO_W_MXFP4) {
            const float sc = e8m0_f32(scal[row * (K / 32) + col / 32]);
            switch (B) {
            case 0: pr = fp4x2_bf16_pow2<0>(wd, sc); break;
            case 1: pr = fp4x2_bf16_pow2<1>(wd, sc); break;
            case 2: pr = fp4x2_bf16_pow2<2>(wd, sc); break;
            default: pr = fp4x2_bf16_pow2<3>(wd, sc); break;
            }
            v0 = bf16_f32(pr & 0xFFFF);
            v1 = bf16_f32(pr >> 16);
        } else {
            const float sc = e4m3_f32(scal[row * (K / 16) + col / 16]);
            const float g = ((const float*)(b + lay.gl))[t];
            if (DEC == 1) {
                switch (B) {
                case 0: pr = fp4x2_bf16<EO_W_NVFP4, 0>(wd, sc); break;
                case 1: pr = fp4x2_bf16<EO_W_NVFP4, 1>(wd, sc); break;
                case 2: pr = fp4x2_bf16<EO_W_NVFP4, 2>(wd, sc); break;
                default: pr = fp4x2_bf16<EO_W_NVFP4, 3>(wd, sc); break;
                }
                v0 = bf16_f32(pr & 0xFFFF) * g;
                v1 = bf16_f32(pr >> 16) * g;
            } else {
                switch (B) {
                case 0: pr = fp4x2_bf16_pow2<0>(wd, 1.0f); break;
                case 1: pr = fp4x2_bf16_pow2<1>(wd, 1.0f); break;
                case 2: pr = fp4x2_bf16_pow2<2>(wd, 1.0f); break;
                default: pr = fp4x2_bf16_pow2<3>(wd, 1.0f); break;
                }
                v0 = bf16_f32(pr & 0xFFFF) * sc * g;
                v1 = bf16_f32(pr >> 16) * sc * g;
            }
        }
    }
    out[i] = v0;
    out[i + 1] = v1;
}

}  // namespace

hipError_t launch_dequant_dec(int dec, int fmt, const Layout& lay, const uint8_t* blk, int H,
                              int I, float* out, hipStream_t s) {
    const int64_t pairs = 3ll * H * I / 2;
    const unsigned grid = (unsigned)((pairs + 255) / 256);
    if (dec == 1)
        k_dequant_dec<1><<<grid, 256, 0, s>>>(fmt, lay, blk, H, I, out);
    else if (dec == 2)
        k_dequant_dec<2><<<grid, 256, 0, s>>>(fmt, lay, blk, H, I, out);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_dequant(int fmt, const Layout& lay, const uint8_t* blk, int H, int I, float* out,
                          hipStream_t s) {
    int64_t n = 3ll * H * I;
    k_dequant<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(fmt, lay, blk, H, I, out);
    return hipGetLastError();
}

}  // namespace eo
