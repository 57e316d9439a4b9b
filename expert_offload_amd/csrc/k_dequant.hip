// Debug decoder: one packed expert block to fp32 [W_gate | W_up | W_down], with
// the same element decoders the FFN kernels use. Values (juejin.cn overview,
// section 5 lists the formats): MXFP4 e2m1 * 2^(e8m0-127); NVFP4
// (e2m1 * e4m3) * g with one rounding on the multiply by g; FP8 e4m3 * s_row
// with one rounding; bf16 widened; fp32 as stored.
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

}  // namespace

hipError_t launch_dequant(int fmt, const Layout& lay, const uint8_t* blk, int H, int I, float* out,
                          hipStream_t s) {
    int64_t n = 3ll * H * I;
    k_dequant<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(fmt, lay, blk, H, I, out);
    return hipGetLastError();
}

}  // namespace eo
