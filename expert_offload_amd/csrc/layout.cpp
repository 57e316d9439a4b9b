// Byte layout of one packed expert block (see eo.h): W13 = [W_gate; W_up]
// (2I rows of H) and W2 = W_down (H rows of I), data sections first, then the
// per-block or per-row scales, then (NVFP4) the three fp32 global scales.
#include "eo_host.h"

namespace eo {

Layout layout_of(int H, int I, int fmt) {
    Layout l;
    const uint64_t n13 = 2ull * I * H, n2 = (uint64_t)H * I;
    switch (fmt) {
    case EO_W_FP32:
        l.d2 = 4 * n13;
        l.s13 = l.s2 = l.gl = l.bytes = 4 * (n13 + n2);
        break;
    case EO_W_BF16:
        l.d2 = 2 * n13;
        l.s13 = l.s2 = l.gl = l.bytes = 2 * (n13 + n2);
        break;
    case EO_W_MXFP4:
        l.d2 = n13 / 2;
        l.s13 = l.d2 + n2 / 2;
        l.s2 = l.s13 + n13 / 32;
        l.gl = l.bytes = l.s2 + n2 / 32;
        break;
    case EO_W_NVFP4:
        l.d2 = n13 / 2;
        l.s13 = l.d2 + n2 / 2;
        l.s2 = l.s13 + n13 / 16;
        l.gl = l.s2 + n2 / 16;
        l.bytes = l.gl + 12;
        break;
    case EO_W_FP8:
        l.d2 = n13;
        l.s13 = l.d2 + n2;
        l.s2 = l.s13 + 4 * 2ull * I;
        l.gl = l.bytes = l.s2 + 4ull * H;
        break;
    default:
        break;
    }
    return l;
}

bool router_chain_layout(const float* R, int E, int H, float* out) {
    if (E < 1 || H < 256 || H % 256 != 0) return false;
    const int J = H / 64;  // steps of each of the 64 chains (h = i + 64 j)
    for (int e = 0; e < E; ++e) {
        const float* r = R + (size_t)e * H;
        float* o = out + (size_t)e * H;
        for (int j = 0; j < J; ++j)
            for (int i = 0; i < 64; ++i) o[((size_t)(j / 4) * 64 + i) * 4 + (j % 4)] = r[i + 64 * j];
    }
    return true;
}

}  // namespace eo
