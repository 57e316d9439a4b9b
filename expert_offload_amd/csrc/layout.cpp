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

}  // namespace eo
