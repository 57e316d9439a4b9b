// The fill's copy loop (device part shared by the fill kernel and the decode
// launch that fills and runs gate/up together).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace eo {

// Workgroups that copy a call's fills: their 16-byte reads over PCIe, 256 KB in
// flight together, fill the link and leave the other CUs free.
constexpr int kFillBlocks = 64;
constexpr int kFillUnroll = 4;

// Workgroup `part` of `nparts`: its share of one S-byte copy (grid-stride over
// 16-byte words). CLAMP: the reads take indexes clamped to the last word
// instead of a bounds check (only the stores are checked), which keeps the
// words in registers where the bounds-checked form would stage them in scratch.
template <bool CLAMP = false>
__device__ __forceinline__ void copy_block(const uint8_t* __restrict__ src8,
                                           uint8_t* __restrict__ dst8, uint64_t S, int part,
                                           int nparts) {
    const uint4* src = (const uint4*)src8;
    uint4* dst = (uint4*)dst8;
    const uint64_t n16 = S / 16;
    const uint64_t step = (uint64_t)nparts * 256 * kFillUnroll;
    for (uint64_t b = (uint64_t)part * 256 * kFillUnroll + threadIdx.x; b < n16; b += step) {
        uint4 v[kFillUnroll];
#pragma unroll
        for (int u = 0; u < kFillUnroll; ++u) {
            const uint64_t i = b + (uint64_t)u * 256;
            if (CLAMP)
                v[u] = src[i < n16 ? i : n16 - 1];
            else if (i < n16)
                v[u] = src[i];
        }
#pragma unroll
        for (int u = 0; u < kFillUnroll; ++u) {
            const uint64_t i = b + (uint64_t)u * 256;
            if (i < n16) dst[i] = v[u];
        }
    }
    const uint64_t tail = S - n16 * 16;
    if (part == 0 && threadIdx.x < tail) dst8[n16 * 16 + threadIdx.x] = src8[n16 * 16 + threadIdx.x];
}

}  // namespace eo
