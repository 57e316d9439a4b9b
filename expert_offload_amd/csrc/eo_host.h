// Host-side declarations shared by the engine and the host-core expert
// routine (no HIP dependency, so the routine builds with the host compiler).
#pragma once

#include <cstdint>
#include <functional>
#include <vector>

#include "../../include/eo.h"

namespace eo {

constexpr int kMaxE = EO_MAX_EXPERTS;
constexpr int kMaxK = 16;
constexpr uint64_t kPoolAlign = 4096;

// Byte offsets of the sections of one packed expert block (see eo.h).
struct Layout {
    uint64_t d13 = 0, d2 = 0, s13 = 0, s2 = 0, gl = 0, bytes = 0;
};
Layout layout_of(int H, int I, int fmt);

// Router weights R [E, H] fp32 rearranged per accumulation chain for the
// many-token router kernel: out[e][j/4][i][j%4] = R[e][i + 64 j] (chain i takes
// h = i, i + 64, ...), so a lane's 16-byte load holds four consecutive steps of
// its chain. The layout takes the chains' H/64 steps in whole groups of four:
// false (out untouched) unless H is a multiple of 256.
bool router_chain_layout(const float* R, int E, int H, float* out);

// Host-core expert routine: for every expert with a non-null `experts` entry,
// y[t] += w[t,j] * FFN_e(x_t) over the pairs (t, j) routed to it, in fp32.
class ThreadPool;
struct HostJob {
    int fmt;
    Layout lay;
    int H, I, T, k;
    const float* x;                 // [T,H] fp32
    const uint16_t* xb = nullptr;   // [T,H] the same values as bf16 bits, when they are bf16
    const int32_t* ids;             // [T,k]
    const float* w;                 // [T,k]
    const uint8_t* const* experts;  // pool block per expert id (null: not host-executed)
    float* y;                       // [T,H] accumulated (zeroed by the caller)
};
void host_ffn(ThreadPool* pool, const HostJob& job, std::vector<float>& scratch);
// True when host_ffn takes the AVX512_BF16 route for bf16, MXFP4, NVFP4 and FP8
// experts (CPU support, unless the environment sets EO_HOST_ISA=avx2).
bool host_ffn_uses_avx512bf16();
// The weight decode of that route, for tests: 32 codes of `fmt` (FP8: 32 bytes,
// giving value / 256; MXFP4 / NVFP4: 16 bytes, giving the unscaled e2m1 values)
// as 32 bf16 bit patterns in out. False when the route is not available.
bool host_decode_codes(int fmt, const uint8_t* codes, uint16_t* out);
ThreadPool* threadpool_create(int n);
void threadpool_destroy(ThreadPool* p);
int threadpool_size(ThreadPool* p);
// Run fn(task) for task in [0, ntasks) on the pool (the calling thread included).
void threadpool_run(ThreadPool* p, int ntasks, const std::function<void(int)>& fn);

}  // namespace eo
