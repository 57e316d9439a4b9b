// Router: fp32 logits in a fixed accumulation order, top-k, softmax.
//
// Routing is the first step of the MoE layer (zhichai.net article, section 2,
// Decode paragraph: each token activates a few routed experts). Top-k ids must
// be reproducible bit for bit, so the logits follow one fixed order: lane i of
// a 64-wide wavefront accumulates the terms h = i, i+64, i+128, ... with fused
// multiply-adds from +0, then an xor butterfly (s = 32..1) adds the 64 partial
// sums; the result is lane 0's value. The wavefront width of CDNA is exactly
// the 64 chains, so each chain is one lane and the butterfly is six shuffles.
#include "dev_common.h"
#include "eo_internal.h"
#include "route_dev.h"
#include "entry_dev.h"

namespace eo {

namespace {

constexpr int kTT = 4;  // tokens per wavefront
constexpr int kEE = 8;  // experts per wavefront

// One wavefront computes z for kTT tokens x kEE experts; 4 wavefronts per block
// share the tokens and take consecutive expert groups.
template <bool BF16>
__global__ __launch_bounds__(256) void k_logits(const void* __restrict__ xv,
                                                const float* __restrict__ R, int T, int E, int H,
                                                float* __restrict__ z) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * kTT;
    const int e0 = (blockIdx.y * 4 + wave) * kEE;
    if (e0 >= E) return;
    float acc[kTT][kEE];
#pragma unroll
    for (int a = 0; a < kTT; ++a)
#pragma unroll
        for (int b = 0; b < kEE; ++b) acc[a][b] = 0.0f;
    int trow[kTT];
#pragma unroll
    for (int a = 0; a < kTT; ++a) trow[a] = min(t0 + a, T - 1);
    int erow[kEE];
#pragma unroll
    for (int b = 0; b < kEE; ++b) erow[b] = min(e0 + b, E - 1);

    for (int h = lane; h < H; h += 64) {
        float xv_[kTT], rv[kEE];
#pragma unroll
        for (int a = 0; a < kTT; ++a) {
            if (BF16)
                xv_[a] = bf16_f32(((const uint16_t*)xv)[(size_t)trow[a] * H + h]);
            else
                xv_[a] = ((const float*)xv)[(size_t)trow[a] * H + h];
        }
#pragma unroll
        for (int b = 0; b < kEE; ++b) rv[b] = R[(size_t)erow[b] * H + h];
#pragma unroll
        for (int a = 0; a < kTT; ++a)
#pragma unroll
            for (int b = 0; b < kEE; ++b) acc[a][b] = __builtin_fmaf(xv_[a], rv[b], acc[a][b]);
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
#pragma unroll
        for (int a = 0; a < kTT; ++a)
#pragma unroll
            for (int b = 0; b < kEE; ++b) acc[a][b] = acc[a][b] + __shfl_xor(acc[a][b], s, 64);
    }
    if (lane == 0) {
#pragma unroll
        for (int a = 0; a < kTT; ++a)
#pragma unroll
            for (int b = 0; b < kEE; ++b)
                if (t0 + a < T && e0 + b < E) z[(size_t)(t0 + a) * E + e0 + b] = acc[a][b];
    }
}

// One wavefront per token.
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ z, int T, int E, int k,
                                              const int32_t* __restrict__ forced,
                                              int32_t* __restrict__ ids, float* __restrict__ w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_token(z + (size_t)t * E, E, k, forced ? forced + (size_t)t * k : nullptr,
               ids + (size_t)t * k, w + (size_t)t * k);
}

// ---------------------------------------------------------------- many tokens
// Same accumulation order, with the operands interleaved per chain so that a
// 16-byte load gives a lane several consecutive steps of its own chain and a
// wavefront's load is one contiguous 1 KiB: router Rq[e][j/4][i][j%4] =
// R[e][i + 64 j] (fp32, 4 steps per load) and activations
// xq[t][j/8][i][j%8] = x[t][i + 64 j] (bf16, 8 steps per load). The FMAs still
// run j = 0, 1, ... in order from +0 and the butterfly is unchanged, so z is
// bit-identical to the direct kernel.
constexpr int kTT2 = 8, kEE2 = 8;

__global__ __launch_bounds__(64) void k_chain_transpose(const uint16_t* __restrict__ x, int H,
                                                        uint16_t* __restrict__ xq) {
    const int t = blockIdx.x, i = threadIdx.x, J8 = H / 512;
    const uint16_t* xr = x + (size_t)t * H;
    uint4* dst = (uint4*)xq + (size_t)t * J8 * 64;
    for (int j8 = 0; j8 < J8; ++j8) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            w[q] = (uint32_t)xr[i + 64 * (8 * j8 + 2 * q)] |
                   ((uint32_t)xr[i + 64 * (8 * j8 + 2 * q + 1)] << 16);
        dst[(size_t)j8 * 64 + i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

__global__ __launch_bounds__(256) void k_logits_chains(const uint16_t* __restrict__ xq,
                                                       const float* __restrict__ Rq, int T, int E,
                                                       int H, float* __restrict__ z) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * kTT2;
    const int e0 = (blockIdx.y * 4 + wave) * kEE2;
    const int J8 = H / 512;
    float acc[kTT2][kEE2];
#pragma unroll
    for (int a = 0; a < kTT2; ++a)
#pragma unroll
        for (int b = 0; b < kEE2; ++b) acc[a][b] = 0.0f;
    const uint4* xp[kTT2];
#pragma unroll
    for (int a = 0; a < kTT2; ++a) xp[a] = (const uint4*)xq + (size_t)min(t0 + a, T - 1) * J8 * 64 + lane;
    const float4* rp[kEE2];
#pragma unroll
    for (int b = 0; b < kEE2; ++b) rp[b] = (const float4*)Rq + (size_t)(e0 + b) * (2 * J8) * 64 + lane;
    for (int j8 = 0; j8 < J8; ++j8) {
        float xv[kTT2][8];
#pragma unroll
        for (int a = 0; a < kTT2; ++a) {
            uint4 q = xp[a][(size_t)j8 * 64];
            uint32_t wds[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                xv[a][2 * c] = bf16_f32(wds[c] & 0xFFFFu);
                xv[a][2 * c + 1] = bf16_f32(wds[c] >> 16);
            }
        }
#pragma unroll
        for (int b = 0; b < kEE2; ++b) {
            float4 r0 = rp[b][(size_t)(2 * j8) * 64], r1 = rp[b][(size_t)(2 * j8 + 1) * 64];
            float rv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
#pragma unroll
                for (int a = 0; a < kTT2; ++a) acc[a][b] = __builtin_fmaf(xv[a][jj], rv[jj], acc[a][b]);
        }
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
#pragma unroll
        for (int a = 0; a < kTT2; ++a)
#pragma unroll
            for (int b = 0; b < kEE2; ++b) acc[a][b] = acc[a][b] + __shfl_xor(acc[a][b], s, 64);
    }
    if (lane == 0) {
#pragma unroll
        for (int a = 0; a < kTT2; ++a)
            if (t0 + a < T)
#pragma unroll
                for (int b = 0; b < kEE2; ++b) z[(size_t)(t0 + a) * E + e0 + b] = acc[a][b];
    }
}

// ---------------------------------------------------------------- layer entry
__global__ __launch_bounds__(256) void k_entry(EntryArgs a) {
    extern __shared__ float s_u[];  // [H] fp32 values of the bf16 u
    entry_body(a, s_u);
}

}  // namespace

bool entry_ok(int E, int H, int act_bf16) {
    return act_bf16 && H % 512 == 0 && E % 4 == 0 && H <= 16384;
}

hipError_t launch_entry(const EntryArgs& a, hipStream_t s) {
    k_entry<<<(a.E + 3) / 4, 256, sizeof(float) * a.H, s>>>(a);
    return hipGetLastError();
}

bool route_chains_ok(int T, int E, int H, int act_bf16) {
    return act_bf16 && T >= 32 && H % 512 == 0 && E % (4 * kEE2) == 0;
}

hipError_t launch_route(const void* x, int act_bf16, const float* R, const float* Rt, int T,
                        int E, int H, int k, const int32_t* forced, int32_t* ids, float* w,
                        float* g_z, uint16_t* xT, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (Rt && xT && route_chains_ok(T, E, H, act_bf16)) {
        k_chain_transpose<<<T, 64, 0, s>>>((const uint16_t*)x, H, xT);
        k_logits_chains<<<dim3((T + kTT2 - 1) / kTT2, E / (4 * kEE2)), 256, 0, s>>>(xT, Rt, T, E, H, g_z);
    } else {
        dim3 grid((T + kTT - 1) / kTT, (E + 4 * kEE - 1) / (4 * kEE));
        if (act_bf16)
            k_logits<true><<<grid, 256, 0, s>>>(x, R, T, E, H, g_z);
        else
            k_logits<false><<<grid, 256, 0, s>>>(x, R, T, E, H, g_z);
    }
    k_topk<<<(T + 3) / 4, 256, 0, s>>>(g_z, T, E, k, forced, ids, w);
    return hipGetLastError();
}

}  // namespace eo
