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

__device__ __forceinline__ bool better(float za, int ia, float zb, int ib) {
    return za > zb || (za == zb && ia < ib);
}

// One wavefront per token: k rounds of (max z, min id) over the E logits.
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ z, int T, int E, int k,
                                              const int32_t* __restrict__ forced,
                                              int32_t* __restrict__ ids, float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* zt = z + (size_t)t * E;
    float zs[kMaxK];
    int is[kMaxK];
    if (forced) {
        for (int j = 0; j < k; ++j) {
            is[j] = forced[(size_t)t * k + j];
            // out-of-range ids are reported by the lookup; read in bounds here
            zs[j] = zt[min(max(is[j], 0), E - 1)];
        }
    } else {
        constexpr int kPer = kMaxE / 64;
        float zl[kPer];
        uint32_t taken = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            int e = lane + 64 * i;
            zl[i] = e < E ? zt[e] : -INFINITY;
        }
        for (int j = 0; j < k; ++j) {
            float bz = -INFINITY;
            int bi = 0x7FFFFFFF;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                int e = lane + 64 * i;
                if (e < E && !((taken >> i) & 1u) && (bi == 0x7FFFFFFF || better(zl[i], e, bz, bi))) {
                    bz = zl[i];
                    bi = e;
                }
            }
#pragma unroll
            for (int s = 32; s >= 1; s >>= 1) {
                float oz = __shfl_xor(bz, s, 64);
                int oi = __shfl_xor(bi, s, 64);
                if (oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || better(oz, oi, bz, bi))) {
                    bz = oz;
                    bi = oi;
                }
            }
            zs[j] = bz;
            is[j] = bi;
            if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        }
    }
    if (lane == 0) {
        float zmax = zs[0];
        for (int j = 1; j < k; ++j) zmax = fmaxf(zmax, zs[j]);
        float ex[kMaxK], sum = 0.0f;
        for (int j = 0; j < k; ++j) {
            ex[j] = expf(zs[j] - zmax);
            sum += ex[j];
        }
        for (int j = 0; j < k; ++j) {
            ids[(size_t)t * k + j] = is[j];
            w[(size_t)t * k + j] = ex[j] / sum;
        }
    }
}

// ---------------------------------------------------------------- many tokens
// Same accumulation order, with the operands laid out per chain: chain i of
// row r is stored contiguously (xT[t][i][j] = x[t][i + 64 j], Rt[e][i][j] =
// R[e][i + 64 j]), so lane i reads 8 (x) or 4 (R) consecutive steps j with one
// 16-byte load instead of one element per load. The FMAs still run j = 0, 1, ...
// in order from +0, and the butterfly is unchanged, so z is bit-identical.
constexpr int kTT2 = 8, kEE2 = 8;

__global__ __launch_bounds__(64) void k_chain_transpose(const uint16_t* __restrict__ x, int H,
                                                        uint16_t* __restrict__ xT) {
    const int t = blockIdx.x, i = threadIdx.x, J = H / 64;
    const uint16_t* xr = x + (size_t)t * H;
    uint16_t* dst = xT + ((size_t)t * 64 + i) * J;
    for (int j0 = 0; j0 < J; j0 += 8) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            w[q] = (uint32_t)xr[i + 64 * (j0 + 2 * q)] | ((uint32_t)xr[i + 64 * (j0 + 2 * q + 1)] << 16);
        *(uint4*)(dst + j0) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

__global__ __launch_bounds__(256) void k_logits_chains(const uint16_t* __restrict__ xT,
                                                       const float* __restrict__ Rt, int T, int E,
                                                       int H, float* __restrict__ z) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * kTT2;
    const int e0 = (blockIdx.y * 4 + wave) * kEE2;
    const int J = H / 64;
    float acc[kTT2][kEE2];
#pragma unroll
    for (int a = 0; a < kTT2; ++a)
#pragma unroll
        for (int b = 0; b < kEE2; ++b) acc[a][b] = 0.0f;
    const uint16_t* xp[kTT2];
#pragma unroll
    for (int a = 0; a < kTT2; ++a) xp[a] = xT + ((size_t)min(t0 + a, T - 1) * 64 + lane) * J;
    const float* rp[kEE2];
#pragma unroll
    for (int b = 0; b < kEE2; ++b) rp[b] = Rt + ((size_t)(e0 + b) * 64 + lane) * J;
    for (int j0 = 0; j0 < J; j0 += 8) {
        float xv[kTT2][8];
#pragma unroll
        for (int a = 0; a < kTT2; ++a) {
            uint4 q = *(const uint4*)(xp[a] + j0);
            uint32_t wds[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                xv[a][2 * c] = bf16_f32(wds[c] & 0xFFFFu);
                xv[a][2 * c + 1] = bf16_f32(wds[c] >> 16);
            }
        }
#pragma unroll
        for (int b = 0; b < kEE2; ++b) {
            float4 r0 = *(const float4*)(rp[b] + j0), r1 = *(const float4*)(rp[b] + j0 + 4);
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

}  // namespace

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
