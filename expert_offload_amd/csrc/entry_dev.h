// Layer entry for one token (device part shared by the entry kernels).
#pragma once
#include "dev_common.h"
#include "eo_internal.h"

namespace eo {

// One token entering a layer of the stacked decode step: residual update from
// the previous layer's parts, RMS normalisation, logits. Every block rebuilds
// the token's row (r_new = r + sum of parts + host part, stored in bf16) and
// u = r_new / sqrt(mean(r_new^2) + 1e-6) in the same fixed order as the
// separate residual and normalisation kernels; block 0 writes r_new, y and u.
// Each wavefront then owns one expert's logit: lane i runs chain i over the
// interleaved router Rq[e][:][i][:] against u[i + 64 j] from LDS, then the
// butterfly.
// acc = fma chain over j = 0..J-1 of u[lane + 64 j] * R[e][lane + 64 j] with
// rq = &Rq[e][0][lane] (float4 steps 64 apart), loading CH steps of the chain
// (CH/4 coalesced 16-byte loads) before their FMAs.
template <int CH>
__device__ __forceinline__ float chain_dot(const float4* __restrict__ rq, const float* s_u,
                                           int lane, int J, float acc) {
    for (int j0 = 0; j0 < J; j0 += CH) {
        float rr[CH];
#pragma unroll
        for (int q = 0; q < CH / 4; ++q) {
            float4 v = rq[(size_t)(j0 / 4 + q) * 64];
            rr[4 * q] = v.x; rr[4 * q + 1] = v.y; rr[4 * q + 2] = v.z; rr[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int jj = 0; jj < CH; ++jj) acc = __builtin_fmaf(s_u[lane + 64 * (j0 + jj)], rr[jj], acc);
    }
    return acc;
}

// y = the previous layer's partial outputs summed in part order, then the
// host part, at the 8 values of column block c: the additions of one loop over
// the parts. Every row is requested before the first add, so the reads take one
// memory round trip instead of one per part; the host part, read from host
// memory, is requested first. The places past nparts (and the host part when
// there is none) add +0.0, which changes no bits: y starts at +0.0 and a sum
// of floats is never -0.0 under round to nearest.
template <int NP>
__device__ __forceinline__ void sum_parts_n(const EntryArgs& a, int c, float (&y)[8]) {
    const bool hp = a.y_host != nullptr;
    // with no host part, a part row stands in for its (unused) read
    const float4* ph = (const float4*)(hp ? a.y_host : a.parts) + 2 * c;
    const float4 h0 = ph[0], h1 = ph[1];
    float4 p[NP > 0 ? NP : 1][2];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const float4* pj = (const float4*)(a.parts + (size_t)min(j, a.nparts - 1) * a.H) + 2 * c;
        p[j][0] = pj[0];
        p[j][1] = pj[1];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) y[q] = 0.0f;
    const float4 z4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const bool on = j < a.nparts;
        const float4 p0 = on ? p[j][0] : z4, p1 = on ? p[j][1] : z4;
        y[0] += p0.x; y[1] += p0.y; y[2] += p0.z; y[3] += p0.w;
        y[4] += p1.x; y[5] += p1.y; y[6] += p1.z; y[7] += p1.w;
    }
    const float4 q0 = hp ? h0 : z4, q1 = hp ? h1 : z4;
    y[0] += q0.x; y[1] += q0.y; y[2] += q0.z; y[3] += q0.w;
    y[4] += q1.x; y[5] += q1.y; y[6] += q1.z; y[7] += q1.w;
}

__device__ __forceinline__ void sum_parts(const EntryArgs& a, int c, float (&y)[8]) {
    if (a.nparts <= 0)
        sum_parts_n<0>(a, c, y);
    else if (a.nparts <= 4)
        sum_parts_n<4>(a, c, y);
    else if (a.nparts <= 8)
        sum_parts_n<8>(a, c, y);
    else if (a.nparts <= 12)
        sum_parts_n<12>(a, c, y);
    else
        sum_parts_n<kMaxK + 1>(a, c, y);
}

// s_u: [H] floats of LDS. Wavefronts past the last expert skip the logit.
__device__ __forceinline__ void entry_body(const EntryArgs& a, float* s_u) {
    __shared__ float part[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, nv = H / 8;
    const uint4* rv = (const uint4*)a.r_in;
    const bool writer = blockIdx.x == 0;
    // this wavefront's expert: the first kPre steps of its router chain are
    // loaded now, so their latency hides behind the residual and the norm
    constexpr int kPre = 32;
    const int e = blockIdx.x * 4 + wave;
    const int J = H / 64, npre = min(J, kPre);  // J % 8 == 0
    const float4* rq = (const float4*)a.Rt + (size_t)min(e, a.E - 1) * (J / 4) * 64 + lane;
    float4 pre[kPre / 4];
#pragma unroll
    for (int q = 0; q < kPre / 4; ++q)
        if (4 * q < npre) pre[q] = rq[(size_t)q * 64];
    float ss = 0.0f;
    for (int c = tid; c < nv; c += 256) {
        uint4 v = rv[c];
        uint32_t wd[4] = {v.x, v.y, v.z, v.w};
        if (a.nparts > 0 || a.y_host) {
            float y[8];
            sum_parts(a, c, y);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                wd[q] = f32_bf16_rne(bf16_f32(wd[q] & 0xFFFFu) + y[2 * q]) |
                        (f32_bf16_rne(bf16_f32(wd[q] >> 16) + y[2 * q + 1]) << 16);
            if (writer) {
                ((uint4*)a.r_out)[c] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                if (a.y_out) {
                    ((float4*)a.y_out)[2 * c] = make_float4(y[0], y[1], y[2], y[3]);
                    ((float4*)a.y_out)[2 * c + 1] = make_float4(y[4], y[5], y[6], y[7]);
                }
            }
        } else if (writer && a.r_out != a.r_in) {
            ((uint4*)a.r_out)[c] = v;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float lo = bf16_f32(wd[q] & 0xFFFFu), hi = bf16_f32(wd[q] >> 16);
            ss = fmaf(lo, lo, ss);
            ss = fmaf(hi, hi, ss);
            s_u[8 * c + 2 * q] = lo;  // r_new for now
            s_u[8 * c + 2 * q + 1] = hi;
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    if (lane == 0) part[wave] = ss;
    __syncthreads();
    const float tot = ((part[0] + part[1]) + part[2]) + part[3];
    const float inv = 1.0f / sqrtf(tot / (float)H + 1e-6f);
    for (int c = tid; c < nv; c += 256) {
        uint32_t wd[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t lo = f32_bf16_rne(s_u[8 * c + 2 * q] * inv);
            uint32_t hi = f32_bf16_rne(s_u[8 * c + 2 * q + 1] * inv);
            s_u[8 * c + 2 * q] = bf16_f32(lo);
            s_u[8 * c + 2 * q + 1] = bf16_f32(hi);
            wd[q] = lo | (hi << 16);
        }
        if (writer) ((uint4*)a.u)[c] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
    __syncthreads();
    if (e >= a.E) return;
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < kPre / 4; ++q) {
        if (4 * q < npre) {
            acc = __builtin_fmaf(s_u[lane + 64 * (4 * q)], pre[q].x, acc);
            acc = __builtin_fmaf(s_u[lane + 64 * (4 * q + 1)], pre[q].y, acc);
            acc = __builtin_fmaf(s_u[lane + 64 * (4 * q + 2)], pre[q].z, acc);
            acc = __builtin_fmaf(s_u[lane + 64 * (4 * q + 3)], pre[q].w, acc);
        }
    }
    if (J > kPre) {
        if ((J - kPre) % 32 == 0)
            acc = chain_dot<32>(rq + (size_t)(kPre / 4) * 64, s_u + 64 * kPre, lane, J - kPre, acc);
        else
            acc = chain_dot<8>(rq + (size_t)(kPre / 4) * 64, s_u + 64 * kPre, lane, J - kPre, acc);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc = acc + __shfl_xor(acc, m, 64);
    // a device-scope store: the fused entry + plan kernel reads the logits of
    // every workgroup without a cache writeback or invalidate
    if (lane == 0) __hip_atomic_store(&a.z[e], acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


}  // namespace eo
