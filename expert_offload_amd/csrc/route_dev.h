// Top-k selection and softmax weights of one token, by one wavefront.
//
// Shared by the router's top-k kernel and the plan kernel (which selects the
// experts itself when it is handed logits). Selection is k rounds of
// (max z, then smallest id); the weights are the softmax over the k selected
// logits. With forced ids the given ids are taken in their order and the
// softmax is taken over the logits at them.
#pragma once

#include "dev_common.h"
#include "eo_host.h"

namespace eo {

__device__ __forceinline__ bool topk_better(float za, int ia, float zb, int ib) {
    return za > zb || (za == zb && ia < ib);
}

// A logit read; kCoherent reads at device scope (logits other workgroups of
// the same launch stored at device scope, with no cache invalidate between).
template <bool kCoherent>
__device__ __forceinline__ float zload(const float* p) {
    if (kCoherent) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return *p;
}

// k rounds of (max z, then smallest id) over E <= 64 * kPer logits.
template <int kPer, bool kCoherent = false>
__device__ __forceinline__ void topk_select(const float* __restrict__ zt, int E, int k, float* zs,
                                            int* is) {
    const int lane = threadIdx.x & 63;
    {
        float zl[kPer];
        uint32_t taken = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            int e = lane + 64 * i;
            zl[i] = e < E ? zload<kCoherent>(zt + e) : -INFINITY;
        }
        for (int j = 0; j < k; ++j) {
            float bz = -INFINITY;
            int bi = 0x7FFFFFFF;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                int e = lane + 64 * i;
                if (e < E && !((taken >> i) & 1u) &&
                    (bi == 0x7FFFFFFF || topk_better(zl[i], e, bz, bi))) {
                    bz = zl[i];
                    bi = e;
                }
            }
#pragma unroll
            for (int s = 32; s >= 1; s >>= 1) {
                float oz = __shfl_xor(bz, s, 64);
                int oi = __shfl_xor(bi, s, 64);
                if (oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || topk_better(oz, oi, bz, bi))) {
                    bz = oz;
                    bi = oi;
                }
            }
            zs[j] = bz;
            is[j] = bi;
            if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        }
    }
}

// All 64 lanes of the wavefront call this; lane j < k writes ids[j] and w[j].
// w = softmax over the k selected logits: max, exponentials, their sum in
// j order, then one division per weight.
template <bool kCoherent = false>
__device__ __forceinline__ void topk_token(const float* __restrict__ zt, int E, int k,
                                           const int32_t* __restrict__ forced_t,
                                           int32_t* __restrict__ ids_t, float* __restrict__ w_t) {
    const int lane = threadIdx.x & 63;
    int my_i = 0;  // lane j < k: the j-th selected expert and its logit
    float my_z = -INFINITY;
    // per wavefront of the workgroup (up to 4); E <= 256 logits and -inf up
    // to the next multiple of 4
    __shared__ __attribute__((aligned(16))) float s_zw[4][260];
    __shared__ int32_t s_selw[4][kMaxK];
    float* s_z = s_zw[(threadIdx.x >> 6) & 3];
    int32_t* s_sel = s_selw[(threadIdx.x >> 6) & 3];
    if (forced_t) {
        // the ids and the logits are loaded together (one round trip); an
        // out-of-range id is reported by the lookup, its logit read in bounds
        if (lane < k) my_i = forced_t[lane];
        if (E <= 256) {
            for (int e = lane; e < E; e += 64) s_z[e] = zload<kCoherent>(zt + e);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            if (lane < k) my_z = s_z[min(max(my_i, 0), E - 1)];
        } else if (lane < k) {
            my_z = zload<kCoherent>(zt + min(max(my_i, 0), E - 1));
        }
    } else if (E <= 256) {
        // each logit's rank = how many logits beat it (larger, or equal with a
        // smaller id); the k of rank < k are the selection, in (z desc, id asc)
        // order: the same result as k rounds of selection
        for (int e = lane; e < E; e += 64) s_z[e] = zload<kCoherent>(zt + e);
        if (lane < ((E + 3) & ~3) - E) s_z[E + lane] = -INFINITY;  // never beats a logit
        if (lane < k) s_sel[lane] = -1;  // stays -1 only for unordered (NaN) logits
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        for (int e = lane; e < E; e += 64) {
            const float z = s_z[e];
            int r = 0;
            for (int o = 0; o < E; o += 4) {  // four logits per LDS read
                const float4 zo = *(const float4*)(s_z + o);
                r += zo.x > z || (zo.x == z && o < e);
                r += zo.y > z || (zo.y == z && o + 1 < e);
                r += zo.z > z || (zo.z == z && o + 2 < e);
                r += zo.w > z || (zo.w == z && o + 3 < e);
            }
            if (r < k) s_sel[r] = e;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        if (lane < k) {
            my_i = s_sel[lane];
            my_z = my_i >= 0 ? s_z[my_i] : -INFINITY;
        }
    } else {
        float zs[kMaxK];
        int is[kMaxK];
        topk_select<kMaxE / 64, kCoherent>(zt, E, k, zs, is);
        for (int j = 0; j < k; ++j)
            if (lane == j) {
                my_z = zs[j];
                my_i = is[j];
            }
    }
    float zmax = my_z;  // lanes >= k hold -inf
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) zmax = fmaxf(zmax, __shfl_xor(zmax, m, 64));
    const float ex = expf(my_z - zmax);
    float sum = 0.0f;
    for (int j = 0; j < k; ++j)
        sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
    if (lane < k) {
        ids_t[lane] = my_i;
        w_t[lane] = ex / sum;
    }
}

}  // namespace eo
