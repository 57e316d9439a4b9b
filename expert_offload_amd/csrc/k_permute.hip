// Token permutation by expert, weighted combine, residual and the RMS
// normalisation that turns the residual stream into a layer's input.
//
// Grouped expert execution needs each expert's tokens contiguous: the (token,
// slot) pairs whose expert is device-resident are grouped by expert, stable in
// pair order (t*k + j), into perm_pair; the grouped GEMM reads each grouped
// row's input row of X through it (no permuted copy of X is made). The shared
// expert (papers.ananclaw.com explainer, "core method" section 4, names it as
// an architecture axis) is one more group holding every token. After the
// grouped FFN, each pair's weighted output sits at o_pairs[t*k + j] (shared:
// o_pairs[T*k + t]; bf16 with bf16 activations, else fp32) and the combine sums
// a token's rows in fixed j order in fp32.
#include "dev_common.h"
#include "eo_internal.h"

namespace eo {

namespace {

constexpr int kChunk = 1024;  // pairs per permute block

__device__ __forceinline__ bool pair_resident(const int32_t* e2slot, int all_resident, int e,
                                              int E) {
    if (e < 0 || e >= E) return false;
    return all_resident || e2slot[e] >= 0;
}

// Per-chunk expert histogram: chunk_cnt[b][e].
__global__ __launch_bounds__(1024) void k_hist(const int32_t* __restrict__ ids,
                                               const int32_t* __restrict__ e2slot,
                                               int all_resident, int P, int E,
                                               int32_t* __restrict__ chunk_cnt) {
    __shared__ int h[kMaxE];
    for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
    __syncthreads();
    int p = blockIdx.x * kChunk + threadIdx.x;
    if (p < P) {
        int e = ids[p];
        if (pair_resident(e2slot, all_resident, e, E)) atomicAdd(&h[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        chunk_cnt[(size_t)blockIdx.x * E + e] = h[e];
}

// Single block: per expert, exclusive scan over chunks (in place: chunk base
// within the expert); group counts, offsets and tile offsets.
__global__ __launch_bounds__(1024) void k_scan(int32_t* __restrict__ chunk_cnt, int nchunks,
                                               int E, int has_shared, int T,
                                               int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ tile_off) {
    __shared__ int cnt[kMaxE + 1];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int run = 0;
        for (int b = 0; b < nchunks; ++b) {
            int c = chunk_cnt[(size_t)b * E + e];
            chunk_cnt[(size_t)b * E + e] = run;
            run += c;
        }
        cnt[e] = run;
    }
    if (threadIdx.x == 0) cnt[E] = has_shared ? T : 0;
    __syncthreads();
    if (threadIdx.x == 0) {
        int off = 0, toff = 0;
        for (int g = 0; g <= E; ++g) {
            counts[g] = cnt[g];
            offsets[g] = off;
            tile_off[g] = toff;
            off += cnt[g];
            toff += (cnt[g] + kTileM - 1) / kTileM;
        }
        offsets[E + 1] = off;
        tile_off[E + 1] = toff;
    }
}

// Scatter: stable rank of each pair within its expert inside the chunk, then
// its destination row; rows of x are copied by whole wavefronts (16 B/lane).
__global__ __launch_bounds__(1024) void k_scatter(const int32_t* __restrict__ ids,
                                                  const int32_t* __restrict__ e2slot,
                                                  int all_resident, int P, int E,
                                                  const int32_t* __restrict__ chunk_base,
                                                  const int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ perm_pair) {
    __shared__ int se[kChunk];
    const int tid = threadIdx.x;
    const int p = blockIdx.x * kChunk + tid;
    int e = -1;
    if (p < P) {
        int ee = ids[p];
        if (pair_resident(e2slot, all_resident, ee, E)) e = ee;
    }
    se[tid] = e;
    __syncthreads();
    if (e >= 0) {
        int r = 0;
        for (int i = 0; i < tid; ++i) r += (se[i] == e);
        perm_pair[offsets[e] + chunk_base[(size_t)blockIdx.x * E + e] + r] = p;
    }
}

// Shared-expert group: rows offsets[E] + t hold token t.
__global__ __launch_bounds__(256) void k_shared_rows(int T, int Tk, const int32_t* __restrict__ offsets,
                                                     int E, int32_t* __restrict__ perm_pair) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < T) perm_pair[offsets[E] + t] = Tk + t;
}

// Four consecutive pair outputs as fp32 (bf16 storage with bf16 activations).
template <bool BF16>
__device__ __forceinline__ float4 pair4(const void* o_pairs, size_t row, int H, int h4) {
    if (BF16) {
        uint2 v = ((const uint2*)((const uint16_t*)o_pairs + row * H))[h4];
        return make_float4(bf16_f32(v.x & 0xFFFFu), bf16_f32(v.x >> 16), bf16_f32(v.y & 0xFFFFu),
                           bf16_f32(v.y >> 16));
    }
    return ((const float4*)((const float*)o_pairs + row * H))[h4];
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ o_pairs,
                                                 const int32_t* __restrict__ ids,
                                                 const int32_t* __restrict__ e2slot,
                                                 int all_resident, int has_shared,
                                                 const float* __restrict__ y_host, int T, int k,
                                                 int E, int H, float* __restrict__ y,
                                                 void* __restrict__ x_res) {
    const int t = blockIdx.y;
    const int h4 = blockIdx.x * blockDim.x + threadIdx.x;
    if (h4 * 4 >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        int e = ids[(size_t)t * k + j];
        if (!pair_resident(e2slot, all_resident, e, E)) continue;
        float4 v = pair4<BF16>(o_pairs, (size_t)t * k + j, H, h4);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (has_shared) {
        float4 v = pair4<BF16>(o_pairs, (size_t)T * k + t, H, h4);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (y_host) {
        float4 v = ((const float4*)(y_host + (size_t)t * H))[h4];
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (y) ((float4*)(y + (size_t)t * H))[h4] = acc;
    if (x_res) {
        if (BF16) {
            uint2* xp = (uint2*)((uint16_t*)x_res + (size_t)t * H) + h4;
            uint2 xv = *xp;
            float a = bf16_f32(xv.x & 0xFFFFu) + acc.x, b = bf16_f32(xv.x >> 16) + acc.y;
            float c = bf16_f32(xv.y & 0xFFFFu) + acc.z, d = bf16_f32(xv.y >> 16) + acc.w;
            *xp = make_uint2(f32_bf16_rne(a) | (f32_bf16_rne(b) << 16),
                             f32_bf16_rne(c) | (f32_bf16_rne(d) << 16));
        } else {
            float4* xp = (float4*)((float*)x_res + (size_t)t * H) + h4;
            float4 xv = *xp;
            *xp = make_float4(xv.x + acc.x, xv.y + acc.y, xv.z + acc.z, xv.w + acc.w);
        }
    }
}

// Layer input from the residual stream: u = r / sqrt(mean(r^2) + 1e-6), one
// block per token. The sum of squares is taken in fp32 in a fixed order (per
// lane, then a butterfly within each wavefront, then the wavefronts in order),
// so the result does not depend on scheduling; u is rounded to the storage type.
template <bool BF16>
__global__ __launch_bounds__(256) void k_rmsnorm(const void* __restrict__ r, void* __restrict__ u,
                                                 int H) {
    __shared__ float part[4];
    const int t = blockIdx.x, tid = threadIdx.x;
    const int nv = BF16 ? H / 8 : H / 4;  // 16-byte vectors per row
    const uint4* rv = (const uint4*)((const uint8_t*)r + (size_t)t * H * (BF16 ? 2 : 4));
    uint4* uv = (uint4*)((uint8_t*)u + (size_t)t * H * (BF16 ? 2 : 4));
    float ss = 0.0f;
    for (int c = tid; c < nv; c += 256) {
        uint4 v = rv[c];
        if (BF16) {
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float a = bf16_f32(w[i] & 0xFFFFu), b = bf16_f32(w[i] >> 16);
                ss = fmaf(a, a, ss);
                ss = fmaf(b, b, ss);
            }
        } else {
            float f[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                          __uint_as_float(v.w)};
#pragma unroll
            for (int i = 0; i < 4; ++i) ss = fmaf(f[i], f[i], ss);
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    if ((tid & 63) == 0) part[tid >> 6] = ss;
    __syncthreads();
    const float tot = ((part[0] + part[1]) + part[2]) + part[3];
    const float inv = 1.0f / sqrtf(tot / (float)H + 1e-6f);
    for (int c = tid; c < nv; c += 256) {
        uint4 v = rv[c];
        if (BF16) {
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                w[i] = f32_bf16_rne(bf16_f32(w[i] & 0xFFFFu) * inv) |
                       (f32_bf16_rne(bf16_f32(w[i] >> 16) * inv) << 16);
            uv[c] = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
            uv[c] = make_uint4(__float_as_uint(__uint_as_float(v.x) * inv),
                               __float_as_uint(__uint_as_float(v.y) * inv),
                               __float_as_uint(__uint_as_float(v.z) * inv),
                               __float_as_uint(__uint_as_float(v.w) * inv));
        }
    }
}

}  // namespace

hipError_t launch_rmsnorm(const void* r, void* u, int T, int H, int act_bf16, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (act_bf16)
        k_rmsnorm<true><<<T, 256, 0, s>>>(r, u, H);
    else
        k_rmsnorm<false><<<T, 256, 0, s>>>(r, u, H);
    return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, const int32_t* e2slot, int all_resident, int T,
                          int k, int E, int has_shared, PermuteBufs b, hipStream_t s) {
    const int P = T * k;
    const int nchunks = (P + kChunk - 1) / kChunk;
    if (nchunks > 0)
        k_hist<<<nchunks, 1024, 0, s>>>(ids, e2slot, all_resident, P, E, b.chunk_cnt);
    k_scan<<<1, 1024, 0, s>>>(b.chunk_cnt, nchunks, E, has_shared, T, b.counts, b.offsets,
                              b.tile_off);
    if (nchunks > 0)
        k_scatter<<<nchunks, 1024, 0, s>>>(ids, e2slot, all_resident, P, E, b.chunk_cnt,
                                           b.offsets, b.perm_pair);
    if (has_shared)
        k_shared_rows<<<(T + 255) / 256, 256, 0, s>>>(T, P, b.offsets, E, b.perm_pair);
    return hipGetLastError();
}

hipError_t launch_combine(const void* o_pairs, const int32_t* ids, const int32_t* e2slot,
                          int all_resident, int has_shared, const float* y_host, int T, int k,
                          int H, float* y, void* x_res, int act_bf16, hipStream_t s, int E) {
    dim3 grid((H / 4 + 255) / 256, T);
    if (act_bf16)
        k_combine<true><<<grid, 256, 0, s>>>(o_pairs, ids, e2slot, all_resident, has_shared,
                                             y_host, T, k, E, H, y, x_res);
    else
        k_combine<false><<<grid, 256, 0, s>>>(o_pairs, ids, e2slot, all_resident, has_shared,
                                              y_host, T, k, E, H, y, x_res);
    return hipGetLastError();
}


}  // namespace eo
