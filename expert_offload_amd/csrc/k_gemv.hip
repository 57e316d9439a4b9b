// Decode expert FFN (T = 1): dequant-GEMV over the resident routed experts and
// the shared expert, straight from the cache slots.
//
// A decode step reads every selected expert's weights once to produce one
// token (zhichai.net article, section 2, Decode paragraph: hits are served from
// the device cache), so the kernel is bound by HBM bandwidth: weights are read
// in 16-byte chunks per lane, decoded in registers and multiplied into fp32
// accumulators; nothing is staged.
//   phase A: for each expert j, h_j = silu(W_gate x) * (W_up x)   (fp32 [I])
//   phase B: y_j = w_j * W_down h_j                               (fp32 [H])
// followed by a reduction over j in fixed order (plus host-executed results).
// Experts the plan sends to the host are skipped here (phase B writes zeros).
#include <hip/hip_ext.h>

#include <cstdlib>

#include "decode_dev.h"
#include "dev_common.h"
#include "eo_internal.h"
#include "fill_dev.h"

namespace eo {

namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct GemvArgs {
    GroupW gw;
    Layout lay;
    const DevPlan* plan;
    const int32_t* ids;
    const float* w;
    int k, E, H, I, nexp;
    const void* x;
    float* h;      // [nexp, I]
    float* yp;     // [nexp, H]
    GemvExperts ex;  // when ex.valid: weight base and routing weight per slot j
};

// Elements per 16-byte weight chunk.
template <int FMT> struct Cw;
template <> struct Cw<EO_W_FP32> { static constexpr int n = 4; };
template <> struct Cw<EO_W_BF16> { static constexpr int n = 8; };
template <> struct Cw<EO_W_FP8> { static constexpr int n = 16; };
template <> struct Cw<EO_W_MXFP4> { static constexpr int n = 32; };
template <> struct Cw<EO_W_NVFP4> { static constexpr int n = 32; };

__device__ __forceinline__ float2 bf16pair(uint32_t v) {
    return make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xFFFF0000u));
}

// x values of one chunk, as fp32.
template <int N, bool XBF16>
__device__ __forceinline__ void load_x(const void* x, int base, float* xv) {
    if (XBF16) {
        const uint4* p = (const uint4*)((const uint16_t*)x + base);
#pragma unroll
        for (int q = 0; q < N / 8; ++q) {
            uint4 v = p[q];
            uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float2 f = bf16pair(wds[i]);
                xv[q * 8 + 2 * i] = f.x;
                xv[q * 8 + 2 * i + 1] = f.y;
            }
        }
    } else {
        const float4* p = (const float4*)((const float*)x + base);
#pragma unroll
        for (int q = 0; q < N / 4; ++q) {
            float4 v = p[q];
            xv[4 * q] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
        }
    }
}

// Dot of one weight chunk (row `row` of a matrix with K columns, chunk c) with
// xv; includes per-block scales (MXFP4 e8m0, NVFP4 e4m3) but not per-row or
// per-tensor factors.
template <int FMT>
__device__ __forceinline__ float chunk_dot(const uint8_t* data, const uint8_t* scal, int row,
                                           int K, int c, const float* xv) {
    constexpr int N = Cw<FMT>::n;
    float s = 0.0f;
    if (FMT == EO_W_FP32) {
        float4 v = *(const float4*)((const float*)data + (size_t)row * K + c * N);
        s = v.x * xv[0] + v.y * xv[1] + v.z * xv[2] + v.w * xv[3];
    } else if (FMT == EO_W_BF16) {
        uint4 v = *(const uint4*)((const uint16_t*)data + (size_t)row * K + c * N);
        uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float2 f = bf16pair(wds[i]);
            s = fmaf(f.x, xv[2 * i], s);
            s = fmaf(f.y, xv[2 * i + 1], s);
        }
    } else if (FMT == EO_W_FP8) {
        uint4 v = *(const uint4*)(data + (size_t)row * K + c * N);
        uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < 4; ++b) s = fmaf(e4m3_f32((wds[i] >> (8 * b)) & 0xFF), xv[4 * i + b], s);
    } else {
        uint4 v = *(const uint4*)(data + (size_t)row * (K / 2) + c * 16);
        uint32_t wds[4] = {v.x, v.y, v.z, v.w};
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                uint32_t byte = (wds[i] >> (8 * b)) & 0xFF;
                float lo = e2m1_f32(byte & 0xF), hi = e2m1_f32(byte >> 4);
                int e = 8 * i + 2 * b;
                if (i < 2) {
                    s0 = fmaf(lo, xv[e], s0);
                    s0 = fmaf(hi, xv[e + 1], s0);
                } else {
                    s1 = fmaf(lo, xv[e], s1);
                    s1 = fmaf(hi, xv[e + 1], s1);
                }
            }
        if (FMT == EO_W_MXFP4) {
            s = (s0 + s1) * e8m0_f32(scal[(size_t)row * (K / 32) + c]);
        } else {
            const uint8_t* sp = scal + (size_t)row * (K / 16) + 2 * c;
            s = s0 * e4m3_f32(sp[0]) + s1 * e4m3_f32(sp[1]);
        }
    }
    return s;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
    return v;
}

// Resolve expert j of this decode call: weight base, or null if host-executed.
__device__ __forceinline__ const uint8_t* expert_base(const GemvArgs& a, int j) {
    if (a.ex.valid) return a.ex.base[j];
    if (j == a.k) return a.gw.shared_w;
    const int s = a.plan->tok_slot[j];
    if (s < 0) return nullptr;
    return a.gw.slots + (uint64_t)s * a.gw.stride;
}

constexpr int kRowsA = 4;  // gate rows (and as many up rows) per wavefront
constexpr int kRowsB = 8;  // down rows per wavefront

template <int FMT, bool XBF16>
__global__ __launch_bounds__(256) void k_gemv_up(GemvArgs a) {
    const int j = blockIdx.y;
    const uint8_t* wb = expert_base(a, j);
    if (!wb) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = (blockIdx.x * 4 + wave) * kRowsA;
    const uint8_t* data = wb + a.lay.d13;
    const uint8_t* scal = wb + a.lay.s13;
    constexpr int N = Cw<FMT>::n;
    const int nch = a.H / N;
    float acc[2 * kRowsA];
#pragma unroll
    for (int r = 0; r < 2 * kRowsA; ++r) acc[r] = 0.0f;
    for (int c = lane; c < nch; c += 64) {
        float xv[N];
        load_x<N, XBF16>(a.x, c * N, xv);
#pragma unroll
        for (int r = 0; r < kRowsA; ++r) {
            acc[r] += chunk_dot<FMT>(data, scal, r0 + r, a.H, c, xv);
            acc[kRowsA + r] += chunk_dot<FMT>(data, scal, a.I + r0 + r, a.H, c, xv);
        }
    }
#pragma unroll
    for (int r = 0; r < 2 * kRowsA; ++r) acc[r] = wave_sum(acc[r]);
    if (lane < kRowsA) {
        float g = acc[0], u = acc[kRowsA];
#pragma unroll
        for (int r = 1; r < kRowsA; ++r)
            if (lane == r) { g = acc[r]; u = acc[kRowsA + r]; }
        const int row = r0 + lane;
        if (FMT == EO_W_FP8) {
            g *= ((const float*)scal)[row];
            u *= ((const float*)scal)[a.I + row];
        } else if (FMT == EO_W_NVFP4) {
            const float* gl = (const float*)(wb + a.lay.gl);
            g *= gl[0];
            u *= gl[1];
        }
        a.h[(size_t)j * a.I + row] = silu_f32(g) * u;
    }
}

template <int FMT>
__global__ __launch_bounds__(256) void k_gemv_down(GemvArgs a) {
    const int j = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int o0 = (blockIdx.x * 4 + wave) * kRowsB;
    const uint8_t* wb = expert_base(a, j);
    if (!wb) {
        if (lane < kRowsB) a.yp[(size_t)j * a.H + o0 + lane] = 0.0f;
        return;
    }
    const uint8_t* data = wb + a.lay.d2;
    const uint8_t* scal = wb + a.lay.s2;
    constexpr int N = Cw<FMT>::n;
    const int nch = a.I / N;
    const float* hj = a.h + (size_t)j * a.I;
    float acc[kRowsB];
#pragma unroll
    for (int r = 0; r < kRowsB; ++r) acc[r] = 0.0f;
    for (int c = lane; c < nch; c += 64) {
        float xv[N];
        load_x<N, false>(hj, c * N, xv);
#pragma unroll
        for (int r = 0; r < kRowsB; ++r) acc[r] += chunk_dot<FMT>(data, scal, o0 + r, a.I, c, xv);
    }
#pragma unroll
    for (int r = 0; r < kRowsB; ++r) acc[r] = wave_sum(acc[r]);
    if (lane < kRowsB) {
        float v = acc[0];
#pragma unroll
        for (int r = 1; r < kRowsB; ++r)
            if (lane == r) v = acc[r];
        const int row = o0 + lane;
        if (FMT == EO_W_FP8) v *= ((const float*)scal)[row];
        else if (FMT == EO_W_NVFP4) v *= ((const float*)(wb + a.lay.gl))[2];
        float wj = j < a.k ? a.w[j] : 1.0f;
        a.yp[(size_t)j * a.H + row] = v * wj;
    }
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_gemv_reduce(const float* __restrict__ yp, int nparts,
                                                     const float* __restrict__ y_host, int H,
                                                     float* __restrict__ y, const void* x_in,
                                                     void* x_res) {
    int o = blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= H) return;
    float s = 0.0f;
    for (int j = 0; j < nparts; ++j) s += yp[(size_t)j * H + o];
    if (y_host) s += y_host[o];
    if (y) y[o] = s;
    if (x_res) {
        if (BF16) {
            const uint16_t* xi = (const uint16_t*)x_in;
            ((uint16_t*)x_res)[o] = (uint16_t)f32_bf16_rne(bf16_f32(xi[o]) + s);
        } else {
            const float* xi = (const float*)x_in;
            ((float*)x_res)[o] = xi[o] + s;
        }
    }
}


// ------------------------------------------------------------------ fast path
// For bf16 activations and the shapes instantiated below: gate/up kernel
// (h written as bf16) then down kernel. Each lane group of G lanes owns R rows
// and NC 16-byte chunks per row; all loads of a wavefront are issued before its
// arithmetic, so each lane keeps R * NC * 16 bytes in flight. bf16 products
// use v_dot2_f32_bf16; fp4 codes become bf16 pairs with the scaled convert
// (MXFP4: times 2^(e8m0-127), exact; NVFP4: unscaled, then the two e4m3 block
// scales on the partial sums).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x2_t as_bf2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

__device__ __forceinline__ float dot8(uint4 w, uint4 x, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(w.x), as_bf2(x.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(w.y), as_bf2(x.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(w.z), as_bf2(x.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(w.w), as_bf2(x.w), acc, false);
    return acc;
}

// 8 fp4 codes of one 32-bit word (two per byte, low nibble first) times x.
template <int B>
__device__ __forceinline__ float fp4_byte(uint32_t w, float sc, uint32_t xw, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(as_bf2(fp4x2_bf16_pow2<B>(w, sc)), as_bf2(xw), acc,
                                           false);
}
__device__ __forceinline__ float fp4_word(uint32_t w, float sc, uint4 x, float acc) {
    acc = fp4_byte<0>(w, sc, x.x, acc);
    acc = fp4_byte<1>(w, sc, x.y, acc);
    acc = fp4_byte<2>(w, sc, x.z, acc);
    acc = fp4_byte<3>(w, sc, x.w, acc);
    return acc;
}

template <int FMT> struct FastC;  // bf16 x elements per chunk, x uint4 per chunk
template <> struct FastC<EO_W_BF16> { static constexpr int n = 8, xq = 1; };
template <> struct FastC<EO_W_FP8> { static constexpr int n = 16, xq = 2; };
template <> struct FastC<EO_W_MXFP4> { static constexpr int n = 32, xq = 4; };
template <> struct FastC<EO_W_NVFP4> { static constexpr int n = 32, xq = 4; };

// A weight chunk: streamed once per call, so the load carries the nontemporal
// hint and does not allocate in the caches (x and the scales stay cached).
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint8_t* p) {
    const u32x4_nt v = __builtin_nontemporal_load((const u32x4_nt*)p);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int FMT>
__device__ __forceinline__ const uint8_t* row_ptr(const uint8_t* data, int row, int K) {
    if (FMT == EO_W_BF16) return data + (size_t)row * K * 2;
    if (FMT == EO_W_FP8) return data + (size_t)row * K;
    return data + (size_t)row * (K / 2);
}

// Partial dots of R weight rows with the bf16 vector x over this lane's chunks
// c = gl + G*i (i < NC); block scales are applied, row/tensor scales are not.
// XC: x is read at device scope (written by other workgroups of the same launch).
template <int FMT, int G, int NC, int R, bool XC = false>
__device__ __forceinline__ void rows_dot(const uint8_t* data, const uint8_t* scal, int K,
                                         const int (&rows)[R], const uint16_t* x, int gl,
                                         float (&out)[R]) {
    constexpr int XQ = FastC<FMT>::xq, N = FastC<FMT>::n;
    uint4 wq[R][NC];
    uint4 xq[NC][XQ];
    uint32_t sq[R][NC];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < NC; ++i)
            wq[r][i] = load_stream(row_ptr<FMT>(data, rows[r], K) + (size_t)(gl + G * i) * 16);
#pragma unroll
    for (int i = 0; i < NC; ++i)
#pragma unroll
        for (int q = 0; q < XQ; ++q) {
            const uint16_t* px = x + (size_t)(gl + G * i) * N + 8 * q;
            if (XC) {
                const uint32_t* p32 = (const uint32_t*)px;
                xq[i][q] = make_uint4(__hip_atomic_load(p32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                                      __hip_atomic_load(p32 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                                      __hip_atomic_load(p32 + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                                      __hip_atomic_load(p32 + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            } else {
                xq[i][q] = *(const uint4*)px;
            }
        }
    if (FMT == EO_W_MXFP4 || FMT == EO_W_NVFP4) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                const int c = gl + G * i;
                if (FMT == EO_W_MXFP4)
                    sq[r][i] = scal[(size_t)rows[r] * (K / 32) + c];
                else
                    sq[r][i] = *(const uint16_t*)(scal + (size_t)rows[r] * (K / 16) + 2 * c);
            }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const uint4 w = wq[r][i];
            if (FMT == EO_W_BF16) {
                acc = dot8(w, xq[i][0], acc);
            } else if (FMT == EO_W_FP8) {
                acc = dot8(make_uint4(e4m3x2_bf16(w.x), e4m3x2_bf16(w.x >> 16),
                                      e4m3x2_bf16(w.y), e4m3x2_bf16(w.y >> 16)), xq[i][0], acc);
                acc = dot8(make_uint4(e4m3x2_bf16(w.z), e4m3x2_bf16(w.z >> 16),
                                      e4m3x2_bf16(w.w), e4m3x2_bf16(w.w >> 16)), xq[i][1], acc);
            } else if (FMT == EO_W_MXFP4) {
                const float sc = e8m0_f32(sq[r][i]);
                acc = fp4_word(w.x, sc, xq[i][0], acc);
                acc = fp4_word(w.y, sc, xq[i][1], acc);
                acc = fp4_word(w.z, sc, xq[i][2], acc);
                acc = fp4_word(w.w, sc, xq[i][3], acc);
            } else {  // NVFP4: exact e2m1 values, then the two e4m3 block scales
                float a0 = fp4_word(w.x, 1.0f, xq[i][0], 0.0f);
                a0 = fp4_word(w.y, 1.0f, xq[i][1], a0);
                float a1 = fp4_word(w.z, 1.0f, xq[i][2], 0.0f);
                a1 = fp4_word(w.w, 1.0f, xq[i][3], a1);
                acc = fmaf(a0, e4m3_f32(sq[r][i] & 0xFF), acc);
                acc = fmaf(a1, e4m3_f32(sq[r][i] >> 8), acc);
            }
        }
        out[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int s = G / 2; s >= 1; s >>= 1) out[r] += __shfl_xor(out[r], s, 64);
}

// Gate/up rows of workgroup `bidx`: expert slot bidx / nA_per, row block bidx % nA_per.
// HC: h is stored at device scope (read by other workgroups of the same launch).
template <int FMT, int GA, int NCA, int RA, bool HC = false>
__device__ __forceinline__ void gu_body(const GemvArgs& a, uint16_t* __restrict__ hb, int nA_per,
                                        int bidx) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = bidx / nA_per, blk = bidx % nA_per;
    const uint8_t* wb = expert_base(a, j);
    if (!wb) return;
    const int grp = lane / GA, gl = lane % GA;
    const int r0 = ((blk * 4 + wave) * (64 / GA) + grp) * RA;
    int rows[2 * RA];
#pragma unroll
    for (int r = 0; r < RA; ++r) {
        rows[r] = r0 + r;
        rows[RA + r] = a.I + r0 + r;
    }
    float out[2 * RA];
    rows_dot<FMT, GA, NCA, 2 * RA>(wb + a.lay.d13, wb + a.lay.s13, a.H, rows, (const uint16_t*)a.x,
                                   gl, out);
    if (gl == 0) {
        float sg = 1.0f, su = 1.0f;
        const float* rs = (const float*)(wb + a.lay.s13);
        if (FMT == EO_W_NVFP4) {
            const float* g = (const float*)(wb + a.lay.gl);
            sg = g[0];
            su = g[1];
        }
#pragma unroll
        for (int r = 0; r < RA; ++r) {
            float g = out[r] * (FMT == EO_W_FP8 ? rs[r0 + r] : sg);
            float u = out[RA + r] * (FMT == EO_W_FP8 ? rs[a.I + r0 + r] : su);
            const uint16_t hv = (uint16_t)f32_bf16_rne(silu_f32(g) * u);
            if (HC)
                __hip_atomic_store(hb + (size_t)j * a.I + r0 + r, hv, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            else
                hb[(size_t)j * a.I + r0 + r] = hv;
        }
    }
}

template <int FMT, int GA, int NCA, int RA>
__global__ __launch_bounds__(256) void k_gemv_gu(GemvArgs a, uint16_t* __restrict__ hb, int nA_per) {
    gu_body<FMT, GA, NCA, RA>(a, hb, nA_per, blockIdx.x);
}

// Down rows of workgroup `bidx`: expert slot bidx / nB_per, row block bidx % nB_per.
// XC: h is read at device scope.
template <int FMT, int GB, int NCB, int RB, bool XC = false>
__device__ __forceinline__ void dn_body(const GemvArgs& a, const uint16_t* __restrict__ hb,
                                        int nB_per, int bidx) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = bidx / nB_per, blk = bidx % nB_per;
    const int grp = lane / GB, gl = lane % GB;
    const int o0 = ((blk * 4 + wave) * (64 / GB) + grp) * RB;
    const uint8_t* wb = expert_base(a, j);
    if (!wb) {
        if (gl == 0)
#pragma unroll
            for (int r = 0; r < RB; ++r) a.yp[(size_t)j * a.H + o0 + r] = 0.0f;
        return;
    }
    int rows[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) rows[r] = o0 + r;
    float out[RB];
    rows_dot<FMT, GB, NCB, RB, XC>(wb + a.lay.d2, wb + a.lay.s2, a.I, rows, hb + (size_t)j * a.I,
                                   gl, out);
    if (gl == 0) {
        const float wj = a.ex.valid ? a.ex.w[j] : (j < a.k ? a.w[j] : 1.0f);
        const float* rs = (const float*)(wb + a.lay.s2);
        const float gs = FMT == EO_W_NVFP4 ? ((const float*)(wb + a.lay.gl))[2] : 1.0f;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            float v = out[r] * (FMT == EO_W_FP8 ? rs[o0 + r] : gs);
            a.yp[(size_t)j * a.H + o0 + r] = v * wj;
        }
    }
}

// Gate/up workgroups of each hit expert slot of a layer call with fills are
// counted on kSub counters, one 128-byte line apiece (workgroup blk on counter
// blk % kSub); the one that completes a counter counts it on the slot's total.
constexpr int kSub = 64;
struct DownSync {
    uint32_t* sub;   // [nexp][kSub] x 32 words
    uint32_t* done;  // [nexp] x 32 words: counters complete
};
__host__ __device__ constexpr size_t down_sync_words() { return (size_t)(kMaxK + 1) * (kSub + 1) * 32; }

// Whether expert slot j of a one-token plan is a hit (resident before this
// call: not filled, not host-executed); the shared expert counts as one.
__device__ __forceinline__ bool slot_hit(const GemvArgs& a, int j) {
    const DevPlan* p = a.plan;
    if (j == a.k) return a.gw.shared_w != nullptr;
    if (p->pad != 0) return false;
    const int sl = p->tok_slot[j];
    bool filled = false;
    for (int r = 0; r < p->q_fill; ++r) filled |= p->fill_slot[r] == sl;
    return sl >= 0 && !filled;
}

// ds != null (behind the fill + GEMV launch): on a layer call with fills the
// hit slots' rows were done by that launch, so their workgroups leave at once,
// and workgroup 0 clears its counters for the next launch.
template <int FMT, int GB, int NCB, int RB>
__global__ __launch_bounds__(256) void k_gemv_dn(GemvArgs a, const uint16_t* __restrict__ hb,
                                                 int nB_per, DownSync ds) {
    if (ds.sub && a.plan->pad == 0 && a.plan->q_fill > 0) {
        if (blockIdx.x == 0)
            for (int i = threadIdx.x; i < a.nexp * (kSub + 1); i += 256)
                (i < a.nexp * kSub ? ds.sub[i * 32] : ds.done[(i - a.nexp * kSub) * 32]) = 0;
        if (slot_hit(a, blockIdx.x / nB_per)) return;
    }
    dn_body<FMT, GB, NCB, RB>(a, hb, nB_per, blockIdx.x);
}

// The fills of a one-token call, the gate/up rows and the hit slots' down rows
// in one launch.
struct FillSync {
    const uint8_t* pool;  // the layer's pinned pool, device-visible
    uint8_t* slots;       // the cache slots the fills write (the GEMV's gw.slots)
    uint64_t S_pad;
    uint32_t* ready;  // [kMaxK]: fill workgroups done with the r-th fill's gate/up bytes
    int32_t* err;     // set when a wait for the fills runs out
    uint64_t wait_ticks;  // longest wait, in ticks of the device's 100 MHz wall clock
    DownSync down;        // counters of the hit slots' gate/up rows (zero between launches)
};

// Rank among this call's fills of a one-token plan's expert slot j, or -1.
__device__ __forceinline__ int fill_rank(const DevPlan* p, int j, int k) {
    if (j >= k || p->pad != 0) return -1;
    const int sl = p->tok_slot[j];
    int rank = -1;
    for (int r = 0; r < p->q_fill; ++r)
        if (p->fill_slot[r] == sl) rank = r;
    return sl >= 0 ? rank : -1;
}

// Workgroups [0, kFillBlocks) copy the fills as the fill kernel does, in two
// passes: first, for each filled expert, the bytes gate/up reads (its weights,
// their scales and the global scales), released at device scope (the counter's
// increment carries the release: the L2 lines written are written back) and
// counted; then the down projection's bytes, which the next launch reads. The
// next nexp * nA_per workgroups run gate/up; those of a filled expert first
// wait for its counter to reach kFillBlocks (lower workgroup ids, dispatched
// first: the wait ends), then acquire at device scope before they read the
// slot, while the fill workgroups copy the down rows. On a layer call with
// fills, the hit slots' gate/up workgroups store h at device scope and count
// themselves, and the last nexp * nB_per workgroups run those slots' down rows
// once their counts are complete (one polling thread per workgroup, reading h
// at device scope), so that only the filled experts' down rows are left to the
// down kernel behind this launch.
template <int FMT, int GA, int NCA, int RA, int GB, int NCB, int RB>
__global__ __launch_bounds__(256) void k_fill_gu(GemvArgs a, uint16_t* __restrict__ hb, int nA_per,
                                                 int nB_per, FillSync f, DownSync ds) {
    if ((int)blockIdx.x < kFillBlocks) {
        const DevPlan* p = a.plan;
        const int q = p->pad == 0 ? p->q_fill : 0;
        const Layout& L = a.lay;
        const int part = blockIdx.x;
        for (int r = 0; r < q; ++r) {
            const uint8_t* src = f.pool + (uint64_t)p->fill_e[r] * f.S_pad;
            uint8_t* dst = f.slots + (uint64_t)p->fill_slot[r] * f.S_pad;
            copy_block<true>(src + L.d13, dst + L.d13, L.d2 - L.d13, part, kFillBlocks);
            copy_block<true>(src + L.s13, dst + L.s13, L.s2 - L.s13, part, kFillBlocks);
            copy_block<true>(src + L.gl, dst + L.gl, L.bytes - L.gl, part, kFillBlocks);
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's stores have completed
            __syncthreads();
            if (threadIdx.x == 0)
                __hip_atomic_fetch_add(&f.ready[r], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
        for (int r = 0; r < q; ++r) {
            const uint8_t* src = f.pool + (uint64_t)p->fill_e[r] * f.S_pad;
            uint8_t* dst = f.slots + (uint64_t)p->fill_slot[r] * f.S_pad;
            copy_block<true>(src + L.d2, dst + L.d2, L.s13 - L.d2, part, kFillBlocks);
            copy_block<true>(src + L.s2, dst + L.s2, L.gl - L.s2, part, kFillBlocks);
        }
        return;
    }
    const int q = a.plan->pad == 0 ? a.plan->q_fill : 0;
    const int nGU = a.nexp * nA_per;
    if ((int)blockIdx.x >= kFillBlocks + nGU) {  // down rows of a hit slot
        const int bidx = blockIdx.x - kFillBlocks - nGU, j = bidx / nB_per;
        if (q == 0 || !slot_hit(a, j)) return;  // the down kernel does these rows
        if (threadIdx.x == 0) {
            const uint32_t nsub = (uint32_t)min(kSub, nA_per);
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            while (__hip_atomic_load(&ds.done[j * 32], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                   nsub) {
                if (__builtin_amdgcn_s_memrealtime() - t0 > f.wait_ticks) {
                    __hip_atomic_store(f.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(32);
            }
        }
        __syncthreads();
        dn_body<FMT, GB, NCB, RB, true>(a, hb, nB_per, bidx);
        return;
    }
    const int bidx = blockIdx.x - kFillBlocks;
    const int j = bidx / nA_per;
    if (q > 0 && slot_hit(a, j)) {  // workgroup-uniform
        gu_body<FMT, GA, NCA, RA, true>(a, hb, nA_per, bidx);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's h stores have completed
        __syncthreads();
        if (threadIdx.x == 0) {
            const int blk = bidx % nA_per, sub = blk % kSub;
            const uint32_t per = (uint32_t)((nA_per - sub + kSub - 1) / kSub);
            if (__hip_atomic_fetch_add(&ds.sub[(j * kSub + sub) * 32], 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT) + 1 == per)
                __hip_atomic_fetch_add(&ds.done[j * 32], 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }
    const int r = fill_rank(a.plan, j, a.k);  // workgroup-uniform
    if (r >= 0) {
        if (threadIdx.x == 0) {
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            while (__hip_atomic_load(&f.ready[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                   (uint32_t)kFillBlocks) {
                if (__builtin_amdgcn_s_memrealtime() - t0 > f.wait_ticks) {
                    __hip_atomic_store(f.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(16);
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
    }
    gu_body<FMT, GA, NCA, RA>(a, hb, nA_per, bidx);
}


// Lanes per row G and chunks per lane NC for a row of `nch` chunks.
bool split_rows(int nch, int* G, int* NC) {
    for (int g = 64; g >= 4; g >>= 1)
        if (nch % g == 0) {
            *G = g;
            *NC = nch / g;
            return true;
        }
    return false;
}

template <int FMT, int GA, int NCA, int RA, int GB, int NCB, int RB>
hipError_t run_fast(const GemvArgs& a, uint16_t* hb, hipStream_t s, hipEvent_t* ev,
                    const FillSync* fill) {
    const int rowsA = 4 * (64 / GA) * RA, rowsB = 4 * (64 / GB) * RB;
    if (a.I % rowsA || a.H % rowsB) return hipErrorNotSupported;
    const int nA_per = a.I / rowsA, nB_per = a.H / rowsB;
    const DownSync ds = fill ? fill->down : DownSync{nullptr, nullptr};
    if (fill)
        hipExtLaunchKernelGGL((k_fill_gu<FMT, GA, NCA, RA, GB, NCB, RB>),
                              dim3(kFillBlocks + a.nexp * (nA_per + nB_per)), dim3(256), 0, s,
                              ev[0], ev[1], 0, a, hb, nA_per, nB_per, *fill, ds);
    else
        hipExtLaunchKernelGGL(k_gemv_gu<FMT, GA, NCA, RA>, dim3(a.nexp * nA_per), dim3(256), 0, s,
                              ev[0], ev[1], 0, a, hb, nA_per);
    hipExtLaunchKernelGGL(k_gemv_dn<FMT, GB, NCB, RB>, dim3(a.nexp * nB_per), dim3(256), 0, s,
                          ev[2], ev[3], 0, a, (const uint16_t*)hb, nB_per, ds);
    return hipGetLastError();
}

// Shapes with a tuned instantiation: (GA, NCA) from H, (GB, NCB) from I.
template <int FMT>
hipError_t fast_dispatch(const GemvArgs& a, uint16_t* hb, hipStream_t s, hipEvent_t* ev,
                         const FillSync* fill = nullptr) {
    constexpr int N = FastC<FMT>::n;
    int GA, NCA, GB, NCB;
    if (a.H % N || a.I % N || !split_rows(a.H / N, &GA, &NCA) || !split_rows(a.I / N, &GB, &NCB))
        return hipErrorNotSupported;
#define EO_FAST(ga, nca, ra, gb, ncb, rb)                         \
    if (GA == ga && NCA == nca && GB == gb && NCB == ncb)         \
        return run_fast<FMT, ga, nca, ra, gb, ncb, rb>(a, hb, s, ev, fill);
    EO_FAST(64, 4, 1, 32, 3, 1)  // bf16 H 2048, I 768
    EO_FAST(64, 1, 4, 32, 1, 4)  // bf16 H 512, I 256
    EO_FAST(32, 1, 4, 16, 1, 4)  // fp8 H 512, I 256
    EO_FAST(64, 2, 4, 64, 1, 4)  // fp4 H 4096, I 2048
    EO_FAST(64, 3, 2, 64, 1, 4)  // fp4 H 6144, I 2048
    EO_FAST(16, 1, 4, 8, 1, 4)   // fp4 H 512, I 256
    EO_FAST(64, 2, 2, 32, 3, 2)  // fp8 H 2048, I 768
    EO_FAST(64, 1, 4, 8, 3, 4)   // fp4 H 2048, I 768
#undef EO_FAST
    return hipErrorNotSupported;
}

template <int FMT, bool XBF16>
void run(const GemvArgs& a, hipStream_t s, hipEvent_t* ev) {
    hipExtLaunchKernelGGL(k_gemv_up<FMT, XBF16>, dim3(a.I / (4 * kRowsA), a.nexp), dim3(256), 0,
                          s, ev[0], ev[1], 0, a);
    hipExtLaunchKernelGGL(k_gemv_down<FMT>, dim3(a.H / (4 * kRowsB), a.nexp), dim3(256), 0, s,
                          ev[2], ev[3], 0, a);
}

}  // namespace

hipError_t launch_ffn_gemv(int fmt, const Layout& lay, GroupW gw, const DevPlan* plan,
                           const int32_t* ids, const float* w, int k, int E, int has_shared,
                           int H, int I, const void* x, int act_bf16, float* h_buf,
                           float* y_parts, hipStream_t s, hipEvent_t* ev, int allow_fast,
                           const GemvExperts* ex) {
    GemvArgs a{};
    a.gw = gw;
    a.lay = lay;
    a.plan = plan;
    a.ids = ids;
    a.w = w;
    a.k = k;
    a.E = E;
    a.H = H;
    a.I = I;
    a.nexp = k + (has_shared ? 1 : 0);
    a.x = x;
    a.h = h_buf;
    a.yp = y_parts;
    if (ex) a.ex = *ex;
    if (allow_fast && act_bf16 && fmt != EO_W_FP32) {
        hipError_t he = hipErrorNotSupported;
        uint16_t* hb = (uint16_t*)h_buf;
        switch (fmt) {
        case EO_W_BF16: he = fast_dispatch<EO_W_BF16>(a, hb, s, ev); break;
        case EO_W_FP8: he = fast_dispatch<EO_W_FP8>(a, hb, s, ev); break;
        case EO_W_MXFP4: he = fast_dispatch<EO_W_MXFP4>(a, hb, s, ev); break;
        case EO_W_NVFP4: he = fast_dispatch<EO_W_NVFP4>(a, hb, s, ev); break;
        default: break;
        }
        if (he != hipErrorNotSupported) return he;
    }
    if (fmt == EO_W_FP32) {
        if (act_bf16) return hipErrorInvalidValue;
        run<EO_W_FP32, false>(a, s, ev);
    } else {
        if (!act_bf16) return hipErrorInvalidValue;
        switch (fmt) {
        case EO_W_BF16: run<EO_W_BF16, true>(a, s, ev); break;
        case EO_W_FP8: run<EO_W_FP8, true>(a, s, ev); break;
        case EO_W_MXFP4: run<EO_W_MXFP4, true>(a, s, ev); break;
        case EO_W_NVFP4: run<EO_W_NVFP4, true>(a, s, ev); break;
        default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

size_t fill_gemv_counter_bytes() { return sizeof(uint32_t) * down_sync_words(); }

hipError_t launch_fill_gemv(int fmt, const Layout& lay, GroupW gw, uint8_t* slots,
                            const DevPlan* plan, const uint8_t* pool_layer_dev, uint64_t S,
                            uint64_t S_pad,
                            const int32_t* ids, const float* w, int k, int E, int has_shared,
                            int H, int I, const void* x, int act_bf16, float* h_buf,
                            float* y_parts, DevState* st, uint32_t* counters,
                            uint64_t wait_ticks, hipStream_t s) {
    if (!act_bf16) return hipErrorNotSupported;
    GemvArgs a{};
    a.gw = gw;
    a.lay = lay;
    a.plan = plan;
    a.ids = ids;
    a.w = w;
    a.k = k;
    a.E = E;
    a.H = H;
    a.I = I;
    a.nexp = k + (has_shared ? 1 : 0);
    a.x = x;
    a.h = h_buf;
    a.yp = y_parts;
    if (slots != gw.slots) return hipErrorInvalidValue;
    if (lay.bytes != S) return hipErrorInvalidValue;
    if (!counters) return hipErrorInvalidValue;
    const DownSync ds{counters, counters + (size_t)(kMaxK + 1) * kSub * 32};
    const FillSync f{pool_layer_dev, slots, S_pad, st->fill_ready, &st->sync_err, wait_ticks, ds};
    uint16_t* hb = (uint16_t*)h_buf;
    hipEvent_t none[4] = {nullptr, nullptr, nullptr, nullptr};
    switch (fmt) {
    case EO_W_BF16: return fast_dispatch<EO_W_BF16>(a, hb, s, none, &f);
    case EO_W_FP8: return fast_dispatch<EO_W_FP8>(a, hb, s, none, &f);
    case EO_W_MXFP4: return fast_dispatch<EO_W_MXFP4>(a, hb, s, none, &f);
    case EO_W_NVFP4: return fast_dispatch<EO_W_NVFP4>(a, hb, s, none, &f);
    default: return hipErrorNotSupported;
    }
}

hipError_t launch_gemv_reduce(const float* y_parts, int nparts, const float* y_host, int H,
                              float* y, void* x_res, int act_bf16, hipStream_t s,
                              const void* x_in) {
    if (!x_in) x_in = x_res;
    if (act_bf16)
        k_gemv_reduce<true><<<(H + 255) / 256, 256, 0, s>>>(y_parts, nparts, y_host, H, y, x_in,
                                                            x_res);
    else
        k_gemv_reduce<false><<<(H + 255) / 256, 256, 0, s>>>(y_parts, nparts, y_host, H, y, x_in,
                                                             x_res);
    return hipGetLastError();
}

}  // namespace eo
