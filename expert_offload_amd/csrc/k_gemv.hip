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
#include "dev_common.h"
#include "eo_internal.h"

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
    if (j == a.k) return a.gw.shared_w;
    int e = a.ids[j];
    if (e < 0 || e >= a.E) return nullptr;
    int s = a.plan->e2slot[e];
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
                                                     float* __restrict__ y, void* __restrict__ x_res) {
    int o = blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= H) return;
    float s = 0.0f;
    for (int j = 0; j < nparts; ++j) s += yp[(size_t)j * H + o];
    if (y_host) s += y_host[o];
    if (y) y[o] = s;
    if (x_res) {
        if (BF16) {
            uint16_t* xp = (uint16_t*)x_res;
            xp[o] = (uint16_t)f32_bf16_rne(bf16_f32(xp[o]) + s);
        } else {
            float* xp = (float*)x_res;
            xp[o] = xp[o] + s;
        }
    }
}

template <int FMT, bool XBF16>
void run(const GemvArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (ev0) (void)hipEventRecord(ev0, s);
    k_gemv_up<FMT, XBF16><<<dim3(a.I / (4 * kRowsA), a.nexp), 256, 0, s>>>(a);
    k_gemv_down<FMT><<<dim3(a.H / (4 * kRowsB), a.nexp), 256, 0, s>>>(a);
    if (ev1) (void)hipEventRecord(ev1, s);
}

}  // namespace

hipError_t launch_ffn_gemv(int fmt, const Layout& lay, GroupW gw, const DevPlan* plan,
                           const int32_t* ids, const float* w, int k, int E, int has_shared,
                           int H, int I, const void* x, int act_bf16, float* h_buf,
                           float* y_parts, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
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
    if (fmt == EO_W_FP32) {
        if (act_bf16) return hipErrorInvalidValue;
        run<EO_W_FP32, false>(a, s, ev0, ev1);
    } else {
        if (!act_bf16) return hipErrorInvalidValue;
        switch (fmt) {
        case EO_W_BF16: run<EO_W_BF16, true>(a, s, ev0, ev1); break;
        case EO_W_FP8: run<EO_W_FP8, true>(a, s, ev0, ev1); break;
        case EO_W_MXFP4: run<EO_W_MXFP4, true>(a, s, ev0, ev1); break;
        case EO_W_NVFP4: run<EO_W_NVFP4, true>(a, s, ev0, ev1); break;
        default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

hipError_t launch_gemv_reduce(const float* y_parts, int nparts, const float* y_host, int H,
                              float* y, void* x_res, int act_bf16, hipStream_t s) {
    if (act_bf16)
        k_gemv_reduce<true><<<(H + 255) / 256, 256, 0, s>>>(y_parts, nparts, y_host, H, y, x_res);
    else
        k_gemv_reduce<false><<<(H + 255) / 256, 256, 0, s>>>(y_parts, nparts, y_host, H, y, x_res);
    return hipGetLastError();
}

}  // namespace eo
