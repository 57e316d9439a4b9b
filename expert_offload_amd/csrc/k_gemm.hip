// Grouped SwiGLU expert FFN for many tokens (prefill, and any call with T > 1).
//
// Per expert e with its M_e grouped rows X_e (bf16; each row is read from the
// layer input through perm_pair, so the input is never copied in grouped order):
//   GEMM1: G = X_e . W13^T, h = silu(G_gate) * G_up  -> bf16 [M_e, I]
//   GEMM2: O = h . W2^T, scaled by the pair's routing weight -> o_pairs (bf16;
//          fp32 on the fp32-weight path)
// on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulate). Weight
// tiles are decoded into LDS as bf16: bf16 as stored; e4m3 (FP8) and
// e2m1 * e8m0 (MXFP4) and e2m1 * e4m3 (NVFP4) are exact in bf16, so the only
// factors left over — the FP8 per-row scale and the NVFP4 per-tensor global
// scale — are applied to the fp32 accumulators in the epilogue. The format
// list is the juejin.cn overview's (section 5).
//
// Five kernels share the grouping (128-row tiles per group from tile_off) and
// the GEMM1 split (each wavefront holds matching gate and up accumulators and
// forms h in registers):
//   v5 (bf16, the default): 128 x 256 tiles, two workgroups per CU, direct-to-
//      LDS rings of two slots for each operand, the weight tile in 128-byte
//      rows (K step 64), the activation tile in 64-byte rows (K step 32);
//   v4 (bf16, on request): the same tiles with one three-stage ring of K-32
//      tiles for both operands;
//   v4q (FP8 / MXFP4 / NVFP4, the default): v4's ring for the activation tile,
//      with each weight row's next 64-byte span of codes in registers, decoded
//      into the ring one tile per step between the two halves of its MFMAs;
//   v3 (any format, on request): the same tiles with the next K tile staged
//      through registers, where fp4/fp8 codes are decoded;
//   k_gemm_mfma: plain 128 x 128 tiles, K step 64 (the reference form).
// EO_GEMM_PATH selects among them for tests. fp32 weights with fp32 activations
// (small test models) use a plain VALU kernel with the same grouping and
// epilogues.
#include <hip/hip_ext.h>

#include <cstdlib>
#include <type_traits>

#include "decode_dev.h"
#include "dev_common.h"
#include "eo_internal.h"

namespace eo {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;  // LDS row stride in bf16

// 3: v5 for bf16, v4q for fp8 / fp4; 2: the one-ring kernels (v4 for bf16,
// v4q for fp8 / fp4); 1: v3 for all; 0: the plain 128 x 128 kernel.
// EO_GEMM_PATH overrides.
int g_gemm_tiles = 3;

struct GemmArgs {
    GroupW gw;
    Layout lay;
    int E, G, K;  // G = groups incl. shared; K = contraction length
    int H, I;
    const int32_t* offsets;
    const int32_t* tile_off;
    const uint16_t* A;    // GEMM1: layer input [T, H]; GEMM2: h [rows, I]
    uint16_t* h_out;      // GEMM1 output [rows, I] bf16
    const int32_t* perm_pair;
    const float* w;
    int Tk, k;
    void* o_pairs;        // GEMM2 output [Tk + T, H]: bf16 (MFMA path) or fp32
};

// Row of A that grouped row r multiplies. GEMM1 reads the layer input row of the
// token of r's (token, slot) pair, or of the token itself for a shared-expert
// row, so no permuted copy of the input is made; GEMM2 reads row r of h.
template <int MODE>
__device__ __forceinline__ int a_row(const GemmArgs& a, int r) {
    if (MODE == 1) return r;
    const int pair = a.perm_pair[r];
    return pair < a.Tk ? pair / a.k : pair - a.Tk;
}

__device__ __forceinline__ int find_group(const int32_t* tile_off, int G, int tile) {
    int lo = 0, hi = G;  // tile_off[lo] <= tile < tile_off[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (tile_off[mid] <= tile) lo = mid; else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ const uint8_t* group_base(const GroupW& gw, int g, int E) {
    if (g == E) return gw.shared_w;
    if (gw.gbase) return gw.gbase[g];
    int s = gw.e2slot ? gw.e2slot[g] : g;
    return gw.slots + (uint64_t)s * gw.stride;
}

// Decode 32 fp4 codes (16 bytes) with per-16 multipliers sc0 (elements 0..15)
// and sc1 (16..31) into 32 bf16 at dst.
template <int FMT>
__device__ __forceinline__ void fp4x32_to_lds(uint4 q, float sc0, float sc1, uint16_t* dst) {
    const uint32_t words[4] = {q.x, q.y, q.z, q.w};
    uint32_t out[16];
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
        const float sc = wi < 2 ? sc0 : sc1;
        out[wi * 4 + 0] = fp4x2_bf16<FMT, 0>(words[wi], sc);
        out[wi * 4 + 1] = fp4x2_bf16<FMT, 1>(words[wi], sc);
        out[wi * 4 + 2] = fp4x2_bf16<FMT, 2>(words[wi], sc);
        out[wi * 4 + 3] = fp4x2_bf16<FMT, 3>(words[wi], sc);
    }
    uint4* d = (uint4*)dst;
    d[0] = make_uint4(out[0], out[1], out[2], out[3]);
    d[1] = make_uint4(out[4], out[5], out[6], out[7]);
    d[2] = make_uint4(out[8], out[9], out[10], out[11]);
    d[3] = make_uint4(out[12], out[13], out[14], out[15]);
}

template <int FMT, int MODE>
__global__ __launch_bounds__(256) void k_gemm_mfma(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDK];

    const int tile = blockIdx.x;
    if (tile >= a.tile_off[a.G]) return;
    const int g = find_group(a.tile_off, a.G, tile);
    const int m0 = a.offsets[g] + (tile - a.tile_off[g]) * BM;
    const int m_end = a.offsets[g + 1];
    const uint8_t* wb = group_base(a.gw, g, a.E);
    const int K = a.K;
    const uint8_t* wdata = wb + (MODE == 0 ? a.lay.d13 : a.lay.d2);
    const uint8_t* wscal = wb + (MODE == 0 ? a.lay.s13 : a.lay.s2);
    const int n0 = blockIdx.y * (MODE == 0 ? 64 : 128);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    auto wrow = [&](int i) -> int {  // LDS B row -> weight row
        if (MODE == 0) return i < 64 ? n0 + i : a.I + n0 + (i - 64);
        return n0 + i;
    };

    for (int k0 = 0; k0 < K; k0 += BK) {
        // A tile: 128 rows x 64 bf16, 4 x 16 B per thread
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            int c = tid + 256 * it, r = c >> 3, seg = c & 7;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (m0 + r < m_end)
                v = *(const uint4*)(a.A + (size_t)a_row<MODE>(a, m0 + r) * K + k0 + seg * 8);
            *(uint4*)(As + r * LDK + seg * 8) = v;
        }
        // B tile: 128 weight rows x 64 elements, decoded to bf16
        if (FMT == EO_W_BF16) {
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                int c = tid + 256 * it, r = c >> 3, seg = c & 7;
                const uint16_t* src = (const uint16_t*)wdata + (size_t)wrow(r) * K + k0 + seg * 8;
                *(uint4*)(Bs + r * LDK + seg * 8) = *(const uint4*)src;
            }
        } else if (FMT == EO_W_FP8) {
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                int c = tid + 256 * it, r = c >> 2, seg = c & 3;
                uint4 q = *(const uint4*)(wdata + (size_t)wrow(r) * K + k0 + seg * 16);
                uint32_t words[4] = {q.x, q.y, q.z, q.w}, out[8];
#pragma unroll
                for (int wi = 0; wi < 4; ++wi) fp8x4_bf16(words[wi], out[2 * wi], out[2 * wi + 1]);
                uint4* d = (uint4*)(Bs + r * LDK + seg * 16);
                d[0] = make_uint4(out[0], out[1], out[2], out[3]);
                d[1] = make_uint4(out[4], out[5], out[6], out[7]);
            }
        } else {  // MXFP4 / NVFP4: one 32-element chunk per thread
            int r = tid >> 1, half = tid & 1;
            int wr = wrow(r);
            int kk = k0 + half * 32;
            uint4 q = *(const uint4*)(wdata + (size_t)wr * (K / 2) + kk / 2);
            float sc0, sc1;
            if (FMT == EO_W_MXFP4) {
                sc0 = sc1 = e8m0_f32(wscal[(size_t)wr * (K / 32) + kk / 32]);
            } else {
                const uint8_t* sp = wscal + (size_t)wr * (K / 16) + kk / 16;
                sc0 = e4m3_f32(sp[0]);
                sc1 = e4m3_f32(sp[1]);
            }
            fp4x32_to_lds<FMT>(q, sc0, sc1, Bs + r * LDK + half * 32);
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int kc = ks * 16 + (lane >> 5) * 8;
            bf16x8 av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                av[i] = *(const bf16x8*)(As + (wm * 64 + i * 32 + (lane & 31)) * LDK + kc);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                int br = MODE == 0 ? (j * 64 + wn * 32 + (lane & 31)) : (wn * 64 + j * 32 + (lane & 31));
                bv[j] = *(const bf16x8*)(Bs + br * LDK + kc);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // epilogue
    const int col = lane & 31;
    if (MODE == 0) {
        const int n = n0 + wn * 32 + col;
        float sg = 1.0f, su = 1.0f;
        if (FMT == EO_W_FP8) {
            sg = ((const float*)wscal)[n];
            su = ((const float*)wscal)[a.I + n];
        } else if (FMT == EO_W_NVFP4) {
            const float* gl = (const float*)(wb + a.lay.gl);
            sg = gl[0];
            su = gl[1];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                int row = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (m0 + row < m_end) {
                    float gv = acc[i][0][v] * sg, uv = acc[i][1][v] * su;
                    float hv = silu_f32(gv) * uv;
                    a.h_out[(size_t)(m0 + row) * a.I + n] = (uint16_t)f32_bf16_rne(hv);
                }
            }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 64 + j * 32 + col;
            float sc = 1.0f;
            if (FMT == EO_W_FP8) sc = ((const float*)wscal)[n];
            else if (FMT == EO_W_NVFP4) sc = ((const float*)(wb + a.lay.gl))[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    int row = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    if (m0 + row < m_end) {
                        int pair = a.perm_pair[m0 + row];
                        float wp = pair < a.Tk ? a.w[pair] : 1.0f;
                        ((uint16_t*)a.o_pairs)[(size_t)pair * a.H + n] =
                            (uint16_t)f32_bf16_rne(acc[i][j][v] * sc * wp);
                    }
                }
        }
    }
}

// fp32 weights and activations: 128 x 64 tile, 8 x 4 outputs per thread.
template <int MODE>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmArgs a, const float* __restrict__ Af,
                                                  float* __restrict__ hf) {
    constexpr int TBM = 128, TBN = 64, TBK = 16;
    __shared__ float As[TBK][TBM + 4];
    __shared__ float Bs[TBK][TBN + 4];
    const int tile = blockIdx.x;
    if (tile >= a.tile_off[a.G]) return;
    const int g = find_group(a.tile_off, a.G, tile);
    const int m0 = a.offsets[g] + (tile - a.tile_off[g]) * TBM;
    const int m_end = a.offsets[g + 1];
    const uint8_t* wb = group_base(a.gw, g, a.E);
    const float* W = (const float*)(wb + (MODE == 0 ? a.lay.d13 : a.lay.d2));
    const int K = a.K;
    const int n0 = blockIdx.y * (MODE == 0 ? 32 : 64);
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    float acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
    for (int k0 = 0; k0 < K; k0 += TBK) {
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            int c = tid + 256 * it, r = c >> 4, kk = c & 15;
            As[kk][r] = (m0 + r < m_end) ? Af[(size_t)a_row<MODE>(a, m0 + r) * K + k0 + kk] : 0.0f;
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            int c = tid + 256 * it, r = c >> 4, kk = c & 15;
            int wr = MODE == 0 ? (r < 32 ? n0 + r : a.I + n0 + r - 32) : n0 + r;
            Bs[kk][r] = W[(size_t)wr * K + k0 + kk];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TBK; ++kk) {
            float av[8], bv[4];
#pragma unroll
            for (int i = 0; i < 8; ++i) av[i] = As[kk][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int row = ty + 16 * i;
        if (m0 + row >= m_end) continue;
        if (MODE == 0) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                int n = n0 + tx + 16 * j;
                hf[(size_t)(m0 + row) * a.I + n] = silu_f32(acc[i][j]) * acc[i][j + 2];
            }
        } else {
            int pair = a.perm_pair[m0 + row];
            float wp = pair < a.Tk ? a.w[pair] : 1.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int n = n0 + tx + 16 * j;
                ((float*)a.o_pairs)[(size_t)pair * a.H + n] = acc[i][j] * wp;
            }
        }
    }
}


// ------------------------------------------------------------------ v3 tiles
// 128 (rows) x 256 (weight rows) per workgroup, K step 32; wavefront (wm, wn)
// owns rows wm*64..+64 and 128 weight rows (2 x 4 MFMA 32x32x16 blocks). GEMM1's
// 256 weight rows are 128 gate rows then the same 128 up rows; a wavefront
// takes gate columns wn*64..+64 and the matching up columns, so h = silu(g)*u
// forms in registers. The next K tile's global loads are issued into registers
// before the current tile's MFMAs; LDS is double-buffered (60 KB) with one
// barrier per K step, which leaves room for two workgroups (8 wavefronts) per
// CU. LDS rows are 40 bf16 (80 B): the 16 lanes of each ds_read_b128 quarter
// hit 16 distinct 16-byte bank groups (the tile writes do not: about 13% of the
// LDS activity of the fp4 kernels is bank conflicts). The epilogue goes through LDS: scaled
// bf16 results are written there, then leave as 16-byte row segments; row ->
// pair index and routing weight are staged once per workgroup.
constexpr int V3M = 128, V3N = 256, V3K = 32, V3L = V3K + 8;
constexpr int V3_OUT_LD = V3N + 8;  // epilogue tile row stride (bf16)
constexpr size_t kV3Pipe = 2 * (V3M + V3N) * V3L * sizeof(uint16_t);     // 61,440 B
constexpr size_t kV3Out = (size_t)V3M * V3_OUT_LD * sizeof(uint16_t);     // 67,584 B
constexpr size_t kV3Lds = (kV3Pipe > kV3Out ? kV3Pipe : kV3Out) + 2 * V3M * sizeof(int32_t);

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int FMT>
struct V3Regs {  // one K tile of global data held by a thread
    uint4 a[2];
    uint4 b[FMT == EO_W_BF16 ? 4 : (FMT == EO_W_FP8 ? 2 : 1)];
    uint32_t sc;  // fp4 block scales of this thread's B chunk
    // fp4: the thread's weight row over four K tiles (64 contiguous bytes) and
    // their block scales, loaded together every fourth tile, so one row's
    // 128-byte line is requested twice per 8 tiles instead of 8 times
    u32x4 s0, s1, s2, s3;
    uint32_t ss0, ss1;
};

template <int FMT, int MODE>
__device__ __forceinline__ int v3_wrow(const GemmArgs& a, int n0, int i) {
    if (MODE == 0) return i < 128 ? n0 + i : a.I + n0 + (i - 128);
    return n0 + i;
}

template <int FMT, int MODE>
__device__ __forceinline__ void v3_load(const GemmArgs& a, const uint8_t* wdata,
                                        const uint8_t* wscal, int m0, int m_end, int n0, int k0,
                                        int tid, V3Regs<FMT>& r) {
    const int K = a.K;
#pragma unroll
    for (int it = 0; it < 2; ++it) {  // A: 128 rows x 32 bf16 = 512 chunks
        int c = tid + 256 * it, row = c >> 2, seg = c & 3;
        r.a[it] = (m0 + row < m_end)
                      ? *(const uint4*)(a.A + (size_t)a_row<MODE>(a, m0 + row) * K + k0 + seg * 8)
                      : make_uint4(0, 0, 0, 0);
    }
    if (FMT == EO_W_BF16) {  // B: 256 rows x 32 bf16 = 1024 chunks
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            int c = tid + 256 * it, row = c >> 2, seg = c & 3;
            r.b[it] = *(const uint4*)((const uint16_t*)wdata +
                                      (size_t)v3_wrow<FMT, MODE>(a, n0, row) * K + k0 + seg * 8);
        }
    } else if (FMT == EO_W_FP8) {  // 256 rows x 32 bytes = 512 chunks
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            int c = tid + 256 * it, row = c >> 1, seg = c & 1;
            r.b[it] = *(const uint4*)(wdata + (size_t)v3_wrow<FMT, MODE>(a, n0, row) * K + k0 +
                                      seg * 16);
        }
    } else {  // fp4: 256 rows x 16 bytes = 256 chunks, one per thread (K % 128 == 0)
        const int row = tid, wr = v3_wrow<FMT, MODE>(a, n0, row);
        const int u = (k0 / V3K) & 3;  // this tile's place in the thread's span
        if (u == 0) {
            const u32x4* rp = (const u32x4*)(wdata + (size_t)wr * (K / 2) + k0 / 2);
            r.s0 = rp[0];
            r.s1 = rp[1];
            r.s2 = rp[2];
            r.s3 = rp[3];
            if (FMT == EO_W_MXFP4) {
                r.ss0 = *(const uint32_t*)(wscal + (size_t)wr * (K / 32) + k0 / 32);
            } else {
                const uint2 q = *(const uint2*)(wscal + (size_t)wr * (K / 16) + k0 / 16);
                r.ss0 = q.x;
                r.ss1 = q.y;
            }
        }
        const u32x4 v = u == 0 ? r.s0 : u == 1 ? r.s1 : u == 2 ? r.s2 : r.s3;
        r.b[0] = make_uint4(v[0], v[1], v[2], v[3]);
        if (FMT == EO_W_MXFP4)
            r.sc = (r.ss0 >> (8 * u)) & 0xFFu;
        else
            r.sc = ((u < 2 ? r.ss0 : r.ss1) >> (16 * (u & 1))) & 0xFFFFu;
    }
}

template <int FMT>
__device__ __forceinline__ void v3_store(uint16_t* As, uint16_t* Bs, int tid, const V3Regs<FMT>& r) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        int c = tid + 256 * it, row = c >> 2, seg = c & 3;
        *(uint4*)(As + row * V3L + seg * 8) = r.a[it];
    }
    if (FMT == EO_W_BF16) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            int c = tid + 256 * it, row = c >> 2, seg = c & 3;
            *(uint4*)(Bs + row * V3L + seg * 8) = r.b[it];
        }
    } else if (FMT == EO_W_FP8) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            int c = tid + 256 * it, row = c >> 1, seg = c & 1;
            const uint4 q = r.b[it];
            uint32_t words[4] = {q.x, q.y, q.z, q.w}, out[8];
#pragma unroll
            for (int wi = 0; wi < 4; ++wi) fp8x4_bf16(words[wi], out[2 * wi], out[2 * wi + 1]);
            uint4* d = (uint4*)(Bs + row * V3L + seg * 16);
            d[0] = make_uint4(out[0], out[1], out[2], out[3]);
            d[1] = make_uint4(out[4], out[5], out[6], out[7]);
        }
    } else {
        float sc0, sc1;
        if (FMT == EO_W_MXFP4) {
            sc0 = sc1 = e8m0_f32(r.sc);
        } else {
            sc0 = e4m3_f32(r.sc & 0xFF);
            sc1 = e4m3_f32(r.sc >> 8);
        }
        fp4x32_to_lds<FMT>(r.b[0], sc0, sc1, Bs + tid * V3L);
    }
}

template <int FMT, int MODE>
__global__ __launch_bounds__(256, 2) void k_gemm_v3(GemmArgs a, int nN) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    // pipeline buffer b: A at smem + b*V3M*V3L, B at smem + 2*V3M*V3L + b*V3N*V3L;
    // after the K loop the same bytes hold the epilogue tile; row info follows.
    int32_t* s_pair = (int32_t*)((uint8_t*)smem + (kV3Pipe > kV3Out ? kV3Pipe : kV3Out));
    float* s_wp = (float*)(s_pair + V3M);

    // Tile order: (row tile, weight tile) with the weight tile fastest, so the
    // nN tiles that share a row tile, and the row tiles of one expert that share
    // its weights, run back to back. Workgroups are dealt to the 8 XCDs round
    // robin (id mod 8); each XCD gets one contiguous share of the real tiles, so
    // that sharing happens in its own L2.
    const int real = a.tile_off[a.G] * nN;
    const int per = (real + 7) >> 3;
    const int logical = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if ((int)(blockIdx.x >> 3) >= per || logical >= real) return;
    const int tile = logical / nN, ntile = logical - tile * nN;
    const int g = find_group(a.tile_off, a.G, tile);
    const int m0 = a.offsets[g] + (tile - a.tile_off[g]) * V3M;
    const int m_end = a.offsets[g + 1];
    const uint8_t* wb = group_base(a.gw, g, a.E);
    const uint8_t* wdata = wb + (MODE == 0 ? a.lay.d13 : a.lay.d2);
    const uint8_t* wscal = wb + (MODE == 0 ? a.lay.s13 : a.lay.s2);
    const int n0 = ntile * (MODE == 0 ? 128 : 256);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int nk = a.K / V3K;

    if (MODE == 1 && tid < V3M) {
        int pair = m0 + tid < m_end ? a.perm_pair[m0 + tid] : -1;
        s_pair[tid] = pair;
        s_wp[tid] = pair < 0 ? 0.0f : (pair < a.Tk ? a.w[pair] : 1.0f);
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    auto brow = [&](int j) -> int {  // LDS B row of N block j of this wavefront
        if (MODE == 0) return (j >> 1) * 128 + wn * 64 + (j & 1) * 32;
        return wn * 128 + j * 32;
    };

    V3Regs<FMT> regs;
    v3_load<FMT, MODE>(a, wdata, wscal, m0, m_end, n0, 0, tid, regs);
    v3_store<FMT>(smem, smem + 2 * V3M * V3L, tid, regs);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) v3_load<FMT, MODE>(a, wdata, wscal, m0, m_end, n0, (kt + 1) * V3K, tid, regs);
        const uint16_t* A_ = smem + cur * (V3M * V3L);
        const uint16_t* B_ = smem + 2 * V3M * V3L + cur * (V3N * V3L);
#pragma unroll
        for (int ks = 0; ks < V3K / 16; ++ks) {
            const int kc = ks * 16 + (lane >> 5) * 8;
            bf16x8 av[2], bv[4];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                av[i] = *(const bf16x8*)(A_ + (wm * 64 + i * 32 + (lane & 31)) * V3L + kc);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bv[j] = *(const bf16x8*)(B_ + (brow(j) + (lane & 31)) * V3L + kc);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk)
            v3_store<FMT>(smem + (cur ^ 1) * (V3M * V3L),
                          smem + 2 * V3M * V3L + (cur ^ 1) * (V3N * V3L), tid, regs);
        __syncthreads();
    }

    // epilogue: scaled bf16 values into the LDS tile (the pipeline buffers are
    // free after the last barrier), then 16-byte row segments to global memory
    uint16_t* ot = smem;
    const int col = lane & 31;
    if (MODE == 0) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int c = wn * 64 + jj * 32 + col;  // column within the 128-wide h tile
            const int n = n0 + c;
            float sg = 1.0f, su = 1.0f;
            if (FMT == EO_W_FP8) {
                sg = ((const float*)wscal)[n];
                su = ((const float*)wscal)[a.I + n];
            } else if (FMT == EO_W_NVFP4) {
                const float* gl = (const float*)(wb + a.lay.gl);
                sg = gl[0];
                su = gl[1];
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    int row = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    float gv = acc[i][jj][v] * sg, uv = acc[i][2 + jj][v] * su;
                    ot[row * V3_OUT_LD + c] = (uint16_t)f32_bf16_rne(silu_f32(gv) * uv);
                }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 8; ++it) {  // 128 rows x 16 segments of 16 B
            int cidx = tid + 256 * it, row = cidx >> 4, seg = cidx & 15;
            if (m0 + row < m_end)
                *(uint4*)(a.h_out + (size_t)(m0 + row) * a.I + n0 + seg * 8) =
                    *(const uint4*)(ot + row * V3_OUT_LD + seg * 8);
        }
    } else {
        const float gs = FMT == EO_W_NVFP4 ? ((const float*)(wb + a.lay.gl))[2] : 1.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = wn * 128 + j * 32 + col;
            const float sc = FMT == EO_W_FP8 ? ((const float*)wscal)[n0 + c] : gs;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    int row = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    ot[row * V3_OUT_LD + c] = (uint16_t)f32_bf16_rne(acc[i][j][v] * sc * s_wp[row]);
                }
        }
        __syncthreads();
        uint16_t* op = (uint16_t*)a.o_pairs;
#pragma unroll
        for (int it = 0; it < 16; ++it) {  // 128 rows x 32 segments of 16 B
            int cidx = tid + 256 * it, row = cidx >> 5, seg = cidx & 31;
            int pair = s_pair[row];
            if (pair >= 0)
                *(uint4*)(op + (size_t)pair * a.H + n0 + seg * 8) =
                    *(const uint4*)(ot + row * V3_OUT_LD + seg * 8);
        }
    }
}

template <int FMT>
bool run_v3(GemmArgs a1, GemmArgs a2, int tiles, int I, int H, hipStream_t s, hipEvent_t* ev) {
    if (I % 128 || H % 256) return false;
    static bool attr = false;
    if (!attr) {
        if (hipFuncSetAttribute((const void*)k_gemm_v3<FMT, 0>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, kV3Lds) != hipSuccess ||
            hipFuncSetAttribute((const void*)k_gemm_v3<FMT, 1>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, kV3Lds) != hipSuccess)
            return false;
        attr = true;
    }
    const int n1 = I / 128, n2 = H / 256;
    auto grid = [&](int nN) { return ((tiles * nN + 7) / 8) * 8; };
    hipExtLaunchKernelGGL(k_gemm_v3<FMT, 0>, dim3(grid(n1)), dim3(256), (uint32_t)kV3Lds, s,
                          ev[0], ev[1], 0, a1, n1);
    hipExtLaunchKernelGGL(k_gemm_v3<FMT, 1>, dim3(grid(n2)), dim3(256), (uint32_t)kV3Lds, s,
                          ev[2], ev[3], 0, a2, n2);
    return true;
}

// ------------------------------------------------------------------ v4 (bf16)
// Same tiles and epilogue as v3, but the K loop is a 3-stage ring filled by
// direct-to-LDS loads (global_load_lds_dwordx4): two K tiles are in flight
// while the third is multiplied, and no VGPRs carry the tiles. Each load
// instruction of a wavefront fills 1 KB of LDS in lane order, so rows are
// unpadded (64 B = 4 segments of 16 B for K step 32) and a lane loads the
// global segment that belongs in its slot: segment s of row r sits in slot
// s ^ ((r >> 2) & 3). With that XOR swizzle the 16 lanes of each ds_read_b128
// quarter (16 rows, one logical segment) hit 16 distinct 16-byte bank groups.
// Barriers are raw s_barrier with explicit vmcnt waits, so outstanding tile
// loads are not drained at each K step, and each step's six tile loads are
// issued between its MFMAs rather than in one burst after the barrier.
// Two workgroups share a CU: measured on the prefill shapes, a 128 x 512 tile
// (one workgroup per CU, 4 x 4 MFMA blocks per wavefront), rings of 4-6 stages
// at one workgroup per CU, one eight-wavefront workgroup whose two halves
// alternate between multiplying and loading, a K step of 64 with A fragments in
// registers, and 64-row tiles at three workgroups per CU are 7-24% slower; the
// second, unsynchronised workgroup covers each workgroup's barrier waits.
constexpr int kV4Ring = 3;                                // stages: two tiles in flight
constexpr size_t kV4Stage = (size_t)(V3M + V3N) * 64;     // 24 KB per stage
template <int S>
constexpr size_t v4_pipe() { return S * kV4Stage; }
template <int S>
constexpr size_t v4_lds() {
    return (v4_pipe<S>() > kV3Out ? v4_pipe<S>() : kV3Out) + 2 * V3M * sizeof(int32_t);
}

// Wait until at most N of this thread's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14));
}

// The same, and all of this thread's LDS operations done.
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | ((N >> 4) << 14));
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row, int seg) { return seg ^ ((row >> 2) & 3); }

// This lane's two A source rows (tile rows (it*4 + wave)*16 + lane/4, rows past
// the group's end repeat its last row), at the lane's swizzled segment.
template <int MODE>
__device__ __forceinline__ void v4_arows(const GemmArgs& a, int m0, int m_end, int wave, int lane,
                                         const uint16_t* (&ap)[2]) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int row = (it * 4 + wave) * 16 + (lane >> 2);
        const int gr = min(m0 + row, m_end - 1);
        ap[it] = a.A + (size_t)a_row<MODE>(a, gr) * a.K + swz(row, lane & 3) * 8;
    }
}

template <int MODE>
__device__ __forceinline__ void v4_issue(const GemmArgs& a, const uint16_t* wdata,
                                         const uint16_t* const (&ap)[2], int n0, int k0,
                                         uint8_t* stage, int wave, int lane) {
    const int K = a.K;
    const int lrow = lane >> 2, slot = lane & 3;
#pragma unroll
    for (int it = 0; it < 2; ++it)  // A: 8 x 1 KB, rows (it*4 + wave)*16 ..
        __builtin_amdgcn_global_load_lds(ap[it] + k0, (lds_void*)(stage + (it * 4 + wave) * 1024),
                                         16, 0, 0);
#pragma unroll
    for (int it = 0; it < 4; ++it) {  // B: 16 x 1 KB
        const int row = (it * 4 + wave) * 16 + lrow;
        const int wr = MODE == 0 ? (row < 128 ? n0 + row : a.I + n0 + row - 128) : n0 + row;
        const uint16_t* src = wdata + (size_t)wr * K + k0 + swz(row, slot) * 8;
        __builtin_amdgcn_global_load_lds(src, (lds_void*)(stage + V3M * 64 + (it * 4 + wave) * 1024),
                                         16, 0, 0);
    }
}

template <int MODE, int S>
__global__ __launch_bounds__(256, 2) void k_gemm_v4(GemmArgs a, int nN) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    uint8_t* sb = (uint8_t*)smem;
    int32_t* s_pair = (int32_t*)(sb + (v4_pipe<S>() > kV3Out ? v4_pipe<S>() : kV3Out));
    float* s_wp = (float*)(s_pair + V3M);

    const int real = a.tile_off[a.G] * nN;
    const int per = (real + 7) >> 3;
    const int logical = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if ((int)(blockIdx.x >> 3) >= per || logical >= real) return;
    const int tile = logical / nN, ntile = logical - tile * nN;
    const int g = find_group(a.tile_off, a.G, tile);
    const int m0 = a.offsets[g] + (tile - a.tile_off[g]) * V3M;
    const int m_end = a.offsets[g + 1];
    const uint8_t* wb = group_base(a.gw, g, a.E);
    const uint16_t* wdata = (const uint16_t*)(wb + (MODE == 0 ? a.lay.d13 : a.lay.d2));
    const int n0 = ntile * (MODE == 0 ? 128 : 256);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int nk = a.K / V3K;

    if (MODE == 1 && tid < V3M) {
        int pair = m0 + tid < m_end ? a.perm_pair[m0 + tid] : -1;
        s_pair[tid] = pair;
        s_wp[tid] = pair < 0 ? 0.0f : (pair < a.Tk ? a.w[pair] : 1.0f);
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const uint16_t* ap[2];
    v4_arows<MODE>(a, m0, m_end, wave, lane, ap);
#pragma unroll
    for (int t = 0; t < S - 1; ++t)
        v4_issue<MODE>(a, wdata, ap, n0, min(t, nk - 1) * V3K, sb + t * kV4Stage, wave, lane);

    int arow[2], aseg[2][2];  // A rows read by this lane and their swizzled slots
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        arow[i] = wm * 64 + i * 32 + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) aseg[i][ks] = swz(arow[i], 2 * ks + (lane >> 5));
    }
    int brow_[4], bseg[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        brow_[j] = (MODE == 0 ? (j >> 1) * 128 + wn * 64 + (j & 1) * 32 : wn * 128 + j * 32) +
                   (lane & 31);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) bseg[j][ks] = swz(brow_[j], 2 * ks + (lane >> 5));
    }

    // Every step issues one tile (past the end, the last tile again), so
    // S - 1 tiles are always in flight at the wait and the body is one
    // block: the loads of tile kt + S - 1 are spread between this step's
    // MFMAs instead of stalling the wavefront in one burst.
    for (int kt = 0; kt < nk; ++kt) {
        wait_vm<(S - 2) * 6>();
        __builtin_amdgcn_s_barrier();
        const uint8_t* st = sb + (kt % S) * kV4Stage;
        bf16x8 av[2][2], bv[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i) av[0][i] = *(const bf16x8*)(st + arow[i] * 64 + aseg[i][0] * 16);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bv[0][j] = *(const bf16x8*)(st + V3M * 64 + brow_[j] * 64 + bseg[j][0] * 16);
        v4_issue<MODE>(a, wdata, ap, n0, min(kt + S - 1, nk - 1) * V3K,
                       sb + ((kt + S - 1) % S) * kV4Stage, wave, lane);
#pragma unroll
        for (int i = 0; i < 2; ++i) av[1][i] = *(const bf16x8*)(st + arow[i] * 64 + aseg[i][1] * 16);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bv[1][j] = *(const bf16x8*)(st + V3M * 64 + brow_[j] * 64 + bseg[j][1] * 16);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[ks][i], bv[ks][j],
                                                                        acc[i][j], 0, 0, 0);
        // order: first half step's 6 operand reads; then 6 x (MFMA, tile
        // load, operand read of the second half); then the other 10 MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int q = 0; q < 6; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 10, 0);
    }
    wait_vm<0>();
    __syncthreads();  // all tile loads landed and all LDS reads done: reuse as the epilogue tile

    uint16_t* ot = smem;
    const int col = lane & 31;
    if (MODE == 0) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int c = wn * 64 + jj * 32 + col;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    int row = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    ot[row * V3_OUT_LD + c] =
                        (uint16_t)f32_bf16_rne(silu_f32(acc[i][jj][v]) * acc[i][2 + jj][v]);
                }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            int cidx = tid + 256 * it, row = cidx >> 4, seg = cidx & 15;
            if (m0 + row < m_end)
                *(uint4*)(a.h_out + (size_t)(m0 + row) * a.I + n0 + seg * 8) =
                    *(const uint4*)(ot + row * V3_OUT_LD + seg * 8);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = wn * 128 + j * 32 + col;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    int row = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    ot[row * V3_OUT_LD + c] = (uint16_t)f32_bf16_rne(acc[i][j][v] * s_wp[row]);
                }
        }
        __syncthreads();
        uint16_t* op = (uint16_t*)a.o_pairs;
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            int cidx = tid + 256 * it, row = cidx >> 5, seg = cidx & 31;
            int pair = s_pair[row];
            if (pair >= 0)
                *(uint4*)(op + (size_t)pair * a.H + n0 + seg * 8) =
                    *(const uint4*)(ot + row * V3_OUT_LD + seg * 8);
        }
    }
}

template <int S>
bool run_v4(GemmArgs a1, GemmArgs a2, int tiles, int I, int H, hipStream_t s, hipEvent_t* ev) {
    static_assert(2 * v4_lds<S>() <= 160 * 1024, "v4 LDS: two workgroups per CU");
    if (I % 128 || H % 256 || H % V3K || I % V3K) return false;
    static bool attr = false;
    if (!attr) {
        if (hipFuncSetAttribute((const void*)k_gemm_v4<0, S>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, v4_lds<S>()) != hipSuccess ||
            hipFuncSetAttribute((const void*)k_gemm_v4<1, S>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, v4_lds<S>()) != hipSuccess)
            return false;
        attr = true;
    }
    const int n1 = I / 128, n2 = H / 256;
    auto grid = [&](int nN) { return ((tiles * nN + 7) / 8) * 8; };
    hipExtLaunchKernelGGL((k_gemm_v4<0, S>), dim3(grid(n1)), dim3(256), (uint32_t)v4_lds<S>(), s,
                          ev[0], ev[1], 0, a1, n1);
    hipExtLaunchKernelGGL((k_gemm_v4<1, S>), dim3(grid(n2)), dim3(256), (uint32_t)v4_lds<S>(), s,
                          ev[2], ev[3], 0, a2, n2);
    return true;
}

// ------------------------------------------------------------------ v5 (bf16)
// v4's tiles, MFMAs and epilogue with the weight tile loaded as 128-byte rows.
// A direct-to-LDS load instruction fills 1 KB: with 64-byte rows it touches 16
// rows, i.e. 16 cache lines, with 128-byte rows 8. In a loop-only probe of the
// same tiles and swizzle the 128-byte rows ran ~20% faster, but v4's
// three-stage ring at K step 64 needs 144 KB. Here the two operands get rings of
// their own, two slots each: A (128 rows) keeps 64-byte rows at K step 32
// (8 KB a slot), B (256 rows) has 128-byte rows at K step 64 (32 KB a slot),
// 80 KB in all, so two workgroups still share a CU. Each K-32 step issues the
// next A tile (2 loads per wavefront), which has one step to land; each even
// step also issues the whole next B tile (8 loads), which has two. (Half of
// the B tile at each step, 6 loads per step as in v4, ran 2-3% slower.)
// Segment s of a 128-byte B row r sits in slot
// s ^ ((r >> 1) & 7): the 16 lanes of a ds_read_b128 quarter (16 rows, one
// logical segment) then hit 16 distinct 16-byte bank groups.
constexpr size_t kV5ASlot = (size_t)V3M * 64;            // 8 KB: 128 rows x K 32
constexpr size_t kV5BSlot = (size_t)V3N * 128;           // 32 KB: 256 rows x K 64
constexpr size_t kV5Lds = 2 * kV5ASlot + 2 * kV5BSlot;   // 80 KB
static_assert(kV3Out + 2 * V3M * sizeof(int32_t) <= kV5Lds, "epilogue tile and pair table");
static_assert(2 * kV5Lds <= 160 * 1024, "v5 LDS: two workgroups per CU");

// Half h (rows h*128 .. h*128 + 127) of the B tile at K offset k0 (64 wide):
// 4 x 1 KB per wavefront, 8 rows of 128 B each.
template <int MODE>
__device__ __forceinline__ void v5_issue_b(const GemmArgs& a, const uint16_t* wdata, int n0,
                                           int k0, int h, uint8_t* bslot, int wave, int lane) {
    const int K = a.K;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int rbase = h * 128 + (it * 4 + wave) * 8;
        const int row = rbase + (lane >> 3);
        const int wr = MODE == 0 ? (h == 0 ? n0 + row : a.I + n0 + row - 128) : n0 + row;
        const int seg = (lane & 7) ^ ((row >> 1) & 7);
        __builtin_amdgcn_global_load_lds(wdata + (size_t)wr * K + k0 + seg * 8,
                                         (lds_void*)(bslot + rbase * 128), 16, 0, 0);
    }
}

// The A tile at K offset k0 (32 wide): 2 x 1 KB per wavefront, as in v4.
__device__ __forceinline__ void v5_issue_a(const uint16_t* const (&ap)[2], int k0, uint8_t* aslot,
                                           int wave) {
#pragma unroll
    for (int it = 0; it < 2; ++it)
        __builtin_amdgcn_global_load_lds(ap[it] + k0, (lds_void*)(aslot + (it * 4 + wave) * 1024),
                                         16, 0, 0);
}

template <int MODE>
__global__ __launch_bounds__(256, 2) void k_gemm_v5(GemmArgs a, int nN) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    uint8_t* sb = (uint8_t*)smem;
    uint8_t* const sa = sb;                   // A slots
    uint8_t* const sw = sb + 2 * kV5ASlot;    // B slots

    const int real = a.tile_off[a.G] * nN;
    const int per = (real + 7) >> 3;
    const int logical = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if ((int)(blockIdx.x >> 3) >= per || logical >= real) return;
    const int tile = logical / nN, ntile = logical - tile * nN;
    const int g = find_group(a.tile_off, a.G, tile);
    const int m0 = a.offsets[g] + (tile - a.tile_off[g]) * V3M;
    const int m_end = a.offsets[g + 1];
    const uint8_t* wb = group_base(a.gw, g, a.E);
    const uint16_t* wdata = (const uint16_t*)(wb + (MODE == 0 ? a.lay.d13 : a.lay.d2));
    const int n0 = ntile * (MODE == 0 ? 128 : 256);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int nk = a.K / V3K;

    // the pair table goes to LDS after the K loop, which uses all of it
    int my_pair = -1;
    if (MODE == 1 && tid < V3M) my_pair = m0 + tid < m_end ? a.perm_pair[m0 + tid] : -1;

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const uint16_t* ap[2];
    v4_arows<MODE>(a, m0, m_end, wave, lane, ap);
    v5_issue_a(ap, 0, sa, wave);
    v5_issue_b<MODE>(a, wdata, n0, 0, 0, sw, wave, lane);
    v5_issue_b<MODE>(a, wdata, n0, 0, 1, sw, wave, lane);

    // A tile with at most 64 rows of its group (the group's ragged end) is
    // split over the four wavefronts by columns alone: each multiplies rows
    // 0..63 by a quarter of the 256 columns (8 MFMAs a step instead of 16),
    // MODE 0 a quarter of the gate columns and the matching up columns. The
    // same MFMAs run in the same K order for each output, so the results are
    // the same bits.
    const bool half = m_end - m0 <= 64;  // workgroup-uniform
    int arow[2], aseg[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        arow[i] = (half ? 0 : wm * 64) + i * 32 + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) aseg[i][ks] = swz(arow[i], 2 * ks + (lane >> 5));
    }
    // byte offset of this lane's B operand in the first K-32 half of a slot;
    // the second half's segments are the first's + 4, i.e. offset ^ 64
    int boff[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int br = half ? (MODE == 0 ? (j & 1) * 128 + wave * 32 : wave * 64 + (j & 1) * 32) +
                                  (lane & 31)
                            : (MODE == 0 ? (j >> 1) * 128 + wn * 64 + (j & 1) * 32
                                         : wn * 128 + j * 32) +
                                  (lane & 31);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            boff[j][ks] = br * 128 + (((2 * ks + (lane >> 5)) ^ ((br >> 1) & 7)) << 4);
    }

    // One K-32 step. At an even step the previous step's loads brought the A
    // tile (wait for all); at an odd step they brought the A tile and the next
    // B tile (its 2 A loads go before the 8 B loads, and loads count down in
    // issue order, so wait until 8 are left). The last two steps load only
    // what is left (the last A tile) and wait for everything, so no load is in
    // flight when the K loop ends. HALF: the ragged tile's 2 column blocks per
    // wavefront (acc[.][0..1]) instead of 4.
    auto step = [&](int kt, auto odd_t, auto last_t, auto half_t) {
        constexpr int ODD = decltype(odd_t)::value, LAST = decltype(last_t)::value;
        constexpr int NB = decltype(half_t)::value ? 2 : 4;
        // this wavefront's LDS reads of the previous step are done too: the
        // compiler may hoist them above their MFMAs, and after the barrier
        // other wavefronts load into the slot they read
        wait_vm_lds<ODD && !LAST ? 8 : 0>();
        __builtin_amdgcn_s_barrier();
        const uint8_t* sta = sa + (kt & 1) * kV5ASlot;
        const uint8_t* stb = sw + ((kt >> 1) & 1) * kV5BSlot;
        constexpr int hx = ODD << 6;
        bf16x8 av[2][2], bv[2][NB];
#pragma unroll
        for (int i = 0; i < 2; ++i) av[0][i] = *(const bf16x8*)(sta + arow[i] * 64 + aseg[i][0] * 16);
#pragma unroll
        for (int j = 0; j < NB; ++j) bv[0][j] = *(const bf16x8*)(stb + (boff[j][0] ^ hx));
        if (!(LAST && ODD)) v5_issue_a(ap, (kt + 1) * V3K, sa + ((kt + 1) & 1) * kV5ASlot, wave);
        if (!ODD && !LAST) {
            v5_issue_b<MODE>(a, wdata, n0, ((kt >> 1) + 1) * 64, 0,
                             sw + (((kt >> 1) + 1) & 1) * kV5BSlot, wave, lane);
            v5_issue_b<MODE>(a, wdata, n0, ((kt >> 1) + 1) * 64, 1,
                             sw + (((kt >> 1) + 1) & 1) * kV5BSlot, wave, lane);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) av[1][i] = *(const bf16x8*)(sta + arow[i] * 64 + aseg[i][1] * 16);
#pragma unroll
        for (int j = 0; j < NB; ++j) bv[1][j] = *(const bf16x8*)(stb + (boff[j][1] ^ hx));
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[ks][i], bv[ks][j],
                                                                        acc[i][j], 0, 0, 0);
        constexpr int NDS = 2 + NB, NM = 4 * NB;  // each half step's LDS reads; MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);
        constexpr int NV = LAST ? (ODD ? 0 : 2) : (ODD ? 2 : 10);  // this step's loads
        constexpr int NQ = NV > NDS ? NV : NDS;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (q < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (q < NV) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
            if (q < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (NM > NQ) __builtin_amdgcn_sched_group_barrier(0x008, NM - NQ, 0);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    auto kloop = [&](auto half_t) {
        for (int kt = 0; kt < nk - 2; kt += 2) {
            step(kt, I0{}, I0{}, half_t);
            step(kt + 1, I1{}, I0{}, half_t);
        }
        step(nk - 2, I0{}, I1{}, half_t);
        step(nk - 1, I1{}, I1{}, half_t);
    };
    if (half)
        kloop(I1{});
    else
        kloop(I0{});
    wait_vm<0>();
    __syncthreads();  // all tile loads landed and all LDS reads done: reuse as the epilogue tile

    uint16_t* ot = smem;
    int32_t* s_pair = (int32_t*)(sb + kV3Out);
    float* s_wp = (float*)(s_pair + V3M);
    const int col = lane & 31;
    if (MODE == 0) {
        if (half) {  // rows 0..63; gate block acc[.][0], up block acc[.][1]
            const int c = wave * 32 + col;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    int row = i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    ot[row * V3_OUT_LD + c] =
                        (uint16_t)f32_bf16_rne(silu_f32(acc[i][0][v]) * acc[i][1][v]);
                }
        } else {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int c = wn * 64 + jj * 32 + col;
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        int row = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                        ot[row * V3_OUT_LD + c] =
                            (uint16_t)f32_bf16_rne(silu_f32(acc[i][jj][v]) * acc[i][2 + jj][v]);
                    }
            }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            int cidx = tid + 256 * it, row = cidx >> 4, seg = cidx & 15;
            if (m0 + row < m_end)
                *(uint4*)(a.h_out + (size_t)(m0 + row) * a.I + n0 + seg * 8) =
                    *(const uint4*)(ot + row * V3_OUT_LD + seg * 8);
        }
    } else {
        if (tid < V3M) {
            s_pair[tid] = my_pair;
            s_wp[tid] = my_pair < 0 ? 0.0f : (my_pair < a.Tk ? a.w[my_pair] : 1.0f);
        }
        __syncthreads();
        if (half) {  // rows 0..63, columns wave * 64 ..
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c = wave * 64 + j * 32 + col;
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        int row = i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                        ot[row * V3_OUT_LD + c] = (uint16_t)f32_bf16_rne(acc[i][j][v] * s_wp[row]);
                    }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = wn * 128 + j * 32 + col;
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        int row = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                        ot[row * V3_OUT_LD + c] = (uint16_t)f32_bf16_rne(acc[i][j][v] * s_wp[row]);
                    }
            }
        }
        __syncthreads();
        uint16_t* op = (uint16_t*)a.o_pairs;
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            int cidx = tid + 256 * it, row = cidx >> 5, seg = cidx & 31;
            int pair = s_pair[row];
            if (pair >= 0)
                *(uint4*)(op + (size_t)pair * a.H + n0 + seg * 8) =
                    *(const uint4*)(ot + row * V3_OUT_LD + seg * 8);
        }
    }
}

bool run_v5(GemmArgs a1, GemmArgs a2, int tiles, int I, int H, hipStream_t s, hipEvent_t* ev) {
    if (I % 128 || H % 256) return false;  // K = H or I: whole K-64 tiles
    static bool attr = false;
    if (!attr) {
        if (hipFuncSetAttribute((const void*)k_gemm_v5<0>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, kV5Lds) != hipSuccess ||
            hipFuncSetAttribute((const void*)k_gemm_v5<1>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, kV5Lds) != hipSuccess)
            return false;
        attr = true;
    }
    const int n1 = I / 128, n2 = H / 256;
    auto grid = [&](int nN) { return ((tiles * nN + 7) / 8) * 8; };
    hipExtLaunchKernelGGL(k_gemm_v5<0>, dim3(grid(n1)), dim3(256), (uint32_t)kV5Lds, s, ev[0],
                          ev[1], 0, a1, n1);
    hipExtLaunchKernelGGL(k_gemm_v5<1>, dim3(grid(n2)), dim3(256), (uint32_t)kV5Lds, s, ev[2],
                          ev[3], 0, a2, n2);
    return true;
}

// ------------------------------------------------------------------ v4q (fp8 / fp4)
// The v4 ring for quantised weights: the A tile arrives by direct-to-LDS loads
// two K tiles ahead; each thread holds one weight row's next 64-byte span of
// codes (two FP8 tiles, four fp4 tiles, with the fp4 block scales) in
// registers, decodes one tile of it per step exactly to bf16 (the scaled
// converts) and writes it into the next stage in the ring's XOR-swizzled
// 64-byte rows. The decode and the next span's loads sit between the two K
// halves' MFMAs (placed before the first half, GEMM1 ran 10-20% slower). The K
// loop is unrolled by the span so that each step's wait for its A tile is a
// constant.

// A load through a global (address space 1) pointer. The weight pointers come
// out of a table, so the compiler cannot tell they are global and would emit
// flat loads; while a flat load is outstanding it waits for vmcnt(0) before
// every LDS access, which drains the ring's activation loads each step.
// T is a scalar or clang vector type (HIP's struct vector types still become
// flat loads).
template <typename T>
__device__ __forceinline__ T gload(const void* p) {
    return *(const __attribute__((address_space(1))) T*)p;
}

// A 16-byte LDS store that the compiler's wait insertion does not see. The
// decoded weight rows go to a stage's B region while the ring's direct-to-LDS
// loads are in flight to A regions; the compiler cannot tell the addresses
// apart and would wait for every outstanding load before a plain LDS store,
// i.e. for the activation tile issued at the top of the same step. The store
// has no outputs; its completion is covered by the lgkmcnt(0) before each
// step's barrier, and one wavefront's LDS operations complete in order.
__device__ __forceinline__ void lds_store16(uint8_t* p, u32x4 v) {
    const uint32_t addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)p;
    asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// One weight row's next 64 contiguous bytes per thread (row = thread): two K
// tiles of FP8 codes, or four of fp4 codes with their block scales. Requested
// together, so a row's 128-byte line is fetched once per span, not once per tile.
template <int FMT>
struct QRegs {
    u32x4 s0, s1, s2, s3;
    uint32_t ss0, ss1;
};

template <int FMT, int MODE>
__device__ __forceinline__ void q_load(const GemmArgs& a, const uint8_t* wdata,
                                       const uint8_t* wscal, int n0, int k0, int tid,
                                       QRegs<FMT>& r) {
    // row tid's span from k0 (k0 % 64 == 0 for FP8, % 128 for fp4): 4 loads,
    // plus 1 for the fp4 block scales
    const int K = a.K;
    const int wr = v3_wrow<FMT, MODE>(a, n0, tid);
    const uint8_t* rp = wdata + (FMT == EO_W_FP8 ? (size_t)wr * K + k0 : (size_t)wr * (K / 2) + k0 / 2);
    r.s0 = gload<u32x4>(rp);
    r.s1 = gload<u32x4>(rp + 16);
    r.s2 = gload<u32x4>(rp + 32);
    r.s3 = gload<u32x4>(rp + 48);
    if (FMT == EO_W_MXFP4) {
        r.ss0 = gload<uint32_t>(wscal + (size_t)wr * (K / 32) + k0 / 32);
    } else if (FMT == EO_W_NVFP4) {
        const uint64_t q = gload<uint64_t>(wscal + (size_t)wr * (K / 16) + k0 / 16);
        r.ss0 = (uint32_t)q;
        r.ss1 = (uint32_t)(q >> 32);
    }
}

// Decodes tile U of the span (fp4) or the loaded tile (FP8) into the stage's
// weight rows.
template <int FMT, int U>
__device__ __forceinline__ void q_store(uint8_t* bst, int tid, const QRegs<FMT>& r) {
    if (FMT == EO_W_FP8) {
        const int row = tid;
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // 16 codes = logical segments 2h, 2h + 1
            const u32x4 v = U == 0 ? (h == 0 ? r.s0 : r.s1) : (h == 0 ? r.s2 : r.s3);
            uint32_t out[8];
#pragma unroll
            for (int wi = 0; wi < 4; ++wi) fp8x4_bf16(v[wi], out[2 * wi], out[2 * wi + 1]);
            lds_store16(bst + row * 64 + swz(row, 2 * h) * 16, u32x4{out[0], out[1], out[2], out[3]});
            lds_store16(bst + row * 64 + swz(row, 2 * h + 1) * 16,
                        u32x4{out[4], out[5], out[6], out[7]});
        }
    } else {
        const u32x4 v = U == 0 ? r.s0 : U == 1 ? r.s1 : U == 2 ? r.s2 : r.s3;
        float sc0, sc1;
        if (FMT == EO_W_MXFP4) {
            sc0 = sc1 = e8m0_f32((r.ss0 >> (8 * U)) & 0xFFu);
        } else {
            const uint32_t sc = ((U < 2 ? r.ss0 : r.ss1) >> (16 * (U & 1))) & 0xFFFFu;
            sc0 = e4m3_f32(sc & 0xFF);
            sc1 = e4m3_f32(sc >> 8);
        }
        const uint32_t words[4] = {v[0], v[1], v[2], v[3]};
        const int row = tid;
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {  // 8 codes = logical segment wi
            const float sc = wi < 2 ? sc0 : sc1;
            lds_store16(bst + row * 64 + swz(row, wi) * 16,
                        u32x4{fp4x2_bf16<FMT, 0>(words[wi], sc), fp4x2_bf16<FMT, 1>(words[wi], sc),
                              fp4x2_bf16<FMT, 2>(words[wi], sc), fp4x2_bf16<FMT, 3>(words[wi], sc)});
        }
    }
}

template <int FMT, int MODE>
__global__ __launch_bounds__(256, 2) void k_gemm_v4q(GemmArgs a, int nN) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    uint8_t* sb = (uint8_t*)smem;
    constexpr int S = kV4Ring;
    int32_t* s_pair = (int32_t*)(sb + (v4_pipe<S>() > kV3Out ? v4_pipe<S>() : kV3Out));
    float* s_wp = (float*)(s_pair + V3M);

    const int real = a.tile_off[a.G] * nN;
    const int per = (real + 7) >> 3;
    const int logical = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if ((int)(blockIdx.x >> 3) >= per || logical >= real) return;
    const int tile = logical / nN, ntile = logical - tile * nN;
    const int g = find_group(a.tile_off, a.G, tile);
    const int m0 = a.offsets[g] + (tile - a.tile_off[g]) * V3M;
    const int m_end = a.offsets[g + 1];
    const uint8_t* wb = group_base(a.gw, g, a.E);
    const uint8_t* wdata = wb + (MODE == 0 ? a.lay.d13 : a.lay.d2);
    const uint8_t* wscal = wb + (MODE == 0 ? a.lay.s13 : a.lay.s2);
    const int n0 = ntile * (MODE == 0 ? 128 : 256);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int nk = a.K / V3K;

    if (MODE == 1 && tid < V3M) {
        int pair = m0 + tid < m_end ? a.perm_pair[m0 + tid] : -1;
        s_pair[tid] = pair;
        s_wp[tid] = pair < 0 ? 0.0f : (pair < a.Tk ? a.w[pair] : 1.0f);
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const uint16_t* ap[2];
    v4_arows<MODE>(a, m0, m_end, wave, lane, ap);
    auto issue_a = [&](int kt, uint8_t* stage) {
#pragma unroll
        for (int it = 0; it < 2; ++it)
            __builtin_amdgcn_global_load_lds(ap[it] + kt * V3K,
                                             (lds_void*)(stage + (it * 4 + wave) * 1024), 16, 0, 0);
    };

    int arow[2], aseg[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        arow[i] = wm * 64 + i * 32 + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) aseg[i][ks] = swz(arow[i], 2 * ks + (lane >> 5));
    }
    int brow_[4], bseg[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        brow_[j] = (MODE == 0 ? (j >> 1) * 128 + wn * 64 + (j & 1) * 32 : wn * 128 + j * 32) +
                   (lane & 31);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) bseg[j][ks] = swz(brow_[j], 2 * ks + (lane >> 5));
    }

    auto mma_half = [&](const uint8_t* st, int ks) {
        bf16x8 av[2], bv[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) av[i] = *(const bf16x8*)(st + arow[i] * 64 + aseg[i][ks] * 16);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bv[j] = *(const bf16x8*)(st + V3M * 64 + brow_[j] * 64 + bseg[j][ks] * 16);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    };
    auto bstage = [&](int kt) { return sb + (kt % S) * kV4Stage + V3M * 64; };

    QRegs<FMT> qr;
    issue_a(0, sb);
    issue_a(min(1, nk - 1), sb + kV4Stage);
    if constexpr (FMT == EO_W_FP8) {
        // nk % 2 == 0: the span of tiles 2j, 2j+1 is decoded during steps 2j-1
        // and 2j; span j+1 is requested at step 2j, right after its last decode,
        // and first used at step 2j+1. Loads issued after A tile kt at the top of
        // step kt: 2 (A tile kt+1), plus the 4 of the span requested at step kt-1
        // when kt is odd (when kt is even that span was consumed by the previous
        // step's decode, so it is done).
        q_load<FMT, MODE>(a, wdata, wscal, n0, 0, tid, qr);
        q_store<FMT, 0>(bstage(0), tid, qr);
        for (int kt0 = 0; kt0 < nk; kt0 += 2) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int kt = kt0 + u;
                if (u == 1)
                    wait_vm<6>();
                else
                    wait_vm<2>();
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this thread's weight-tile writes done
                __builtin_amdgcn_s_barrier();
                issue_a(min(kt + 2, nk - 1), sb + ((kt + 2) % S) * kV4Stage);
                const uint8_t* st = sb + (kt % S) * kV4Stage;
                mma_half(st, 0);
                // decode weight tile kt+1 while the first half's MFMAs run
                if (u == 0) {
                    q_store<FMT, 1>(bstage(kt + 1), tid, qr);
                    q_load<FMT, MODE>(a, wdata, wscal, n0, min(kt0 + 2, nk - 2) * V3K, tid, qr);
                } else {
                    q_store<FMT, 0>(bstage(kt + 1), tid, qr);
                }
                mma_half(st, 1);
            }
        }
    } else {
        // fp4 (nk % 4 == 0): the span of tiles 4j..4j+3 is decoded one tile per
        // step during steps 4j-1..4j+2; span j+1 is requested at step 4j+2, right
        // after its last decode, and first used at step 4j+3. Loads issued after
        // A tile kt at the top of step kt: 2 (A tile kt+1) in general, plus the 5
        // of the span requested at step kt-1 when kt % 4 == 3 (at kt % 4 == 0
        // that span was consumed by the previous step's decode, so it is done).
        q_load<FMT, MODE>(a, wdata, wscal, n0, 0, tid, qr);
        q_store<FMT, 0>(bstage(0), tid, qr);
        for (int kt0 = 0; kt0 < nk; kt0 += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int kt = kt0 + u;
                if (u == 3)
                    wait_vm<7>();
                else
                    wait_vm<2>();
                __builtin_amdgcn_s_waitcnt(0xC07F);
                __builtin_amdgcn_s_barrier();
                issue_a(min(kt + 2, nk - 1), sb + ((kt + 2) % S) * kV4Stage);
                const uint8_t* st = sb + (kt % S) * kV4Stage;
                mma_half(st, 0);
                if (u == 0) q_store<FMT, 1>(bstage(kt + 1), tid, qr);
                if (u == 1) q_store<FMT, 2>(bstage(kt + 1), tid, qr);
                if (u == 2) {
                    q_store<FMT, 3>(bstage(kt + 1), tid, qr);
                    q_load<FMT, MODE>(a, wdata, wscal, n0, min(kt0 + 4, nk - 4) * V3K, tid, qr);
                }
                if (u == 3) q_store<FMT, 0>(bstage(kt + 1), tid, qr);
                mma_half(st, 1);
            }
        }
    }
    wait_vm<0>();
    __syncthreads();  // all tile loads landed and all LDS reads done: reuse as the epilogue tile

    uint16_t* ot = smem;
    const int col = lane & 31;
    if (MODE == 0) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int c = wn * 64 + jj * 32 + col;
            const int n = n0 + c;
            float sg = 1.0f, su = 1.0f;
            if (FMT == EO_W_FP8) {
                sg = ((const float*)wscal)[n];
                su = ((const float*)wscal)[a.I + n];
            } else if (FMT == EO_W_NVFP4) {
                const float* gl = (const float*)(wb + a.lay.gl);
                sg = gl[0];
                su = gl[1];
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    int row = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    float gv = acc[i][jj][v] * sg, uv = acc[i][2 + jj][v] * su;
                    ot[row * V3_OUT_LD + c] = (uint16_t)f32_bf16_rne(silu_f32(gv) * uv);
                }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            int cidx = tid + 256 * it, row = cidx >> 4, seg = cidx & 15;
            if (m0 + row < m_end)
                *(uint4*)(a.h_out + (size_t)(m0 + row) * a.I + n0 + seg * 8) =
                    *(const uint4*)(ot + row * V3_OUT_LD + seg * 8);
        }
    } else {
        const float gs = FMT == EO_W_NVFP4 ? ((const float*)(wb + a.lay.gl))[2] : 1.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = wn * 128 + j * 32 + col;
            const float sc = FMT == EO_W_FP8 ? ((const float*)wscal)[n0 + c] : gs;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    int row = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    ot[row * V3_OUT_LD + c] = (uint16_t)f32_bf16_rne(acc[i][j][v] * sc * s_wp[row]);
                }
        }
        __syncthreads();
        uint16_t* op = (uint16_t*)a.o_pairs;
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            int cidx = tid + 256 * it, row = cidx >> 5, seg = cidx & 31;
            int pair = s_pair[row];
            if (pair >= 0)
                *(uint4*)(op + (size_t)pair * a.H + n0 + seg * 8) =
                    *(const uint4*)(ot + row * V3_OUT_LD + seg * 8);
        }
    }
}

template <int FMT>
bool run_v4q(GemmArgs a1, GemmArgs a2, int tiles, int I, int H, hipStream_t s, hipEvent_t* ev) {
    if (I % 128 || H % 256) return false;  // K = H or I: whole 2- or 4-tile spans
    static bool attr = false;
    if (!attr) {
        const uint32_t lds = (uint32_t)v4_lds<kV4Ring>();
        if (hipFuncSetAttribute((const void*)k_gemm_v4q<FMT, 0>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess ||
            hipFuncSetAttribute((const void*)k_gemm_v4q<FMT, 1>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
            return false;
        attr = true;
    }
    const int n1 = I / 128, n2 = H / 256;
    auto grid = [&](int nN) { return ((tiles * nN + 7) / 8) * 8; };
    hipExtLaunchKernelGGL((k_gemm_v4q<FMT, 0>), dim3(grid(n1)), dim3(256), (uint32_t)v4_lds<kV4Ring>(),
                          s, ev[0], ev[1], 0, a1, n1);
    hipExtLaunchKernelGGL((k_gemm_v4q<FMT, 1>), dim3(grid(n2)), dim3(256), (uint32_t)v4_lds<kV4Ring>(),
                          s, ev[2], ev[3], 0, a2, n2);
    return true;
}

template <int FMT>
void run_mfma(GemmArgs a1, GemmArgs a2, int tiles, int I, int H, hipStream_t s, hipEvent_t* ev) {
    if (FMT == EO_W_BF16 && g_gemm_tiles >= 3)
        if (run_v5(a1, a2, tiles, I, H, s, ev)) return;
    if (FMT == EO_W_BF16 && g_gemm_tiles >= 2) {
        if (run_v4<kV4Ring>(a1, a2, tiles, I, H, s, ev)) return;
    }
    if constexpr (FMT != EO_W_BF16)
        if (g_gemm_tiles >= 2 && run_v4q<FMT>(a1, a2, tiles, I, H, s, ev)) return;
    if (g_gemm_tiles && run_v3<FMT>(a1, a2, tiles, I, H, s, ev)) return;
    hipExtLaunchKernelGGL(k_gemm_mfma<FMT, 0>, dim3(tiles, I / 64), dim3(256), 0, s, ev[0], ev[1],
                          0, a1);
    hipExtLaunchKernelGGL(k_gemm_mfma<FMT, 1>, dim3(tiles, H / 128), dim3(256), 0, s, ev[2], ev[3],
                          0, a2);
}

}  // namespace

hipError_t launch_ffn_gemm(int fmt, const Layout& lay, GroupW gw, int E, int has_shared, int H,
                           int I, int P_max, const int32_t* offsets, const int32_t* tile_off,
                           const void* x, void* h_buf, const int32_t* perm_pair,
                           const int32_t* ids, const float* w, int k, int T, void* o_pairs,
                           hipStream_t s, hipEvent_t* ev) {
    (void)ids;
    // EO_GEMM_PATH (read per call, so that tests can compare the kernels)
    const char* path = getenv("EO_GEMM_PATH");
    g_gemm_tiles = path ? atoi(path) : 3;
    const int G = E + (has_shared ? 1 : 0);
    const int tiles = (P_max + kTileM - 1) / kTileM + G;  // upper bound on row tiles
    GemmArgs a1{};
    a1.gw = gw;
    a1.lay = lay;
    a1.E = E;
    a1.G = G;
    a1.H = H;
    a1.I = I;
    a1.offsets = offsets;
    a1.tile_off = tile_off;
    a1.perm_pair = perm_pair;
    a1.w = w;
    a1.Tk = T * k;
    a1.k = k;
    a1.o_pairs = o_pairs;
    GemmArgs a2 = a1;
    a1.K = H;
    a1.A = (const uint16_t*)x;
    a1.h_out = (uint16_t*)h_buf;
    a2.K = I;
    a2.A = (const uint16_t*)h_buf;
    switch (fmt) {
    case EO_W_FP32:
        hipExtLaunchKernelGGL(k_gemm_f32<0>, dim3(tiles, I / 32), dim3(256), 0, s, ev[0], ev[1],
                              0, a1, (const float*)x, (float*)h_buf);
        hipExtLaunchKernelGGL(k_gemm_f32<1>, dim3(tiles, H / 64), dim3(256), 0, s, ev[2], ev[3], 0,
                              a2, (const float*)h_buf, (float*)nullptr);
        break;
    case EO_W_BF16: run_mfma<EO_W_BF16>(a1, a2, tiles, I, H, s, ev); break;
    case EO_W_FP8: run_mfma<EO_W_FP8>(a1, a2, tiles, I, H, s, ev); break;
    case EO_W_MXFP4: run_mfma<EO_W_MXFP4>(a1, a2, tiles, I, H, s, ev); break;
    case EO_W_NVFP4: run_mfma<EO_W_NVFP4>(a1, a2, tiles, I, H, s, ev); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace eo
