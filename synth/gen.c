/*
 * Seeded synthetic inputs for the MoE expert-offload layer: expert weights
 * packed into the pool's expert-block layout, router weights and activations.
 *
 * This file is input generation only. It holds none of the layer's own
 * arithmetic (no routing, no dequantisation, no FFN): both the HIP library and
 * the CPU oracle consume the bytes written here and decode them with their own,
 * independent code.
 *
 * Random numbers: Philox4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11), written
 * from its published definition. Normals come from the inverse normal CDF
 * (Acklam's rational approximation) of one uniform each.
 *
 * Expert block layout (one routed or shared expert, hidden H, intermediate I):
 *   W13 = [W_gate ; W_up], 2I rows of H elements (row r < I is gate row r,
 *   row I + r is up row r); W2 = W_down, H rows of I elements. Quantisation
 *   blocks run along each row (the contraction axis K).
 *     fp32 : W13 f32 [2I,H] | W2 f32 [H,I]
 *     bf16 : W13 bf16 [2I,H] | W2 bf16 [H,I]
 *     mxfp4: W13 e2m1 [2I,H/2] | W2 e2m1 [H,I/2] | W13 e8m0 [2I,H/32] | W2 e8m0 [H,I/32]
 *     nvfp4: W13 e2m1 [2I,H/2] | W2 e2m1 [H,I/2] | W13 e4m3 [2I,H/16] | W2 e4m3 [H,I/16]
 *            | f32 global scales g_gate, g_up, g_down
 *     fp8  : W13 e4m3 [2I,H] | W2 e4m3 [H,I] | W13 f32 row scale [2I] | W2 f32 row scale [H]
 *   Two fp4 codes share a byte, the even element in the low nibble.
 *
 * Single-threaded: callers parallelise over experts (ctypes releases the GIL),
 * so no thread team lingers after generation.
 *
 * Quantisers (generator side, round-half-to-even, saturating):
 *   mxfp4: shared exponent floor(log2 amax_block) - 2 (OCP MX v1.0), stored as e8m0.
 *   nvfp4: g = amax_tensor / (448*6); block scale e4m3(amax_block / (6 g)).
 *   fp8  : per-row scale amax_row / 448, elements e4m3fn.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { FMT_FP32 = 0, FMT_BF16 = 1, FMT_MXFP4 = 2, FMT_NVFP4 = 3, FMT_FP8 = 4 };

/* ---------------------------------------------------------------- Philox */
static void philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += W0; k1 += W1; }
        uint64_t p0 = (uint64_t)M0 * c0;
        uint64_t p1 = (uint64_t)M1 * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

void synth_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out) {
    philox4x32_10(ctr, key, out);
}

/* Inverse of the standard normal CDF: P. J. Acklam's rational approximation
 * (relative error below 1.2e-9), central region and tails. */
static double inv_norm_cdf(double p) {
    static const double a[6] = {-3.969683028665376e+01, 2.209460984245205e+02,
                                -2.759285104469687e+02, 1.383577518672690e+02,
                                -3.066479806614716e+01, 2.506628277459239e+00};
    static const double b[5] = {-5.447609879822406e+01, 1.615858368580409e+02,
                                -1.556989798598866e+02, 6.680131188771972e+01,
                                -1.328068155288572e+01};
    static const double c[6] = {-7.784894002430293e-03, -3.223964580411365e-01,
                                -2.400758277161838e+00, -2.549732539343734e+00,
                                4.374664141464968e+00, 2.938163982698783e+00};
    static const double d[4] = {7.784695709041462e-03, 3.224671290700398e-01,
                                2.445134137142996e+00, 3.754408661907416e+00};
    const double plow = 0.02425;
    if (p < plow) {
        double q = sqrt(-2.0 * log(p));
        return (((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
               ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1.0);
    }
    if (p > 1.0 - plow) {
        double q = sqrt(-2.0 * log(1.0 - p));
        return -(((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
               ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1.0);
    }
    double q = p - 0.5, r = q * q;
    return (((((a[0] * r + a[1]) * r + a[2]) * r + a[3]) * r + a[4]) * r + a[5]) * q /
           (((((b[0] * r + b[1]) * r + b[2]) * r + b[3]) * r + b[4]) * r + 1.0);
}

/* Element i of stream (seed, purpose, c1, c2, c3): word i%4 of Philox block i/4
 * with counter {i/4, c1, c2, c3} and key {seed, purpose}, as a uniform in (0,1)
 * (32-bit grid, offset by half a step), mapped through the inverse normal CDF. */
static void normal_block(uint32_t seed, uint32_t purpose, uint32_t c1, uint32_t c2, uint32_t c3,
                         uint32_t blk, float z[4]) {
    uint32_t ctr[4] = {blk, c1, c2, c3}, key[2] = {seed, purpose}, w[4];
    philox4x32_10(ctr, key, w);
    for (int j = 0; j < 4; ++j) z[j] = (float)inv_norm_cdf(((double)w[j] + 0.5) * (1.0 / 4294967296.0));
}

static void normal_fill(uint32_t seed, uint32_t purpose, uint32_t c1, uint32_t c2, uint32_t c3,
                        double sigma, int64_t n, float* out) {
    int64_t nblk = (n + 3) / 4;
    for (int64_t b = 0; b < nblk; ++b) {
        float z[4];
        normal_block(seed, purpose, c1, c2, c3, (uint32_t)b, z);
        for (int j = 0; j < 4; ++j) {
            int64_t i = 4 * b + j;
            if (i < n) out[i] = (float)(sigma * (double)z[j]);
        }
    }
}

void synth_normal_f32(uint32_t seed, uint32_t purpose, uint32_t c1, uint32_t c2, uint32_t c3,
                      double sigma, int64_t n, float* out) {
    normal_fill(seed, purpose, c1, c2, c3, sigma, n, out);
}

/* ------------------------------------------------------------ casting */
static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

void synth_f32_to_bf16(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

/* Round a >= 0 to the grid of a minifloat with `mbits` mantissa bits and
 * smallest normal exponent `emin`, half to even, saturating at maxv. */
static double round_minifloat(double a, int mbits, int emin, double maxv) {
    if (!(a > 0.0)) return 0.0;
    int e;
    frexp(a, &e);
    e -= 1; /* a in [2^e, 2^(e+1)) */
    if (e < emin) e = emin;
    double quantum = ldexp(1.0, e - mbits);
    double q = nearbyint(a / quantum) * quantum;
    return q > maxv ? maxv : q;
}

/* Bit pattern (without sign) of a grid value q >= 0. */
static uint32_t encode_minifloat(double q, int mbits, int emin, int bias) {
    if (q == 0.0) return 0;
    int e;
    frexp(q, &e);
    e -= 1;
    if (e < emin) return (uint32_t)(q / ldexp(1.0, emin - mbits));
    uint32_t mant = (uint32_t)(q / ldexp(1.0, e - mbits)) - (1u << mbits);
    return ((uint32_t)(e + bias) << mbits) | mant;
}

/* e2m1 code of v (already divided by its scale), round half to even, saturating:
 * the midpoints of 0, .5, 1, 1.5, 2, 3, 4, 6 are .25, .75, 1.25, 1.75, 2.5, 3.5, 5;
 * a tie goes to the even code (0, 1.0, 2.0, 4.0), hence > before odd codes and
 * >= before even ones. */
static uint8_t e2m1_code(double v) {
    double m = fabs(v);
    uint32_t c = (m > 0.25) + (m >= 0.75) + (m > 1.25) + (m >= 1.75) + (m > 2.5) + (m >= 3.5) +
                 (m > 5.0);
    return (uint8_t)((signbit(v) ? 0x8u : 0u) | c);
}

static uint8_t e4m3_code(double v) {
    double q = round_minifloat(fabs(v), 3, -6, 448.0);
    return (uint8_t)((signbit(v) ? 0x80u : 0u) | encode_minifloat(q, 3, -6, 7));
}

static double e4m3_value_pos(uint8_t c) { /* positive codes only, generator use */
    int ex = (c >> 3) & 0xF, m = c & 7;
    if (ex == 0) return ldexp((double)m, -9);
    return ldexp(1.0 + m / 8.0, ex - 7);
}

uint8_t synth_e2m1_encode(double v) { return e2m1_code(v); }
uint8_t synth_e4m3_encode(double v) { return e4m3_code(v); }

/* ------------------------------------------------------ expert blocks */
uint64_t synth_expert_bytes(int32_t H, int32_t I, int32_t fmt) {
    uint64_t n13 = 2ull * I * H, n2 = (uint64_t)H * I;
    switch (fmt) {
    case FMT_FP32: return 4 * (n13 + n2);
    case FMT_BF16: return 2 * (n13 + n2);
    case FMT_MXFP4: return (n13 + n2) / 2 + (n13 + n2) / 32;
    case FMT_NVFP4: return (n13 + n2) / 2 + (n13 + n2) / 16 + 12;
    case FMT_FP8: return (n13 + n2) + 4ull * (2ull * I + H);
    default: return 0;
    }
}

static float amax_f32(const float* v, int64_t n) {
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > m) m = a;
    }
    return m;
}

/* Quantise `rows` rows of length K (fp32, row-major) into `data` and `scales`
 * according to fmt. `g` is the tensor's nvfp4 global scale. */
static void quantise_rows(const float* w, int64_t rows, int64_t K, int fmt, float g,
                          uint8_t* data, uint8_t* scales) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* row = w + r * K;
        if (fmt == FMT_FP32) {
            memcpy(data + r * K * 4, row, (size_t)K * 4);
        } else if (fmt == FMT_BF16) {
            uint16_t* o = (uint16_t*)(data + r * K * 2);
            for (int64_t i = 0; i < K; ++i) o[i] = f32_to_bf16_rne(row[i]);
        } else if (fmt == FMT_MXFP4) {
            uint8_t* o = data + r * (K / 2);
            for (int64_t b = 0; b < K / 32; ++b) {
                float amax = amax_f32(row + 32 * b, 32);
                int se = -127;
                if (amax > 0.0f) {
                    int e;
                    frexp((double)amax, &e);
                    se = (e - 1) - 2;
                }
                if (se < -127) se = -127;
                if (se > 127) se = 127;
                scales[r * (K / 32) + b] = (uint8_t)(se + 127);
                const double inv = ldexp(1.0, -se); /* exact power of two */
                for (int i = 0; i < 32; i += 2) {
                    uint8_t lo = e2m1_code((double)row[32 * b + i] * inv);
                    uint8_t hi = e2m1_code((double)row[32 * b + i + 1] * inv);
                    o[(32 * b + i) / 2] = (uint8_t)(lo | (hi << 4));
                }
            }
        } else if (fmt == FMT_NVFP4) {
            uint8_t* o = data + r * (K / 2);
            for (int64_t b = 0; b < K / 16; ++b) {
                float amax = amax_f32(row + 16 * b, 16);
                uint8_t sc = (g > 0.0f) ? e4m3_code((double)amax / (6.0 * (double)g)) : 0;
                scales[r * (K / 16) + b] = sc;
                double den = e4m3_value_pos(sc) * (double)g;
                for (int i = 0; i < 16; i += 2) {
                    double a = row[16 * b + i], c = row[16 * b + i + 1];
                    uint8_t lo = den > 0.0 ? e2m1_code(a / den) : 0;
                    uint8_t hi = den > 0.0 ? e2m1_code(c / den) : 0;
                    o[(16 * b + i) / 2] = (uint8_t)(lo | (hi << 4));
                }
            }
        } else if (fmt == FMT_FP8) {
            float amax = amax_f32(row, K);
            float s = (float)((double)amax / 448.0);
            memcpy(scales + r * 4, &s, 4);
            for (int64_t i = 0; i < K; ++i)
                data[r * K + i] = s > 0.0f ? e4m3_code((double)row[i] / (double)s) : 0;
        }
    }
}

/* Pack float weights (gate [I,H], up [I,H], down [H,I]) into one expert block. */
int synth_pack_expert(const float* wg, const float* wu, const float* wd, int32_t H, int32_t I,
                      int32_t fmt, uint8_t* out, uint64_t out_bytes) {
    uint64_t need = synth_expert_bytes(H, I, fmt);
    if (need == 0 || out_bytes < need) return -1;
    if ((fmt == FMT_MXFP4 && (H % 32 || I % 32)) || (fmt == FMT_NVFP4 && (H % 16 || I % 16)))
        return -2;
    int64_t n1 = (int64_t)I * H, n2 = (int64_t)H * I;
    uint64_t d13, d2, s13 = 0, s2 = 0, gl = 0;
    switch (fmt) {
    case FMT_FP32: d13 = 0; d2 = 8ull * n1; break;
    case FMT_BF16: d13 = 0; d2 = 4ull * n1; break;
    case FMT_MXFP4: d13 = 0; d2 = (uint64_t)n1; s13 = d2 + n2 / 2; s2 = s13 + 2 * n1 / 32; break;
    case FMT_NVFP4:
        d13 = 0; d2 = (uint64_t)n1; s13 = d2 + n2 / 2; s2 = s13 + 2 * n1 / 16;
        gl = s2 + n2 / 16; break;
    case FMT_FP8: d13 = 0; d2 = 2ull * n1; s13 = d2 + n2; s2 = s13 + 4ull * 2 * I; break;
    default: return -1;
    }
    float gg = 0, gu = 0, gd = 0;
    if (fmt == FMT_NVFP4) {
        gg = (float)((double)amax_f32(wg, n1) / (448.0 * 6.0));
        gu = (float)((double)amax_f32(wu, n1) / (448.0 * 6.0));
        gd = (float)((double)amax_f32(wd, n2) / (448.0 * 6.0));
        float gs[3] = {gg, gu, gd};
        memcpy(out + gl, gs, 12);
    }
    /* bytes per element of the data section, times 2 for the nibble formats */
    uint64_t row_bytes_h; /* data bytes of one H-long row */
    uint64_t srow_h = 0;  /* scale bytes of one H-long row */
    switch (fmt) {
    case FMT_FP32: row_bytes_h = 4ull * H; break;
    case FMT_BF16: row_bytes_h = 2ull * H; break;
    case FMT_MXFP4: row_bytes_h = H / 2; srow_h = H / 32; break;
    case FMT_NVFP4: row_bytes_h = H / 2; srow_h = H / 16; break;
    default: row_bytes_h = H; srow_h = 4; break;
    }
    quantise_rows(wg, I, H, fmt, gg, out + d13, out + s13);
    quantise_rows(wu, I, H, fmt, gu, out + d13 + (uint64_t)I * row_bytes_h,
                  out + s13 + (uint64_t)I * srow_h);
    quantise_rows(wd, H, I, fmt, gd, out + d2, out + s2);
    return 0;
}

/* Generate one expert's N(0, sigma) fp32 weights from the stream
 * (seed, purpose, tensor, layer, expert) and pack them. */
int synth_expert_block(uint32_t seed, uint32_t purpose, int32_t layer, int32_t expert, int32_t H,
                       int32_t I, int32_t fmt, double sigma, uint8_t* out, uint64_t out_bytes) {
    int64_t n1 = (int64_t)I * H;
    float* w = (float*)malloc(sizeof(float) * 3 * (size_t)n1);
    if (!w) return -3;
    for (int t = 0; t < 3; ++t)
        normal_fill(seed, purpose, (uint32_t)t, (uint32_t)layer, (uint32_t)expert, sigma, n1,
                    w + t * n1);
    int rc = synth_pack_expert(w, w + n1, w + 2 * n1, H, I, fmt, out, out_bytes);
    free(w);
    return rc;
}

/* Same, and also return the unquantised fp32 weights (gate, up, down). */
int synth_expert_block_f32(uint32_t seed, uint32_t purpose, int32_t layer, int32_t expert,
                           int32_t H, int32_t I, int32_t fmt, double sigma, uint8_t* out,
                           uint64_t out_bytes, float* w_out) {
    int64_t n1 = (int64_t)I * H;
    for (int t = 0; t < 3; ++t)
        normal_fill(seed, purpose, (uint32_t)t, (uint32_t)layer, (uint32_t)expert, sigma, n1,
                    w_out + t * n1);
    return synth_pack_expert(w_out, w_out + n1, w_out + 2 * n1, H, I, fmt, out, out_bytes);
}
