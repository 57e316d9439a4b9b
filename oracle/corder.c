/*
 * ORACLE (test infrastructure only; never part of the product path).
 *
 * Router logits z[t,e] = sum_h x[t,h] * R[e,h] in fp32, accumulated in one
 * fixed order so that the top-k choice made from them is reproducible bit for
 * bit on any device that follows the same order:
 *   - 64 partial sums p_i (i = 0..63): p_i starts at +0.0f and takes the terms
 *     h = i, i+64, i+128, ... in ascending order, each as one fused
 *     multiply-add (a single rounding per term);
 *   - then for s = 32, 16, 8, 4, 2, 1: p_i <- p_i + p_(i xor s) for every i;
 *   - z = p_0.
 * The pages leave the accumulation order open (routing is named only as an
 * axis on which MoE architectures differ: papers.ananclaw.com explainer,
 * "core method" section 4; zhichai.net article, section 2, the LRU paragraph).
 * This order is the reading used for bit-exact top-k.
 *
 * Built with gcc -O2 and -ffp-contract=off: the only fused operations are the
 * explicit fmaf calls, and there is no reassociation.
 */
#include <math.h>
#include <stdint.h>

void oracle_router_logits(const float* x, const float* R, int64_t T, int64_t E, int64_t H,
                          float* z) {
    for (int64_t t = 0; t < T; ++t) {
        const float* xt = x + t * H;
        for (int64_t e = 0; e < E; ++e) {
            const float* re = R + e * H;
            float p[64], q[64];
            for (int i = 0; i < 64; ++i) {
                float acc = 0.0f;
                for (int64_t h = i; h < H; h += 64) acc = fmaf(xt[h], re[h], acc);
                p[i] = acc;
            }
            for (int s = 32; s >= 1; s >>= 1) {
                for (int i = 0; i < 64; ++i) q[i] = p[i] + p[i ^ s];
                for (int i = 0; i < 64; ++i) p[i] = q[i];
            }
            z[t * E + e] = p[0];
        }
    }
}
