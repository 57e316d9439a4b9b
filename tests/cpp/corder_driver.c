/* Test driver for the oracle's fixed-order router logits (CPU only):
 *   corder_driver <T> <E> <H>
 * fills x and R with small integers, so that every partial sum is an exact
 * fp32 integer, runs oracle_router_logits and checks each logit against the
 * exact integer dot product. Prints "ok". */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_router_logits(const float* x, const float* R, int64_t T, int64_t E, int64_t H,
                          float* z);

int main(int argc, char** argv) {
    if (argc < 4) return 2;
    const int64_t T = atoll(argv[1]), E = atoll(argv[2]), H = atoll(argv[3]);
    float* x = malloc(sizeof(float) * T * H);
    float* R = malloc(sizeof(float) * E * H);
    float* z = malloc(sizeof(float) * T * E);
    if (!x || !R || !z) return 2;
    for (int64_t i = 0; i < T * H; ++i) x[i] = (float)((i * 7 + 3) % 17 - 8);
    for (int64_t i = 0; i < E * H; ++i) R[i] = (float)((i * 5 + 1) % 13 - 6);
    oracle_router_logits(x, R, T, E, H, z);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t e = 0; e < E; ++e) {
            int64_t s = 0;
            for (int64_t h = 0; h < H; ++h) s += (int64_t)x[t * H + h] * (int64_t)R[e * H + h];
            if (z[t * E + e] != (float)s) {
                printf("mismatch at t %lld e %lld: %g vs %lld\n", (long long)t, (long long)e,
                       z[t * E + e], (long long)s);
                return 1;
            }
        }
    free(x);
    free(R);
    free(z);
    printf("ok\n");
    return 0;
}
