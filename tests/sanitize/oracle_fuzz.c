/* Randomised driver for the CPU oracle's C part (oracle/q8.c), built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers_cpu.py: ragged sizes, every grad dtype, both
 * rounding modes, the carrier, group sums and the scale pass.  Any
 * out-of-bounds access or undefined behaviour aborts; the driver checks the
 * quantiser's range invariants on the way. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void or_q8_update_ex(int8_t *codes, float *absmax, void *grad, int dtype, int64_t numel, float beta,
                     double *block_sumsq, int rounding, uint64_t seed, uint32_t offset, uint32_t tensor);
void or_q8_update_carrier(int8_t *codes, float *absmax, const void *grad, int dtype, int64_t numel, float beta,
                          uint8_t *payload, uint8_t *scales, double *block_sumsq);
void or_group_sums(const double *block_sumsq, const int32_t *block_group, int64_t nblk, int32_t ngroups,
                   double *group_sums);
void or_group_inv_norm(const double *group_sums, int32_t ngroups, float eps, float *inv);
void or_scale_by_group(void *grad, int dtype, int64_t numel, const int32_t *block_group, const float *inv);
void or_round_array(const float *src, int64_t n, int dtype, uint16_t *dst);
void or_widen_array(const uint16_t *src, int64_t n, int dtype, float *dst);

static uint64_t s = 88172645463325252ull;
static uint64_t next(void) { s ^= s << 13; s ^= s >> 7; s ^= s << 17; return s; }
static double unif(void) { return (double)(next() >> 11) * 0x1p-53; }

int main(int argc, char **argv) {
    const int iters = argc > 1 ? atoi(argv[1]) : 300;
    int fails = 0;
    for (int it = 0; it < iters; it++) {
        const int64_t n = (it % 7 == 0) ? 1 + (int64_t)(next() % 300) : 1 + (int64_t)(next() % 6000);
        const int dt = (int)(next() % 3);            /* 0 f32, 1 bf16, 2 f16 */
        const int64_t nblk = (n + 255) / 256;
        int8_t *codes = malloc((size_t)n);
        float *absmax = malloc((size_t)nblk * 4);
        double *sums = malloc((size_t)nblk * 8);
        float *gf = malloc((size_t)n * 4);
        void *grad = malloc((size_t)n * (dt == 0 ? 4 : 2));
        for (int64_t i = 0; i < n; i++) {
            codes[i] = (int8_t)((int)(next() % 255) - 127);
            gf[i] = (float)((unif() - 0.5) * 2e-3 * (next() % 50 == 0 ? 1e4 : 1.0));
        }
        for (int64_t b = 0; b < nblk; b++) absmax[b] = (float)(1e-4 + unif() * 1e-2) * (next() % 40 == 0 ? 0.0f : 1.0f);
        if (dt == 0) memcpy(grad, gf, (size_t)n * 4);
        else or_round_array(gf, n, dt, grad);
        const int rounding = (int)(next() % 2);
        const float beta = (next() % 10 == 0) ? (float)(next() % 2) : 0.95f;
        or_q8_update_ex(codes, absmax, grad, dt, n, beta, sums, rounding, next(), (uint32_t)it, (uint32_t)(it % 5));
        for (int64_t i = 0; i < n; i++)
            if (codes[i] < -127 || codes[i] > 127) fails++;
        for (int64_t b = 0; b < nblk; b++)
            if (!(absmax[b] >= 0.0f) || !(sums[b] >= 0.0)) fails++;
        /* groups: a random assignment of blocks, then norms and the scale pass */
        const int32_t ng = 1 + (int32_t)(next() % 4);
        int32_t *bg = malloc((size_t)nblk * 4);
        for (int64_t b = 0; b < nblk; b++) bg[b] = (int32_t)(b < ng ? b : (int64_t)(next() % (uint64_t)ng));
        double *gs = malloc((size_t)ng * 8);
        float *inv = malloc((size_t)ng * 4);
        or_group_sums(sums, bg, nblk, ng, gs);
        or_group_inv_norm(gs, ng, 1e-7f, inv);
        or_scale_by_group(grad, dt, n, bg, inv);
        if (dt != 0) or_widen_array(grad, n, dt, gf);
        /* the carrier needs a multiple of 32 elements */
        const int64_t nc = n / 32 * 32;
        if (nc > 0) {
            uint8_t *payload = malloc((size_t)nc);
            uint8_t *scales = malloc((size_t)nc / 32);
            const int64_t nbc = (nc + 255) / 256;
            or_q8_update_carrier(codes, absmax, grad, dt, nc, 0.9f, payload, scales, sums);
            for (int64_t b = 0; b < nbc; b++)
                if (!(absmax[b] >= 0.0f)) fails++;
            free(payload);
            free(scales);
        }
        free(codes); free(absmax); free(sums); free(gf); free(grad); free(bg); free(gs); free(inv);
    }
    printf("oracle_fuzz: %d iterations, %d failed checks\n", iters, fails);
    return fails ? 1 : 0;
}
