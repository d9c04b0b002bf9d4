/* Runs the CPU oracle (compiled into this driver) on tiny random inputs over
 * many shapes and parameter settings, under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every buffer the oracle touches is exactly the
 * size its callers allocate. */
#include <stdio.h>

#include "../../oracle/fsl_oracle.c"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) / 9007199254740992.0;
}

int main(void) {
    int runs = 0, bad = 0;
    const int64_t Ns[] = {1, 2, 7, 40, 133, 257};
    const int32_t ws[] = {1, 5, 16, 300};
    const int32_t Ps[] = {-1, 0, 3};
    for (size_t a = 0; a < sizeof(Ns) / sizeof(Ns[0]); ++a)
        for (size_t b = 0; b < sizeof(ws) / sizeof(ws[0]); ++b)
            for (size_t c = 0; c < sizeof(Ps) / sizeof(Ps[0]); ++c)
                for (int32_t K = 1; K <= 3; K += 2) {
                    orc_head p;
                    memset(&p, 0, sizeof(p));
                    p.N = Ns[a]; p.d = 8; p.w = ws[b]; p.s = 4; p.P = Ps[c]; p.W = 2; p.K = K; p.B = 8;
                    p.scale = 0.35; p.rho = 1.0; p.rope_base = 10000.0; p.rms_eps = 1e-6;
                    p.sigma = 4.0; p.lambda = 1.0; p.gamma = 0.5;
                    const int64_t n = p.N * p.d;
                    float *q = malloc(sizeof(float) * n), *k = malloc(sizeof(float) * n), *v = malloc(sizeof(float) * n);
                    for (int64_t i = 0; i < n; ++i) {
                        q[i] = (float)(uniform() * 2 - 1);
                        k[i] = (float)(uniform() * 2 - 1);
                        v[i] = (float)(uniform() * 2 - 1);
                    }
                    const int64_t R = p.N;
                    int64_t *rows = malloc(sizeof(int64_t) * R);
                    for (int64_t i = 0; i < R; ++i) rows[i] = i;
                    double *out = malloc(sizeof(double) * R * p.d), *ow = malloc(sizeof(double) * R * p.d);
                    double *ol = malloc(sizeof(double) * R * p.d), *margin = malloc(sizeof(double) * R);
                    int32_t *sel = malloc(sizeof(int32_t) * R * p.K);
                    const int64_t C = orc_num_cells(&p) > 0 ? orc_num_cells(&p) : 1;
                    const int64_t nblk = orc_num_blocks(&p);
                    const int32_t cap = p.P < 0 ? (int32_t)C : p.P + p.W;
                    int32_t *pool = malloc(sizeof(int32_t) * nblk * cap);
                    float *kbar = malloc(sizeof(float) * C * p.d), *amax = malloc(sizeof(float) * C);
                    const int rc = orc_forward_head(q, k, v, &p, rows, R, out, ow, ol, sel, margin, pool, cap, kbar,
                                                    amax, 1);
                    if (rc != 0) ++bad;
                    for (int64_t i = 0; i < R * p.d; ++i)
                        if (out[i] != out[i]) ++bad;  /* NaN */
                    free(q); free(k); free(v); free(rows); free(out); free(ow); free(ol); free(margin); free(sel);
                    free(pool); free(kbar); free(amax);
                    ++runs;
                }
    printf("oracle driver: %d shapes, %d failures\n", runs, bad);
    return bad == 0 ? 0 : 1;
}
