/*
 * Host sanitizer driver for the fp64 oracle (test infrastructure): every
 * entry point of orthros_oracle.c on small random inputs and on its edge
 * cases (one row, a window of one, windows above the length, row samples,
 * uneven head maps, an incremental cache filled to capacity, rejected
 * arguments). Built with AddressSanitizer and UndefinedBehaviorSanitizer;
 * any out-of-bounds access, use after free or undefined operation aborts
 * the run. It also checks that every weight row sums to one and that the
 * outputs are finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_swa(int B, int T, int Hq, int Hkv, int D, int64_t W,
               const int32_t *head_map, const double *q_pre,
               const double *alpha, const double *beta, const double *k,
               const double *v, double *o, double *lse, int64_t n_sel,
               const int64_t *rows_sel);
int oracle_xattn(int B, int T_in, int T_out, int Hq, int Hkv, int D,
                 const int32_t *head_map, const double *qx_pre,
                 const double *alpha_x, const double *beta_x, const double *k,
                 const double *v, double *o_x, double *lse, int64_t n_sel,
                 const int64_t *rows_sel);
int oracle_row_weights(int T, int Hkv, int D, int64_t t, int64_t W, int g,
                       const double *q_pre_row, const double *alpha_h,
                       const double *beta_h, const double *k, const double *v,
                       double *weights_out);
void *oracle_cache_new(int B, int Hkv, int D, int64_t cap);
void oracle_cache_free(void *p);
int64_t oracle_cache_len(const void *p, int b);
int oracle_cache_append(void *p, int n, const double *k_new,
                        const double *v_new);
int oracle_cache_decode_pair(void *p, int Hq, int64_t W,
                             const int32_t *head_map, const double *q_pre,
                             const double *qx_pre, const double *alpha,
                             const double *beta, const double *alpha_x,
                             const double *beta_x, const double *k_new,
                             const double *v_new, double *o, double *o_x);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
/* Exactly-sized heap arrays, so that the sanitizer sees any overrun. */
static double *arr(size_t n) {
    double *p = (double *)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = urand();
    return p;
}

static int failures = 0;
#define CHECK(c, ...) do { if (!(c)) { ++failures; \
    fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
    fprintf(stderr, __VA_ARGS__); fprintf(stderr, "\n"); } } while (0)

static void all_finite(const double *p, size_t n, const char *what) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) { CHECK(0, "%s[%zu] not finite", what, i); return; }
}

static void batched_case(int B, int T, int Hq, int Hkv, int D, int64_t W,
                         const int32_t *map) {
    double *q = arr((size_t)B * T * Hq * D), *k = arr((size_t)B * T * Hkv * D);
    double *v = arr((size_t)B * T * Hkv * D), *a = arr((size_t)Hq * D);
    double *b = arr((size_t)Hq * D), *o = arr((size_t)B * T * Hq * D);
    double *lse = arr((size_t)B * T * Hq);
    CHECK(oracle_swa(B, T, Hq, Hkv, D, W, map, q, a, b, k, v, o, lse, 0, NULL) == 0,
          "swa B=%d T=%d W=%lld", B, T, (long long)W);
    all_finite(o, (size_t)B * T * Hq * D, "swa o");
    /* a row sample: compact outputs */
    int64_t rows[6] = {0, 0, B - 1, T - 1, 0, T / 2};
    double *os = arr(3 * (size_t)Hq * D), *ls = arr(3 * (size_t)Hq);
    CHECK(oracle_swa(B, T, Hq, Hkv, D, W, map, q, a, b, k, v, os, ls, 3, rows) == 0,
          "swa rows");
    /* output stream: every T_out from 1 to T */
    for (int T_out = 1; T_out <= T; T_out += (T_out < 3 ? 1 : T / 3 + 1)) {
        int T_in = T - T_out;
        double *qx = arr((size_t)B * T_out * Hq * D);
        double *ox = arr((size_t)B * T_out * Hq * D), *lx = arr((size_t)B * T_out * Hq);
        CHECK(oracle_xattn(B, T_in, T_out, Hq, Hkv, D, map, qx, a, b, k, v, ox,
                           lx, 0, NULL) == 0, "xattn T_out=%d", T_out);
        all_finite(ox, (size_t)B * T_out * Hq * D, "xattn o");
        free(qx); free(ox); free(lx);
    }
    /* weights of single rows sum to one over exactly their range */
    double *w = arr((size_t)T);
    for (int64_t t = 0; t < T; t += (T > 8 ? T / 8 : 1)) {
        int g = map ? map[0] : 0;
        CHECK(oracle_row_weights(T, Hkv, D, t, W, g, q, a, b, k, v, w) == 0, "weights");
        double s = 0.0;
        int64_t lo = (t - W + 1 > 0) ? t - W + 1 : 0;
        for (int64_t j = 0; j < T; ++j) {
            s += w[j];
            if (j < lo || j > t) CHECK(w[j] == 0.0, "weight outside the range");
        }
        CHECK(fabs(s - 1.0) < 1e-12, "weights sum %g", s);
    }
    free(q); free(k); free(v); free(a); free(b); free(o); free(lse);
    free(os); free(ls); free(w);
}

static void cache_case(int B, int Hkv, int Hq, int D, int T0, int steps,
                       int64_t W, const int32_t *map) {
    int64_t cap = T0 + steps;
    void *c = oracle_cache_new(B, Hkv, D, cap);
    CHECK(c != NULL, "cache_new");
    double *k0 = arr((size_t)B * T0 * Hkv * D), *v0 = arr((size_t)B * T0 * Hkv * D);
    CHECK(oracle_cache_append(c, T0, k0, v0) == 0, "append");
    double *a = arr((size_t)Hq * D), *b = arr((size_t)Hq * D);
    for (int s = 0; s < steps; ++s) {
        double *q = arr((size_t)B * Hq * D), *qx = arr((size_t)B * Hq * D);
        double *kn = arr((size_t)B * Hkv * D), *vn = arr((size_t)B * Hkv * D);
        double *o = arr((size_t)B * Hq * D), *ox = arr((size_t)B * Hq * D);
        CHECK(oracle_cache_decode_pair(c, Hq, W, map, q, qx, a, b, a, b, kn, vn,
                                       o, ox) == 0, "decode step %d", s);
        all_finite(o, (size_t)B * Hq * D, "decode o");
        all_finite(ox, (size_t)B * Hq * D, "decode o_x");
        free(q); free(qx); free(kn); free(vn); free(o); free(ox);
    }
    for (int bb = 0; bb < B; ++bb) CHECK(oracle_cache_len(c, bb) == cap, "length");
    CHECK(oracle_cache_len(c, B) == -1, "length out of range");
    /* full: one more append is rejected and changes nothing */
    double *kn = arr((size_t)B * Hkv * D), *vn = arr((size_t)B * Hkv * D);
    CHECK(oracle_cache_append(c, 1, kn, vn) != 0, "append past capacity");
    CHECK(oracle_cache_len(c, 0) == cap, "length after rejection");
    free(kn); free(vn); free(k0); free(v0); free(a); free(b);
    oracle_cache_free(c);
}

int main(void) {
    int32_t uneven[6] = {0, 0, 0, 1, 2, 2};
    batched_case(1, 1, 2, 2, 8, 1, NULL);       /* one row */
    batched_case(2, 17, 4, 2, 16, 1, NULL);     /* window of one */
    batched_case(1, 33, 4, 1, 8, 5, NULL);
    batched_case(2, 20, 4, 2, 8, 64, NULL);     /* window above T */
    batched_case(1, 24, 6, 3, 8, 7, uneven);
    cache_case(2, 2, 4, 8, 5, 9, 3, NULL);
    cache_case(1, 3, 6, 16, 1, 4, 100, uneven);
    /* rejected arguments return an error and touch nothing */
    double *x = arr(64);
    int32_t bad[2] = {0, 3};
    CHECK(oracle_swa(1, 4, 2, 2, 4, 0, NULL, x, x, x, x, x, x, x, 0, NULL) != 0, "W=0");
    CHECK(oracle_swa(1, 4, 2, 2, 4, 2, bad, x, x, x, x, x, x, x, 0, NULL) != 0, "map");
    CHECK(oracle_swa(1, 4, 3, 2, 4, 2, NULL, x, x, x, x, x, x, x, 0, NULL) != 0,
          "Hq not a multiple of Hkv");
    CHECK(oracle_xattn(1, 2, 0, 2, 2, 4, NULL, x, x, x, x, x, x, x, 0, NULL) != 0,
          "T_out=0");
    int64_t out_of_range[2] = {0, 4};
    CHECK(oracle_swa(1, 4, 2, 2, 4, 2, NULL, x, x, x, x, x, x, x, 1,
                     out_of_range) != 0, "row out of range");
    CHECK(oracle_row_weights(4, 2, 4, 4, 2, 0, x, x, x, x, x, x) != 0, "t=T");
    CHECK(oracle_cache_new(0, 1, 1, 1) == NULL, "empty cache");
    free(x);
    if (failures) { fprintf(stderr, "%d failures\n", failures); return 1; }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
