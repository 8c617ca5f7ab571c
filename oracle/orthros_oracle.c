/*
 * Plain fp64 CPU oracle for Orthros attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or
 * calls this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do. It shares no code, header, table or helper with the
 * HIP library.
 *
 * What it computes (pages: "Orthros: Phase-Aware Heterogeneous Attention for
 * Efficient Transformers", paper text §3.1, the definitions of q_i, q'_i,
 * k_i, v_i and the two output equations for o_t and o'_t; the same two
 * equations appear in the paper-notes page of the same title, key design 1
 * and 2, and in the reproduction note "Orthros：阶段异构注意力", core formulas):
 *
 *   q_t  = alpha  (.) q_pre_t + beta           every base row t
 *   q'_t = alpha' (.) qx_pre_t + beta'         output rows only
 *   o_t  = sum_{j=lo(t)}^{t} softmax_j(q_t . k_j / sqrt(D)) v_j,
 *          lo(t) = max(0, t - W + 1)           (0-based form of max(1,t-w+1))
 *   o'_t = sum_{j=0}^{t} softmax_j(q'_t . k_j / sqrt(D)) v_j
 *
 * The output rows are the last T_out positions, t = T_in + r (paper text
 * §3.1: output sequence indices T_in+1..T in 1-based form).
 *
 * Readings where the pages leave a step open:
 *  - D in sqrt(D) is the per-head dimension.
 *  - alpha/beta hold one value per channel of the full Hq*D query projection.
 *  - GQA: q head h reads KV head head_map[h] (default h / (Hq/Hkv)).
 *  - Decode (paper text §3.2, Decoding): the new base token's K/V is
 *    appended first, then both queries attend; the base query therefore
 *    sees its own key.
 *
 * Each row is evaluated the plain way: scores for every key in range, the
 * row maximum, exponentials, their sum, then the weighted sum of values.
 * Two passes, no online rescaling, no tiling.
 *
 * Layouts (all row-major, contiguous, fp64):
 *   q_pre  [B, nrows, Hq, D]       k, v  [B, T, Hkv, D]  (projection layout)
 *   o      [B, nrows, Hq, D]       lse   [B, nrows, Hq]   (natural log)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* One query row against keys lo..hi (inclusive) of one KV head.
 * kv_stride is the element distance between consecutive keys. */
static int attend_row(const double *q_pre, const double *alpha,
                      const double *beta, const double *k, const double *v,
                      int64_t kv_stride, int D, int64_t lo, int64_t hi,
                      double *o, double *lse, double *weights)
{
    int64_t n = hi - lo + 1;
    double *q = (double *)malloc(sizeof(double) * (size_t)D);
    double *s = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!q || !s) { free(q); free(s); return -1; }

    /* Scale-offset affine on the projected query. */
    for (int d = 0; d < D; ++d) q[d] = alpha[d] * q_pre[d] + beta[d];

    /* Scores and their maximum. */
    double inv_sqrt_d = 1.0 / sqrt((double)D);
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        const double *kj = k + (lo + j) * kv_stride;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += q[d] * kj[d];
        s[j] = dot * inv_sqrt_d;
        if (s[j] > m) m = s[j];
    }

    /* Exponentials, normaliser, weighted sum of values. */
    double den = 0.0;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double p = exp(s[j] - m);
        s[j] = p;
        den += p;
        const double *vj = v + (lo + j) * kv_stride;
        for (int d = 0; d < D; ++d) o[d] += p * vj[d];
    }
    for (int d = 0; d < D; ++d) o[d] /= den;
    if (lse) *lse = m + log(den);
    if (weights)
        for (int64_t j = 0; j < n; ++j) weights[j] = s[j] / den;

    free(q);
    free(s);
    return 0;
}

static int kv_head_of(const int32_t *head_map, int h, int Hq, int Hkv)
{
    return head_map ? head_map[h] : h / (Hq / Hkv);
}

static int check_map(const int32_t *head_map, int Hq, int Hkv)
{
    if (Hq <= 0 || Hkv <= 0) return -1;
    if (!head_map) return (Hq % Hkv == 0) ? 0 : -1;
    for (int h = 0; h < Hq; ++h)
        if (head_map[h] < 0 || head_map[h] >= Hkv) return -1;
    return 0;
}

/*
 * Generic driver: query rows r (position t = q_offset + r) of every batch b
 * and q head h, key range [lo(t), t] with lo(t) = max(0, t - W + 1);
 * W <= 0 means unbounded (lo = 0).
 * rows_sel: optional list of n_sel (b, r) pairs (int64 pairs); NULL = all.
 */
static int attend_all(int B, int nrows, int64_t q_offset, int T, int Hq,
                      int Hkv, int D, int64_t W, const int32_t *head_map,
                      const double *q_pre, const double *alpha,
                      const double *beta, const double *k, const double *v,
                      double *o, double *lse, int64_t n_sel,
                      const int64_t *rows_sel)
{
    if (B <= 0 || nrows < 0 || T <= 0 || D <= 0) return -1;
    if (check_map(head_map, Hq, Hkv)) return -1;
    if (q_offset < 0 || q_offset + nrows > T) return -1;

    int64_t n_items = rows_sel ? n_sel : (int64_t)B * nrows;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t it = 0; it < n_items * Hq; ++it) {
        int64_t item = it / Hq;
        int h = (int)(it % Hq);
        int64_t b, r;
        if (rows_sel) { b = rows_sel[2 * item]; r = rows_sel[2 * item + 1]; }
        else { b = item / nrows; r = item % nrows; }
        if (b < 0 || b >= B || r < 0 || r >= nrows) { err |= 1; continue; }
        int64_t t = q_offset + r;
        int64_t lo = (W > 0 && t - W + 1 > 0) ? t - W + 1 : 0;
        int g = kv_head_of(head_map, h, Hq, Hkv);
        const double *qrow = q_pre + ((b * nrows + r) * Hq + h) * D;
        const double *kb = k + (b * (int64_t)T * Hkv + g) * D;
        const double *vb = v + (b * (int64_t)T * Hkv + g) * D;
        /* outputs are indexed by the item so that a row sample gets a
         * compact output array */
        double *orow = o + (item * Hq + h) * D;
        double *lrow = lse ? lse + item * Hq + h : NULL;
        err |= attend_row(qrow, alpha + (int64_t)h * D, beta + (int64_t)h * D,
                          kb, vb, (int64_t)Hkv * D, D, lo, t, orow, lrow,
                          NULL) != 0;
    }
    return err ? -1 : 0;
}

/* Base stream: sliding-window attention over every position t in [0, T). */
int oracle_swa(int B, int T, int Hq, int Hkv, int D, int64_t W,
               const int32_t *head_map, const double *q_pre,
               const double *alpha, const double *beta, const double *k,
               const double *v, double *o, double *lse, int64_t n_sel,
               const int64_t *rows_sel)
{
    if (W < 1) return -1;
    return attend_all(B, T, 0, T, Hq, Hkv, D, W, head_map, q_pre, alpha, beta,
                      k, v, o, lse, n_sel, rows_sel);
}

/* Output stream: full causal cross-attention for rows t = T_in + r,
 * r in [0, T_out), over keys [0, t] of the base stream's K/V. */
int oracle_xattn(int B, int T_in, int T_out, int Hq, int Hkv, int D,
                 const int32_t *head_map, const double *qx_pre,
                 const double *alpha_x, const double *beta_x, const double *k,
                 const double *v, double *o_x, double *lse, int64_t n_sel,
                 const int64_t *rows_sel)
{
    if (T_in < 0 || T_out < 1) return -1;
    return attend_all(B, T_out, T_in, T_in + T_out, Hq, Hkv, D, 0, head_map,
                      qx_pre, alpha_x, beta_x, k, v, o_x, lse, n_sel,
                      rows_sel);
}

/* Normalised softmax weights of one row (for support / sum checks):
 * weights_out[0..T) gets the weight of key j, zero outside [lo, t]. */
int oracle_row_weights(int T, int Hkv, int D, int64_t t, int64_t W, int g,
                       const double *q_pre_row, const double *alpha_h,
                       const double *beta_h, const double *k, const double *v,
                       double *weights_out)
{
    if (t < 0 || t >= T || g < 0 || g >= Hkv) return -1;
    int64_t lo = (W > 0 && t - W + 1 > 0) ? t - W + 1 : 0;
    double *o = (double *)malloc(sizeof(double) * (size_t)D);
    if (!o) return -1;
    for (int64_t j = 0; j < T; ++j) weights_out[j] = 0.0;
    int rc = attend_row(q_pre_row, alpha_h, beta_h, k + (int64_t)g * D,
                        v + (int64_t)g * D, (int64_t)Hkv * D, D, lo, t, o,
                        NULL, weights_out + lo);
    free(o);
    return rc;
}

/*
 * Incremental mode: an explicit growing per-layer cache, separate from the
 * batched functions above, so that comparing the two is a real check
 * (reproduction note "Orthros：阶段异构注意力", local-reproduction results:
 * cached prefill/decode must match the batched computation within 1e-4).
 * Storage: per batch, per KV head, a growing list of keys [cap][D].
 */
typedef struct {
    int B, Hkv, D;
    int64_t cap;
    int64_t *len;   /* [B] */
    double *k, *v;  /* [B][Hkv][cap][D] */
} oracle_cache;

void *oracle_cache_new(int B, int Hkv, int D, int64_t cap)
{
    if (B <= 0 || Hkv <= 0 || D <= 0 || cap <= 0) return NULL;
    oracle_cache *c = (oracle_cache *)calloc(1, sizeof(*c));
    if (!c) return NULL;
    c->B = B; c->Hkv = Hkv; c->D = D; c->cap = cap;
    size_t n = (size_t)B * Hkv * cap * D;
    c->len = (int64_t *)calloc((size_t)B, sizeof(int64_t));
    c->k = (double *)calloc(n, sizeof(double));
    c->v = (double *)calloc(n, sizeof(double));
    if (!c->len || !c->k || !c->v) {
        free(c->len); free(c->k); free(c->v); free(c);
        return NULL;
    }
    return c;
}

void oracle_cache_free(void *p)
{
    oracle_cache *c = (oracle_cache *)p;
    if (!c) return;
    free(c->len); free(c->k); free(c->v); free(c);
}

int64_t oracle_cache_len(const void *p, int b)
{
    const oracle_cache *c = (const oracle_cache *)p;
    return (c && b >= 0 && b < c->B) ? c->len[b] : -1;
}

/* Append n new base tokens per batch: k_new, v_new [B, n, Hkv, D]. */
int oracle_cache_append(void *p, int n, const double *k_new,
                        const double *v_new)
{
    oracle_cache *c = (oracle_cache *)p;
    if (!c || n < 0) return -1;
    for (int b = 0; b < c->B; ++b)
        if (c->len[b] + n > c->cap) return -1;
    for (int b = 0; b < c->B; ++b) {
        for (int i = 0; i < n; ++i)
            for (int g = 0; g < c->Hkv; ++g) {
                int64_t pos = c->len[b] + i;
                double *kd = c->k + (((int64_t)b * c->Hkv + g) * c->cap + pos) * c->D;
                double *vd = c->v + (((int64_t)b * c->Hkv + g) * c->cap + pos) * c->D;
                const double *ks = k_new + (((int64_t)b * n + i) * c->Hkv + g) * c->D;
                const double *vs = v_new + (((int64_t)b * n + i) * c->Hkv + g) * c->D;
                memcpy(kd, ks, sizeof(double) * (size_t)c->D);
                memcpy(vd, vs, sizeof(double) * (size_t)c->D);
            }
        c->len[b] += n;
    }
    return 0;
}

/*
 * One decode pair step (paper text §3.2, Decoding; §3.1, the decoupled pair):
 * the base token's K/V is appended at index n = old length, then
 *   base query   over keys [max(0, n-W+1), n]
 *   output query over keys [0, n].
 * q_pre, qx_pre [B, Hq, D]; k_new, v_new [B, Hkv, D]; o, o_x [B, Hq, D].
 */
int oracle_cache_decode_pair(void *p, int Hq, int64_t W,
                             const int32_t *head_map, const double *q_pre,
                             const double *qx_pre, const double *alpha,
                             const double *beta, const double *alpha_x,
                             const double *beta_x, const double *k_new,
                             const double *v_new, double *o, double *o_x)
{
    oracle_cache *c = (oracle_cache *)p;
    if (!c || W < 1 || check_map(head_map, Hq, c->Hkv)) return -1;
    if (oracle_cache_append(p, 1, k_new, v_new)) return -1;
    int D = c->D, err = 0;
    for (int b = 0; b < c->B; ++b) {
        int64_t t = c->len[b] - 1;
        int64_t lo = (t - W + 1 > 0) ? t - W + 1 : 0;
        for (int h = 0; h < Hq; ++h) {
            int g = kv_head_of(head_map, h, Hq, c->Hkv);
            const double *kb = c->k + ((int64_t)b * c->Hkv + g) * c->cap * D;
            const double *vb = c->v + ((int64_t)b * c->Hkv + g) * c->cap * D;
            int64_t qi = ((int64_t)b * Hq + h) * D;
            err |= attend_row(q_pre + qi, alpha + (int64_t)h * D,
                              beta + (int64_t)h * D, kb, vb, D, D, lo, t,
                              o + qi, NULL, NULL);
            err |= attend_row(qx_pre + qi, alpha_x + (int64_t)h * D,
                              beta_x + (int64_t)h * D, kb, vb, D, D, 0, t,
                              o_x + qi, NULL, NULL);
        }
    }
    return err ? -1 : 0;
}

/* Threads the OpenMP runtime will use (for reporting the baseline). */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
#else
int oracle_num_threads(void) { return 1; }
#endif
