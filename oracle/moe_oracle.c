/*
 * moe_oracle.c — plain, slow, fp64 CPU oracle for the Mixtral sparse-MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h).  Built with
 * gcc -O2 -ffp-contract=off, no fast-math, no BLAS: every sum is a left-to-
 * right fp64 loop so that a reader can check it against the definition.
 */
#include "moe_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---- element access ---------------------------------------------------- */

static double widen_bf16(uint16_t bits) {
    /* bf16 is the top half of an IEEE fp32 pattern */
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(const void *base, int dt, size_t i) {
    if (dt == 0) return (double)((const float *)base)[i];
    return widen_bf16(((const uint16_t *)base)[i]);
}

/* bf16 keeps 8 significant bits and fp32's exponent range.  Round to nearest,
 * ties to even: scale the significand to [128,256), round with rint (the
 * default rounding mode is nearest-even), scale back. */
double orc_bf16_round(double v) {
    if (!isfinite(v) || v == 0.0) return v;
    double a = fabs(v);
    double r;
    if (a < ldexp(1.0, -126)) {
        /* subnormal range: fixed spacing 2^-133 */
        r = rint(a * ldexp(1.0, 133)) * ldexp(1.0, -133);
    } else {
        int e;
        double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
        r = ldexp(rint(ldexp(m, 8)), e - 8);
    }
    /* largest finite bf16 is (2 - 2^-7) * 2^127; anything that rounds past it
     * overflows to infinity */
    if (r > ldexp(255.0, 120)) r = INFINITY;
    return v < 0 ? -r : r;
}

/* ---- a tiny static parallel-for over [0, n) ---------------------------- */

typedef void (*range_fn)(void *ctx, long lo, long hi);
typedef struct {
    range_fn fn;
    void *ctx;
    long lo, hi;
} range_job;

static void *range_thread(void *p) {
    range_job *j = (range_job *)p;
    j->fn(j->ctx, j->lo, j->hi);
    return NULL;
}

static void parallel_for(long n, int nthreads, range_fn fn, void *ctx) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((long)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
    if (nthreads == 1) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t th[256];
    range_job jobs[256];
    int started[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i].fn = fn;
        jobs[i].ctx = ctx;
        jobs[i].lo = n * i / nthreads;
        jobs[i].hi = n * (i + 1) / nthreads;
        started[i] = pthread_create(&th[i], NULL, range_thread, &jobs[i]) == 0;
        if (!started[i]) fn(ctx, jobs[i].lo, jobs[i].hi);
    }
    for (int i = 0; i < nthreads; ++i)
        if (started[i]) pthread_join(th[i], NULL);
}

/* ---- router scores ------------------------------------------------------ */

/* One score per expert: the token's vector times the gate matrix, no bias
 * [ennepo lecture, router passage; tokentrails lineage, step "The router"]. */
static void logits_one(const void *x, int x_dt, size_t row, const float *Wg, int d,
                       int E, double *out) {
    for (int e = 0; e < E; ++e) {
        double s = 0.0;
        for (int i = 0; i < d; ++i)
            s += load_elem(x, x_dt, row * (size_t)d + i) * (double)Wg[(size_t)e * d + i];
        out[e] = s;
    }
}

typedef struct {
    const void *x;
    int x_dt;
    const float *Wg;
    int d, E;
    double *logits;
} logits_ctx;

static void logits_range(void *p, long lo, long hi) {
    logits_ctx *c = (logits_ctx *)p;
    for (long t = lo; t < hi; ++t)
        logits_one(c->x, c->x_dt, (size_t)t, c->Wg, c->d, c->E, c->logits + (size_t)t * c->E);
}

int orc_router_logits(const void *x, int x_dt, const float *Wg, long T, int d, int E,
                      double *logits, int nthreads) {
    if (T < 0 || d < 1 || E < 1 || (x_dt != 0 && x_dt != 1) || (T > 0 && (!x || !Wg || !logits)))
        return -1;
    logits_ctx c = {x, x_dt, Wg, d, E, logits};
    parallel_for(T, nthreads, logits_range, &c);
    return 0;
}

/* ---- top-k and the softmax over the kept scores ------------------------ */

/* TopK keeps the K largest scores and sends the rest to -inf, then a softmax
 * runs over what is left [flashpapers summary, "How It Works"].  The softmax
 * of -inf entries is exactly zero, so the gate of a kept expert is its
 * softmax over the K kept scores alone. */
static void topk_one(const double *l, int E, int k, int32_t *idx, double *gates,
                     double *gap_order, double *gap_set) {
    int kept[64];
    int used[64];
    for (int e = 0; e < E; ++e) used[e] = 0;
    for (int j = 0; j < k; ++j) {
        int best = -1;
        float bestv = 0.0f;
        for (int e = 0; e < E; ++e) {
            if (used[e]) continue;
            float v = (float)l[e]; /* decide on the fp32 score */
            if (best < 0 || v > bestv) { /* strict '>' keeps the lower index on ties */
                best = e;
                bestv = v;
            }
        }
        used[best] = 1;
        kept[j] = best;
    }
    double lmax = l[kept[0]];
    double z = 0.0;
    for (int j = 0; j < k; ++j) z += exp(l[kept[j]] - lmax);
    for (int j = 0; j < k; ++j) {
        if (idx) idx[j] = kept[j];
        if (gates) gates[j] = exp(l[kept[j]] - lmax) / z;
    }
    if (gap_order) {
        double g = INFINITY;
        for (int j = 0; j + 1 < k; ++j) {
            double diff = l[kept[j]] - l[kept[j + 1]];
            if (diff < g) g = diff;
        }
        *gap_order = g;
    }
    if (gap_set) {
        double worst_out = -INFINITY;
        for (int e = 0; e < E; ++e)
            if (!used[e] && l[e] > worst_out) worst_out = l[e];
        double lowest_in = INFINITY;
        for (int j = 0; j < k; ++j)
            if (l[kept[j]] < lowest_in) lowest_in = l[kept[j]];
        *gap_set = (k == E) ? INFINITY : lowest_in - worst_out;
    }
}

int orc_topk_gates(const double *logits, long T, int E, int k, int32_t *idx,
                   double *gates, double *gap_order, double *gap_set) {
    if (T < 0 || E < 1 || E > 64 || k < 1 || k > E || (T > 0 && !logits)) return -1;
    for (long t = 0; t < T; ++t)
        topk_one(logits + (size_t)t * E, E, k, idx ? idx + (size_t)t * k : NULL,
                 gates ? gates + (size_t)t * k : NULL, gap_order ? gap_order + t : NULL,
                 gap_set ? gap_set + t : NULL);
    return 0;
}

/* ---- load statistics ---------------------------------------------------- */

/* The loss the pages add in training is smallest when both the routed tokens
 * and the router's probabilities spread evenly over the experts
 * [tokentrails lineage, step "Load balancing"].  f is the share of routed
 * assignments per expert, P the mean over tokens of the full softmax over
 * the E scores; the loss multiplies their dot product by the expert count. */
int orc_balance(const double *logits, const int32_t *idx, long T, int E, int k, double *f,
                double *P, double *laux) {
    if (T < 1 || E < 1 || E > 64 || k < 1 || k > E || !logits || !idx || !f || !P || !laux)
        return -1;
    for (int e = 0; e < E; ++e) {
        f[e] = 0.0;
        P[e] = 0.0;
    }
    for (long a = 0; a < T * (long)k; ++a) {
        if (idx[a] < 0 || idx[a] >= E) return -1;
        f[idx[a]] += 1.0;
    }
    for (int e = 0; e < E; ++e) f[e] /= (double)(T * (long)k);
    for (long t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        double m = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > m) m = l[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e) z += exp(l[e] - m);
        for (int e = 0; e < E; ++e) P[e] += exp(l[e] - m) / z;
    }
    double s = 0.0;
    for (int e = 0; e < E; ++e) {
        P[e] /= (double)T;
        s += f[e] * P[e];
    }
    *laux = (double)E * s;
    return 0;
}

/* ---- grouping assignments by expert ------------------------------------ */

/* Each expert receives the rows routed to it and some receive none
 * [tokentrails lineage, step "Two experts per token"].  A counting sort in
 * assignment order makes the grouping stable. */
int orc_permute(const int32_t *idx, long T, int E, int k, int32_t *counts,
                int32_t *offsets, int32_t *row_of, int32_t *token_of) {
    if (T < 0 || E < 1 || k < 1 || !counts || !offsets) return -1;
    long A = T * (long)k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (long a = 0; a < A; ++a) {
        int e = idx[a];
        if (e < 0 || e >= E) return -1;
        counts[e] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t next[64];
    for (int e = 0; e < E; ++e) next[e] = offsets[e];
    for (long a = 0; a < A; ++a) {
        int e = idx[a];
        int32_t r = next[e]++;
        if (row_of) row_of[a] = r;
        if (token_of) token_of[r] = (int32_t)(a / k);
    }
    return 0;
}

/* ---- one SwiGLU expert --------------------------------------------------- */

static double silu(double u) { return u / (1.0 + exp(-u)); }

/* E(x) = w2(silu(w1 x) * w3 x)  [tokentrails lineage, Code listing;
 * fdeinterviews breakdown: each expert is a SwiGLU block].  With round_mid
 * the intermediate silu(w1 x) * w3 x is rounded to bf16 before w2 (the
 * quantisation point of a bf16 data path). */
int orc_swiglu_expert(const double *x, const void *W1, const void *W3, const void *W2,
                      int w_dt, int e, int d, int d_ff, int round_mid, double *out) {
    if (!x || !W1 || !W3 || !W2 || !out || d < 1 || d_ff < 1 || e < 0) return -1;
    double *h = (double *)malloc(sizeof(double) * (size_t)d_ff);
    if (!h) return -1;
    size_t base13 = (size_t)e * d_ff * d;
    for (int j = 0; j < d_ff; ++j) {
        double u = 0.0, v = 0.0;
        for (int i = 0; i < d; ++i) {
            u += load_elem(W1, w_dt, base13 + (size_t)j * d + i) * x[i];
            v += load_elem(W3, w_dt, base13 + (size_t)j * d + i) * x[i];
        }
        h[j] = silu(u) * v;
        if (round_mid) h[j] = orc_bf16_round(h[j]);
    }
    size_t base2 = (size_t)e * d * d_ff;
    for (int i = 0; i < d; ++i) {
        double s = 0.0;
        for (int j = 0; j < d_ff; ++j) s += load_elem(W2, w_dt, base2 + (size_t)i * d_ff + j) * h[j];
        out[i] = s;
    }
    free(h);
    return 0;
}

/* ---- the layer on one row ------------------------------------------------ */

/* y = sum over the kept experts of g_i E_i(x); an expert whose gate is zero is
 * never evaluated and its weights are never read [flashpapers summary, "How
 * It Works"; ennepo lecture, combine passage: the unchosen experts' weights
 * stay unread]. */
static int moe_one(const double *x, const float *Wg, const void *W1, const void *W3,
                   const void *W2, int w_dt, int d, int d_ff, int E, int k, int round_mid,
                   double *y, int32_t *idx, double *gates, double *gap_order,
                   double *gap_set) {
    double l[64];
    double g[64];
    int32_t sel[64];
    for (int e = 0; e < E; ++e) {
        double s = 0.0;
        for (int i = 0; i < d; ++i) s += x[i] * (double)Wg[(size_t)e * d + i];
        l[e] = s;
    }
    topk_one(l, E, k, sel, g, gap_order, gap_set);
    double *o = (double *)malloc(sizeof(double) * (size_t)d);
    if (!o) return -1;
    for (int i = 0; i < d; ++i) y[i] = 0.0;
    for (int j = 0; j < k; ++j) {
        if (orc_swiglu_expert(x, W1, W3, W2, w_dt, sel[j], d, d_ff, round_mid, o) != 0) {
            free(o);
            return -1;
        }
        for (int i = 0; i < d; ++i) y[i] += g[j] * o[i];
    }
    free(o);
    for (int j = 0; j < k; ++j) {
        if (idx) idx[j] = sel[j];
        if (gates) gates[j] = g[j];
    }
    return 0;
}

typedef struct {
    const void *x;
    int x_dt;
    const float *Wg;
    const void *W1, *W3, *W2;
    int w_dt, d, d_ff, E, k, round_mid;
    const int64_t *rows;
    double *y;
    int32_t *idx;
    double *gates, *gap_order, *gap_set;
    int failed;
} rows_ctx;

static void rows_range(void *p, long lo, long hi) {
    rows_ctx *c = (rows_ctx *)p;
    double *xr = (double *)malloc(sizeof(double) * (size_t)c->d);
    if (!xr) {
        c->failed = 1;
        return;
    }
    for (long n = lo; n < hi; ++n) {
        size_t r = (size_t)c->rows[n];
        for (int i = 0; i < c->d; ++i) xr[i] = load_elem(c->x, c->x_dt, r * c->d + i);
        if (moe_one(xr, c->Wg, c->W1, c->W3, c->W2, c->w_dt, c->d, c->d_ff, c->E, c->k, c->round_mid,
                    c->y + (size_t)n * c->d, c->idx ? c->idx + (size_t)n * c->k : NULL,
                    c->gates ? c->gates + (size_t)n * c->k : NULL,
                    c->gap_order ? c->gap_order + n : NULL,
                    c->gap_set ? c->gap_set + n : NULL) != 0)
            c->failed = 1;
    }
    free(xr);
}

int orc_moe_rows(const void *x, int x_dt, const float *Wg, const void *W1,
                 const void *W3, const void *W2, int w_dt, int d, int d_ff, int E,
                 int k, int round_mid, const int64_t *rows, long n, double *y, int32_t *idx,
                 double *gates, double *gap_order, double *gap_set, int nthreads) {
    if (n < 0 || d < 1 || d_ff < 1 || E < 1 || E > 64 || k < 1 || k > E) return -1;
    if (n > 0 && (!x || !Wg || !W1 || !W3 || !W2 || !rows || !y)) return -1;
    rows_ctx c = {x, x_dt, Wg, W1, W3, W2, w_dt, d, d_ff, E, k, round_mid, rows, y, idx,
                  gates, gap_order, gap_set, 0};
    parallel_for(n, nthreads, rows_range, &c);
    return c.failed ? -1 : 0;
}

/* ---- the decoder-block wrapper ------------------------------------------ */

/* rms_norm with unit gain [tokentrails lineage, Code listing; the block is
 * LLaMA's, which normalises by the root mean square]. */
int orc_rmsnorm(const double *h, int d, double eps, double *out) {
    if (!h || !out || d < 1) return -1;
    double ss = 0.0;
    for (int i = 0; i < d; ++i) ss += h[i] * h[i];
    double scale = 1.0 / sqrt(ss / d + eps);
    for (int i = 0; i < d; ++i) out[i] = h[i] * scale;
    return 0;
}

int orc_rmsnorm_rows(const double *h, long n, int d, double eps, int round_bf16, double *out) {
    if (n < 0 || d < 1 || (n > 0 && (!h || !out))) return -1;
    for (long r = 0; r < n; ++r) {
        orc_rmsnorm(h + (size_t)r * d, d, eps, out + (size_t)r * d);
        if (round_bf16)
            for (int i = 0; i < d; ++i) out[(size_t)r * d + i] = orc_bf16_round(out[(size_t)r * d + i]);
    }
    return 0;
}

typedef struct {
    double *h;
    const float *Wg;
    const void *W1, *W3, *W2;
    int d, d_ff, E, k, round_mid;
    double eps;
    int32_t *idx;
    double *gates, *gap_order, *gap_set;
    int failed;
} block_ctx;

static void block_range(void *p, long lo, long hi) {
    block_ctx *c = (block_ctx *)p;
    double *xn = (double *)malloc(sizeof(double) * (size_t)c->d);
    double *y = (double *)malloc(sizeof(double) * (size_t)c->d);
    if (!xn || !y) {
        c->failed = 1;
        free(xn);
        free(y);
        return;
    }
    for (long n = lo; n < hi; ++n) {
        double *h = c->h + (size_t)n * c->d;
        orc_rmsnorm(h, c->d, c->eps, xn);
        for (int i = 0; i < c->d; ++i) xn[i] = orc_bf16_round(xn[i]); /* bf16 activations */
        if (moe_one(xn, c->Wg, c->W1, c->W3, c->W2, 1, c->d, c->d_ff, c->E, c->k, c->round_mid, y,
                    c->idx ? c->idx + (size_t)n * c->k : NULL,
                    c->gates ? c->gates + (size_t)n * c->k : NULL,
                    c->gap_order ? c->gap_order + n : NULL,
                    c->gap_set ? c->gap_set + n : NULL) != 0)
            c->failed = 1;
        for (int i = 0; i < c->d; ++i) h[i] = orc_bf16_round(h[i] + y[i]); /* residual, bf16 */
    }
    free(xn);
    free(y);
}

int orc_block_step(double *h, long n, const float *Wg, const void *W1, const void *W3,
                   const void *W2, int d, int d_ff, int E, int k, double eps, int round_mid,
                   int32_t *idx, double *gates, double *gap_order, double *gap_set,
                   int nthreads) {
    if (n < 0 || d < 1 || d_ff < 1 || E < 1 || E > 64 || k < 1 || k > E) return -1;
    if (n > 0 && (!h || !Wg || !W1 || !W3 || !W2)) return -1;
    block_ctx c = {h,   Wg,   W1, W3,  W2,    d,         d_ff,    E, k,
                   round_mid, eps, idx, gates, gap_order, gap_set, 0};
    parallel_for(n, nthreads, block_range, &c);
    return c.failed ? -1 : 0;
}
