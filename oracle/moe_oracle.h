/*
 * moe_oracle.h — fp64 CPU oracle for the Mixtral sparse-MoE feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this code; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no source, header, table or helper with the
 * HIP implementation.
 *
 * What it computes (sources are the pages about "Mixtral of Experts"):
 *   - router scores  l_e = x . Wg_e, one per expert, no bias
 *       [ennepo lecture, the router passage; tokentrails lineage, step "The router"]
 *   - keep the K largest scores, softmax over only those K
 *       [flashpapers summary, "How It Works" (TopK sets the rest to -inf);
 *        tokentrails lineage, step "The router": g = softmax(top-2(x.Wg))]
 *   - each expert is the SwiGLU MLP  w2(silu(w1 x) * w3 x)
 *       [fdeinterviews breakdown, "The paper in one minute";
 *        tokentrails lineage, Code listing]
 *   - y = sum over kept experts of g_i * E_i(x); unkept experts are never read
 *       [flashpapers summary, "How It Works"; tokentrails lineage, step
 *        "Two experts per token": y = ga.Ea(x) + gb.Eb(x)]
 *   - the decoder-block wrapper  out = h + moe(rms_norm(h))
 *       [tokentrails lineage, Code listing]
 *
 * Conventions shared by every entry point:
 *   - dtype codes: 0 = IEEE fp32, 1 = bf16 (raw 16-bit patterns, uint16).
 *   - all matrices are row-major and caller-owned; the oracle allocates only
 *     private temporaries.
 *   - Wg is fp32 [E][d]; W1, W3 are [E][d_ff][d]; W2 is [E][d][d_ff]
 *     (nn.Linear storage: [out][in]).
 *   - return 0 on success, -1 on a bad argument.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Round a double to the nearest bf16 value (ties to even), returned as a double. */
double orc_bf16_round(double v);

/* logits[t][e] = sum_i x[t][i] * Wg[e][i], accumulated in fp64. */
int orc_router_logits(const void *x, int x_dt, const float *Wg, long T, int d, int E,
                      double *logits, int nthreads);

/* Top-k selection and gate weights for T rows of E logits.
 * The choice is made on the logits rounded to fp32 (the precision the router
 * delivers its scores in); equal fp32 scores go to the lower expert index.
 * idx[t][j] is the j-th choice; gates[t][j] = softmax over the k kept fp64
 * logits; gap_order[t] = min over j<k-1 of l(j)-l(j+1); gap_set[t] =
 * l(k-1) - max over unkept l (or +inf when k == E).  Any output may be NULL. */
int orc_topk_gates(const double *logits, long T, int E, int k, int32_t *idx,
                   double *gates, double *gap_order, double *gap_set);

/* Router load statistics and the load-balancing loss
 * [tokentrails lineage, step "Load balancing" and the Code listing's last
 * line: Laux = N * sum_i f_i * P_i, N the number of experts]:
 *   f[e] = share of the T*k assignments routed to expert e (sums to 1),
 *   P[e] = the router's softmax probability of expert e over all E scores,
 *          averaged over the T tokens (sums to 1),
 *   laux = E * sum_e f[e] * P[e].
 * logits [T][E] fp64, idx [T][k] the choices; T >= 1. */
int orc_balance(const double *logits, const int32_t *idx, long T, int E, int k, double *f,
                double *P, double *laux);

/* Stable counting sort of the T*k assignments by expert.  Assignment (t,j)
 * gets a row in expert idx[t][j]'s contiguous block; inside a block rows go in
 * ascending t, then j.  counts[E], offsets[E+1] (exclusive scan),
 * row_of[T][k], token_of[T*k]. */
int orc_permute(const int32_t *idx, long T, int E, int k, int32_t *counts,
                int32_t *offsets, int32_t *row_of, int32_t *token_of);

/* One expert on one input row x[d] (fp64): out[d] = W2_e (silu(W1_e x) * W3_e x).
 * round_mid != 0 rounds the intermediate silu(W1_e x) * W3_e x to bf16 first. */
int orc_swiglu_expert(const double *x, const void *W1, const void *W3, const void *W2,
                      int w_dt, int e, int d, int d_ff, int round_mid, double *out);

/* The whole layer for a list of rows (rows[n] indexes x).  Outputs per listed
 * row: y[n][d] (fp64), idx[n][k], gates[n][k], gap_order[n], gap_set[n]
 * (NULL to skip).  round_mid as for orc_swiglu_expert.  Threads split the
 * list statically. */
int orc_moe_rows(const void *x, int x_dt, const float *Wg, const void *W1,
                 const void *W3, const void *W2, int w_dt, int d, int d_ff, int E,
                 int k, int round_mid, const int64_t *rows, long n, double *y, int32_t *idx,
                 double *gates, double *gap_order, double *gap_set, int nthreads);

/* RMSNorm with unit gain: out_i = h_i / sqrt(mean(h^2) + eps), fp64. */
int orc_rmsnorm(const double *h, int d, double eps, double *out);

/* rmsnorm of each of n rows of h[n][d]; with round_bf16 != 0 each output is
 * rounded to the nearest bf16 value (the activations the router then sees). */
int orc_rmsnorm_rows(const double *h, long n, int d, double eps, int round_bf16, double *out);

/* One decoder-block MoE step on n independent rows held as bf16 values in
 * fp64 (h[n][d], updated in place):
 *     xn = bf16(rmsnorm(h));  h <- bf16(h + moe(xn)).
 * Weights are bf16; round_mid as for orc_swiglu_expert.  Routing of the step
 * is returned as for orc_moe_rows. */
int orc_block_step(double *h, long n, const float *Wg, const void *W1, const void *W3,
                   const void *W2, int d, int d_ff, int E, int k, double eps, int round_mid,
                   int32_t *idx, double *gates, double *gap_order, double *gap_set,
                   int nthreads);

#ifdef __cplusplus
}
#endif
#endif
