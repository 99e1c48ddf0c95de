/*
 * moe.h — C ABI of libmoe.so: the Mixtral sparse-MoE feed-forward layer on
 * one AMD MI355X (gfx950), in hand-written HIP kernels.
 *
 * The layer (pages about "Mixtral of Experts"):
 *   scores   l_e = x . Wg_e for each of E experts, no bias
 *            [ennepo lecture, router passage; tokentrails lineage, step "The router"]
 *   choice   keep the k largest scores, softmax over only those k
 *            [flashpapers summary, "How It Works"; tokentrails lineage,
 *             g = softmax(top-2(x . Wg))]
 *   experts  E_e(x) = W2_e (silu(W1_e x) * W3_e x)   (SwiGLU)
 *            [fdeinterviews breakdown, "The paper in one minute"; tokentrails Code listing]
 *   output   y = sum_j g_j E_{idx_j}(x); experts not chosen are never read
 *            [flashpapers summary, "How It Works"; tokentrails step "Two experts per token"]
 *   block    h <- h + moe(rms_norm(h))   [tokentrails lineage, Code listing]
 *
 * Conventions for every call:
 *   - Pointers are device pointers (hipMalloc / torch CUDA tensors) unless a
 *     comment says otherwise.  The caller owns every buffer.  The library
 *     allocates and frees nothing and keeps no state between calls; calls on
 *     distinct streams with distinct outputs and workspaces may run together.
 *   - `stream` is a hipStream_t passed as void* (NULL: the null stream).  Each
 *     call only enqueues work on it and returns; nothing synchronises.  A
 *     fault inside a kernel surfaces at the caller's next synchronisation.
 *   - Layouts are row-major.  x is [T][d]; Wg is fp32 [E][d]; W1 and W3 are
 *     [E][d_ff][d]; W2 is [E][d][d_ff] (nn.Linear storage, [out][in], so the
 *     pages' x . Wg is x . Wg^T here).  y has x's shape and dtype.
 *   - `dt` is the dtype of activations and expert weights: MOE_F32 or MOE_BF16
 *     (bf16 = the upper 16 bits of an IEEE fp32).  Arithmetic inside the
 *     expert GEMMs accumulates in fp32; the router accumulates its products in
 *     fp64 and rounds each score to fp32.
 *   - Requirements, each answered by a status code and never by an abort:
 *       T >= 0 (T == 0: nothing is enqueued, MOE_OK), T*k < 2^31;
 *       1 <= E <= 64, 1 <= k <= min(E, 8);
 *       d and d_ff positive multiples of 64;
 *       every activation / weight / output pointer 16-byte aligned, int32 and
 *       fp32 index/gate arrays 4-byte aligned; no NULL where data is needed.
 *     Violations return MOE_ERR_INVALID_ARG (or MOE_ERR_UNSUPPORTED for
 *     shapes outside these limits) before anything is enqueued.
 *   - Inputs must be finite; the result for NaN/Inf inputs is unspecified.
 *   - A failed launch returns MOE_ERR_HIP; moe_last_error() then describes it.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,  /* NULL, misaligned or negative argument */
    MOE_ERR_UNSUPPORTED = 2,  /* shape outside the limits above */
    MOE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
    MOE_ERR_HIP = 4           /* the HIP runtime rejected a launch */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Text for a status code (static storage). */
const char *moe_status_string(moe_status s);

/* Detail of the last non-OK status returned on the calling thread
 * (thread-local static storage, "" if none). */
const char *moe_last_error(void);

/* Bytes of workspace that moe_forward and moe_block_forward need (and that
 * is also enough for moe_permute and moe_expert_ffn).  Returns 0 for shapes
 * the library rejects.  Layout inside is private; 256-byte alignment of the
 * workspace pointer is required. */
size_t moe_workspace_size(int64_t T, int d, int d_ff, int E, int k, moe_dtype dt);

/* Name of the kernel family that runs the expert GEMMs of moe_forward,
 * moe_expert_ffn and moe_block_forward for this shape (the choice depends on
 * the average rows per expert, T*k/E, on dt and on d, d_ff): one of
 * "stream_gemm_kernel", "skinny_gemm_kernel", "grouped_gemm_kernel (...)",
 * "wide_gemm_kernel (...)".  For the fused layer, whose choice can differ,
 * see moe_forward_kernels.  Static storage; "" for shapes the library
 * rejects.  Host only, enqueues nothing. */
const char *moe_expert_ffn_kernels(int64_t T, int d, int d_ff, int E, int k, moe_dtype dt);

/* The same for the expert GEMMs of moe_forward, moe_forward_noalloc,
 * moe_forward_profiled and moe_block_forward at T tokens: where
 * moe_expert_ffn_kernels names "stream_gemm_kernel" and T is 1 to 8 with
 * T*k <= 32 (and, on 256 CUs, d_ff <= 16384, d <= 32768 up to four tokens
 * and d <= 16384 for five to eight), the layer runs "stream_cols_kernel"
 * (each workgroup streams its own columns of every active expert over the
 * whole K, GEMM2 forms y); from 9 to 32 tokens with T*k <= 64 (and d <= 4096
 * on 256 CUs) it runs GEMM1 on the former and GEMM2 on the latter, named
 * "stream_gemm_kernel + stream_cols_kernel (W2)"; otherwise the same name.
 * Static storage; "" for shapes the library rejects.  Host only, enqueues
 * nothing. */
const char *moe_forward_kernels(int64_t T, int d, int d_ff, int E, int k, moe_dtype dt);

/* Router: scores, top-k and gates for T tokens.
 *   x [T][d] (dt), Wg fp32 [E][d]
 *   -> topk_idx int32 [T][k]: chosen experts, best first; equal fp32 scores
 *      go to the lower expert index
 *   -> topk_w fp32 [T][k]: softmax over the k kept scores (sums to 1)
 *   -> logits_or_null fp32 [T][E]: the scores (optional)
 * Defined by: ennepo lecture (router passage: a linear layer gives one score
 * per expert, all but the k best go to -inf, and a softmax leaves k
 * probabilities summing to one); flashpapers summary "How It Works". */
moe_status moe_route(const void *x, const float *Wg, moe_dtype dt, int64_t T, int d, int E,
                     int k, int32_t *topk_idx, float *topk_w, float *logits_or_null,
                     void *stream);

/* Router plus its load statistics, for training's load-balancing loss:
 * the same topk_idx / topk_w as moe_route, and
 *   -> f_out fp32 [E]: share of the T*k routed assignments that went to
 *      expert e (sums to 1),
 *   -> P_out fp32 [E]: the router's softmax probability of expert e over all
 *      E scores, averaged over the T tokens (sums to 1),
 *   -> laux_out fp32 [1]: E * sum_e f_out[e] * P_out[e] (1 when routing and
 *      probabilities are spread evenly, E when all go to one expert).
 * Statistics are summed in fp64 in a fixed order (deterministic) and rounded
 * once to fp32.  T >= 1.  ws: at least moe_route_balance_workspace_size(T, E)
 * bytes (256-byte aligned).
 * Defined by: tokentrails lineage, step "Load balancing" (Laux = N sum f_i
 * P_i) and the Code listing's last line (share routed times mean
 * probability, times the number of experts). */
size_t moe_route_balance_workspace_size(int64_t T, int E);
moe_status moe_route_balance(const void *x, const float *Wg, moe_dtype dt, int64_t T, int d,
                             int E, int k, int32_t *topk_idx, float *topk_w, float *f_out,
                             float *P_out, float *laux_out, void *ws, size_t ws_bytes,
                             void *stream);

/* Dispatch: group the T*k (token, slot) assignments by expert.
 *   topk_idx int32 [T][k] with entries in [0, E)
 *   -> counts int32 [E]; offsets int32 [E+1] = exclusive scan of counts
 *   -> row_of int32 [T][k]: the row of assignment (t, j) in expert order
 *   -> token_of int32 [T*k]: the token of each row
 *   -> x_perm [T*k][d] (dt): x_perm[row_of[t][j]] = x[t]
 * Inside an expert's block rows are in ascending (t, j) order, so the result
 * is unique and deterministic.  Experts may receive no rows.  Entries of
 * topk_idx outside [0, E) are skipped and get row_of = -1.
 * ws: at least moe_permute_workspace_size(T, E, k) bytes, 256-byte aligned
 * (moe_workspace_size(...) bytes are also enough).  That size is 0 up to
 * 4096 assignments, where one workgroup groups them and ws may be NULL;
 * larger batches are cut into chunks whose per-expert counts ws holds.
 * MOE_ERR_WORKSPACE if ws is missing or too small.
 * Defined by: tokentrails lineage, step "Two experts per token" (tokens are
 * sent to their experts; some experts get more of the batch, some none);
 * flashpapers summary "How It Works" (an expert with G_i = 0 is skipped). */
size_t moe_permute_workspace_size(int64_t T, int E, int k);
moe_status moe_permute(const void *x, const int32_t *topk_idx, moe_dtype dt, int64_t T, int d,
                       int E, int k, int32_t *counts, int32_t *offsets, int32_t *row_of,
                       int32_t *token_of, void *x_perm, void *ws, size_t ws_bytes,
                       void *stream);

/* Experts: for every expert e and every row r in [offsets[e], offsets[e+1]):
 *     out_perm[r] = W2_e (silu(W1_e x_perm[r]) * W3_e x_perm[r])
 * x_perm, out_perm [T*k][d] (dt); offsets int32 [E+1] on the device (as
 * produced by moe_permute; offsets[E] <= T*k).  Rows at or beyond offsets[E]
 * are left untouched.  ws holds the SwiGLU intermediate (rows x d_ff) and,
 * for large bf16 batches and for decode-sized ones (the weight-streaming
 * kernels, up to 26 rows per expert), fp32 partial sums of tiles split along
 * K where whole tiles would leave CUs idle (summed in a fixed order: results
 * are deterministic); moe_workspace_size() bytes always suffice.
 * Defined by: fdeinterviews breakdown, "The paper in one minute" (the experts
 * are SwiGLU blocks);
 * tokentrails lineage, Code listing (w2(silu(w1(x)) * w3(x))). */
moe_status moe_expert_ffn(const void *x_perm, const int32_t *offsets, const void *W1,
                          const void *W3, const void *W2, moe_dtype dt, int64_t T, int d,
                          int d_ff, int E, int k, void *out_perm, void *ws, size_t ws_bytes,
                          void *stream);

/* Combine: y[t] = sum_j topk_w[t][j] * out_perm[row_of[t][j]]  (+ residual[t])
 * summed in fp32 in slot order, then rounded once to dt.  residual_or_null
 * [T][d] (dt) may equal y (in-place residual add).
 * Defined by: tokentrails lineage, step "Two experts per token"
 * (y = ga.Ea(x) + gb.Eb(x)); ennepo lecture (output is the first probability
 * times expert one's output plus the second times expert two's). */
moe_status moe_combine(const void *out_perm, const int32_t *row_of, const float *topk_w,
                       const void *residual_or_null, moe_dtype dt, int64_t T, int d, int k,
                       void *y, void *stream);

/* The whole layer: route, dispatch, experts, combine.  y [T][d] (dt).
 * ws: at least moe_workspace_size(T, d, d_ff, E, k, dt) bytes. */
moe_status moe_forward(const void *x, const float *Wg, const void *W1, const void *W3,
                       const void *W2, moe_dtype dt, int64_t T, int d, int d_ff, int E, int k,
                       void *y, void *ws, size_t ws_bytes, void *stream);

/* moe_forward for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer, the same kernels and bit-identical results, with the workspace
 * replaced by a static device array inside the library of
 * moe_forward_noalloc_max_scratch() bytes (96 MiB of the library's device
 * data: every GPU the library runs on holds its own copy, from the library's
 * first use on it until the process ends, whether or not this is called).  The caller still
 * passes x, the weights and y.  Shapes whose workspace,
 * moe_workspace_size(...), exceeds the array return MOE_ERR_WORKSPACE
 * before anything is enqueued (for d = 4096, d_ff = 14336, E = 8, k = 2 the
 * limit is T = 292).  The call allocates and frees nothing.  Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller. */
size_t moe_forward_noalloc_max_scratch(void);
moe_status moe_forward_noalloc(const void *x, const float *Wg, const void *W1, const void *W3,
                               const void *W2, moe_dtype dt, int64_t T, int d, int d_ff, int E,
                               int k, void *y, void *stream);

/* moe_forward with stage markers, for measurement.  `events` points to 6
 * hipEvent_t handles (passed as void*, created by the caller; any entry may
 * be NULL).  events[i] is recorded on `stream` just before stage i is
 * enqueued and events[5] after the last: 0 router, 1 dispatch, 2 expert GEMM1
 * (W1/W3 + SwiGLU), 3 expert GEMM2 (W2), 4 combine.  The elapsed time
 * between events[i] and events[i+1] is stage i's device time.  events[3] is
 * recorded right after the GEMM1 kernel itself, so events[2]..events[3]
 * bracket that one kernel; a pass that completes GEMM1's K-split tiles
 * (the wide kernels' fixup) counts to stage 3.  Otherwise identical to
 * moe_forward. */
moe_status moe_forward_profiled(const void *x, const float *Wg, const void *W1, const void *W3,
                                const void *W2, moe_dtype dt, int64_t T, int d, int d_ff, int E,
                                int k, void *y, void *ws, size_t ws_bytes, void *const *events,
                                void *stream);

/* RMSNorm with unit gain: out[t] = h[t] / sqrt(mean(h[t]^2) + eps), computed
 * in fp64 and rounded once to dt.  h, out [T][d] (dt).
 * Defined by: tokentrails lineage, Code listing (rms_norm before the MoE;
 * the block is LLaMA's). */
moe_status moe_rmsnorm(const void *h, moe_dtype dt, int64_t T, int d, float eps, void *out,
                       void *stream);

/* One decoder-block MoE step, in place:  h <- h + moe(rms_norm(h)).
 * rms_norm's output is rounded to dt before routing; the residual sum is
 * taken in fp32 and rounded once to dt.  Optional outputs of the step's
 * routing: topk_idx_or_null int32 [T][k], topk_w_or_null fp32 [T][k].
 * ws: at least moe_workspace_size(...) bytes.
 * Defined by: tokentrails lineage, Code listing (h = x + attn(...);
 * out = h + moe(rms_norm(h))). */
moe_status moe_block_forward(void *h, const float *Wg, const void *W1, const void *W3,
                             const void *W2, moe_dtype dt, int64_t T, int d, int d_ff, int E,
                             int k, float eps, int32_t *topk_idx_or_null,
                             float *topk_w_or_null, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
