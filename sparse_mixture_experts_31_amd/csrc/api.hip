// api.hip — the C ABI of libmoe.so (declared in include/moe.h): argument
// checks, workspace carving and kernel launches.  No call allocates, frees,
// copies to the host or synchronises.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "../../include/moe.h"
#include "common.h"

namespace {

thread_local char g_err[512];

moe_status fail(moe_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

moe_status ok() {
    g_err[0] = 0;
    return MOE_OK;
}

moe_status hip_status(hipError_t e, const char *where) {
    if (e == hipSuccess) return ok();
    return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int elem_size(moe_dtype dt) { return dt == MOE_F32 ? 4 : 2; }

moe_status check_shape(int64_t T, int d, int d_ff, int E, int k, moe_dtype dt, bool need_dff) {
    if (dt != MOE_F32 && dt != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %lld is negative", (long long)T);
    if (d <= 0 || (need_dff && d_ff <= 0) || E <= 0 || k <= 0)
        return fail(MOE_ERR_INVALID_ARG, "sizes must be positive (d=%d d_ff=%d E=%d k=%d)", d,
                    d_ff, E, k);
    if (E > 64) return fail(MOE_ERR_UNSUPPORTED, "E = %d exceeds 64", E);
    if (k > E || k > 8) return fail(MOE_ERR_UNSUPPORTED, "k = %d must be <= min(E, 8)", k);
    if (d % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "d = %d is not a multiple of 64", d);
    if (need_dff && d_ff % 64 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "d_ff = %d is not a multiple of 64", d_ff);
    if (T * (int64_t)k >= (1LL << 31))
        return fail(MOE_ERR_UNSUPPORTED, "T*k = %lld does not fit int32 row indices",
                    (long long)(T * k));
    return MOE_OK;
}

#define REQUIRE_PTR(p, a)                                                                    \
    do {                                                                                     \
        if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", #p);              \
        if (!aligned((p), (a)))                                                              \
            return fail(MOE_ERR_INVALID_ARG, "%s is not %d-byte aligned", #p, (int)(a));     \
    } while (0)

#define CHECK(expr)                                                                          \
    do {                                                                                     \
        moe_status _s = (expr);                                                              \
        if (_s != MOE_OK) return _s;                                                         \
    } while (0)

#define LAUNCH(expr, what)                                                                   \
    do {                                                                                     \
        hipError_t _e = (expr);                                                              \
        if (_e != hipSuccess) return hip_status(_e, what);                                   \
    } while (0)

constexpr size_t kAlign = 256;
size_t up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

// Workspace segments of the fused calls, in order.
struct Carve {
    size_t idx, gw, counts, offsets, row_of, token_of, x_perm, o_perm, h, xn, split, dsc,
        total;
    size_t split_bytes;
};

Carve carve(int64_t T, int d, int d_ff, int E, int k, moe_dtype dt) {
    const size_t A = (size_t)T * k, es = elem_size(dt);
    Carve c;
    size_t o = 0;
    c.idx = o;      o += up(A * 4);
    c.gw = o;       o += up(A * 4);
    c.counts = o;   o += up((size_t)E * 4);
    c.offsets = o;  o += up((size_t)(E + 1) * 4);
    c.row_of = o;   o += up(A * 4);
    c.token_of = o; o += up(A * 4);
    c.x_perm = o;   o += up(A * d * es);
    c.o_perm = o;   o += up(A * d * 4);  // expert outputs stay fp32 until combined
    c.h = o;        o += up(A * d_ff * es);
    c.xn = o;       o += up((size_t)T * d * es);
    c.split_bytes = moe_expert_ffn_scratch_bytes((int)dt, (int64_t)A, d, d_ff, E);
    c.split = o;    o += up(c.split_bytes);  // partial sums of K-split expert tiles
    c.dsc = o;      o += up(moe_dispatch_scratch_bytes((int64_t)A, E));  // dispatch chunk counts
    c.total = o;
    return c;
}

template <typename P>
P *at(void *ws, size_t off) {
    return (P *)((char *)ws + off);
}

}  // namespace

extern "C" {

const char *moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "MOE_ERR_UNKNOWN";
}

const char *moe_last_error(void) { return g_err; }

size_t moe_workspace_size(int64_t T, int d, int d_ff, int E, int k, moe_dtype dt) {
    if (check_shape(T, d, d_ff, E, k, dt, true) != MOE_OK) return 0;
    return carve(T, d, d_ff, E, k, dt).total;
}

moe_status moe_route(const void *x, const float *Wg, moe_dtype dt, int64_t T, int d, int E,
                     int k, int32_t *topk_idx, float *topk_w, float *logits_or_null,
                     void *stream) {
    CHECK(check_shape(T, d, 64, E, k, dt, false));
    if (T == 0) return ok();
    REQUIRE_PTR(x, 16);
    REQUIRE_PTR(Wg, 16);
    REQUIRE_PTR(topk_idx, 4);
    REQUIRE_PTR(topk_w, 4);
    if (logits_or_null && !aligned(logits_or_null, 4))
        return fail(MOE_ERR_INVALID_ARG, "logits_or_null is not 4-byte aligned");
    LAUNCH(moe_launch_router(x, (int)dt, Wg, T, d, E, k, topk_idx, topk_w, logits_or_null,
                             (hipStream_t)stream),
           "router");
    return ok();
}

const char *moe_expert_ffn_kernels(int64_t T, int d, int d_ff, int E, int k, moe_dtype dt) {
    if (check_shape(T, d, d_ff, E, k, dt, true) != MOE_OK) return "";
    return moe_expert_ffn_kernel_name((int)dt, T * k, d, d_ff, E);
}

const char *moe_forward_kernels(int64_t T, int d, int d_ff, int E, int k, moe_dtype dt) {
    if (check_shape(T, d, d_ff, E, k, dt, true) != MOE_OK) return "";
    return moe_forward_kernel_name((int)dt, T, k, d, d_ff, E);
}

size_t moe_route_balance_workspace_size(int64_t T, int E) {
    if (T < 1 || E < 1 || E > 64) return 0;
    const size_t blocks = (size_t)moe_router_blocks(T);
    return up(blocks * E * sizeof(double)) + up(blocks * E * sizeof(int32_t));
}

moe_status moe_route_balance(const void *x, const float *Wg, moe_dtype dt, int64_t T, int d,
                             int E, int k, int32_t *topk_idx, float *topk_w, float *f_out,
                             float *P_out, float *laux_out, void *ws, size_t ws_bytes,
                             void *stream) {
    CHECK(check_shape(T, d, 64, E, k, dt, false));
    if (T < 1) return fail(MOE_ERR_INVALID_ARG, "load statistics need T >= 1 (T = %lld)",
                           (long long)T);
    REQUIRE_PTR(x, 16);
    REQUIRE_PTR(Wg, 16);
    REQUIRE_PTR(topk_idx, 4);
    REQUIRE_PTR(topk_w, 4);
    REQUIRE_PTR(f_out, 4);
    REQUIRE_PTR(P_out, 4);
    REQUIRE_PTR(laux_out, 4);
    const size_t need = moe_route_balance_workspace_size(T, E);
    if (!ws || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, need);
    REQUIRE_PTR(ws, kAlign);
    const size_t blocks = (size_t)moe_router_blocks(T);
    double *part_p = (double *)ws;
    int32_t *part_c = at<int32_t>(ws, up(blocks * E * sizeof(double)));
    LAUNCH(moe_launch_route_balance(x, (int)dt, Wg, T, d, E, k, topk_idx, topk_w, part_p, part_c,
                                    f_out, P_out, laux_out, (hipStream_t)stream),
           "route_balance");
    return ok();
}

size_t moe_permute_workspace_size(int64_t T, int E, int k) {
    if (T < 0 || E < 1 || E > 64 || k < 1 || k > E || k > 8 || T * (int64_t)k >= (1LL << 31))
        return 0;
    return moe_dispatch_scratch_bytes(T * k, E);
}

moe_status moe_permute(const void *x, const int32_t *topk_idx, moe_dtype dt, int64_t T, int d,
                       int E, int k, int32_t *counts, int32_t *offsets, int32_t *row_of,
                       int32_t *token_of, void *x_perm, void *ws, size_t ws_bytes,
                       void *stream) {
    CHECK(check_shape(T, d, 64, E, k, dt, false));
    REQUIRE_PTR(counts, 4);
    REQUIRE_PTR(offsets, 4);
    if (T == 0) {
        // still define the (empty) grouping
        LAUNCH(moe_launch_dispatch_index(topk_idx, 0, E, k, counts, offsets, row_of, token_of,
                                         nullptr, (hipStream_t)stream),
               "dispatch");
        return ok();
    }
    REQUIRE_PTR(x, 16);
    REQUIRE_PTR(topk_idx, 4);
    REQUIRE_PTR(row_of, 4);
    REQUIRE_PTR(token_of, 4);
    REQUIRE_PTR(x_perm, 16);
    const size_t need = moe_dispatch_scratch_bytes(T * k, E);
    if (need > 0) {
        if (!ws || ws_bytes < need)
            return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, need);
        REQUIRE_PTR(ws, kAlign);
    }
    hipStream_t s = (hipStream_t)stream;
    LAUNCH(moe_launch_dispatch_index(topk_idx, T * k, E, k, counts, offsets, row_of, token_of,
                                     need > 0 ? (int32_t *)ws : nullptr, s),
           "dispatch");
    LAUNCH(moe_launch_gather_rows(x, (int)dt, T, d, k, row_of, x_perm, s), "gather");
    return ok();
}

moe_status moe_expert_ffn(const void *x_perm, const int32_t *offsets, const void *W1,
                          const void *W3, const void *W2, moe_dtype dt, int64_t T, int d,
                          int d_ff, int E, int k, void *out_perm, void *ws, size_t ws_bytes,
                          void *stream) {
    CHECK(check_shape(T, d, d_ff, E, k, dt, true));
    if (T == 0) return ok();
    REQUIRE_PTR(x_perm, 16);
    REQUIRE_PTR(offsets, 4);
    REQUIRE_PTR(W1, 16);
    REQUIRE_PTR(W3, 16);
    REQUIRE_PTR(W2, 16);
    REQUIRE_PTR(out_perm, 16);
    // workspace: the SwiGLU intermediate, then scratch for K-split tiles
    const size_t h_bytes = up((size_t)T * k * d_ff * elem_size(dt));
    const size_t split_bytes = moe_expert_ffn_scratch_bytes((int)dt, T * k, d, d_ff, E);
    const size_t need = h_bytes + split_bytes;
    if (!ws || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, need);
    REQUIRE_PTR(ws, kAlign);
    LAUNCH(moe_launch_expert_ffn(x_perm, nullptr, offsets, W1, W3, W2, (int)dt, 0, T * k, d,
                                 d_ff, E, ws,
                                 out_perm, split_bytes ? at<char>(ws, h_bytes) : nullptr,
                                 split_bytes, nullptr, (hipStream_t)stream),
           "expert_ffn");
    return ok();
}

moe_status moe_combine(const void *out_perm, const int32_t *row_of, const float *topk_w,
                       const void *residual_or_null, moe_dtype dt, int64_t T, int d, int k,
                       void *y, void *stream) {
    CHECK(check_shape(T, d, 64, 64, k, dt, false));
    if (T == 0) return ok();
    REQUIRE_PTR(out_perm, 16);
    REQUIRE_PTR(row_of, 4);
    REQUIRE_PTR(topk_w, 4);
    REQUIRE_PTR(y, 16);
    if (residual_or_null && !aligned(residual_or_null, 16))
        return fail(MOE_ERR_INVALID_ARG, "residual_or_null is not 16-byte aligned");
    LAUNCH(moe_launch_combine(out_perm, 0, row_of, topk_w, residual_or_null, (int)dt, T, d, k, y,
                              (hipStream_t)stream),
           "combine");
    return ok();
}

static moe_status forward_impl(const void *x, const float *Wg, const void *W1, const void *W3,
                               const void *W2, moe_dtype dt, int64_t T, int d, int d_ff, int E,
                               int k, const void *residual, void *y, int32_t *idx_out,
                               float *w_out, void *ws, const Carve &c, void *const *ev,
                               hipStream_t s) {
    int32_t *idx = idx_out ? idx_out : at<int32_t>(ws, c.idx);
    float *gw = w_out ? w_out : at<float>(ws, c.gw);
    int32_t *counts = at<int32_t>(ws, c.counts);
    int32_t *offsets = at<int32_t>(ws, c.offsets);
    int32_t *row_of = at<int32_t>(ws, c.row_of);
    int32_t *token_of = at<int32_t>(ws, c.token_of);
    void *x_perm = at<char>(ws, c.x_perm);
    void *o_perm = at<char>(ws, c.o_perm);
    void *hbuf = at<char>(ws, c.h);
    const int64_t A = T * k;
    auto mark = [&](int i) -> hipError_t {
        return (ev && ev[i]) ? hipEventRecord((hipEvent_t)ev[i], s) : hipSuccess;
    };
    // Decode sizes on the weight-streaming tile kernels: GEMM1 finishes its
    // K-split tiles itself, with one counter per tile that the router zeroes.
    const bool streams = moe_expert_ffn_streams((int)dt, A, d, d_ff, E);
    const int n_ctr =
        streams && c.split_bytes ? moe_stream_layer_counters((int)dt, T, k, d, d_ff, E) : 0;
    int32_t *ctr = n_ctr ? at<int32_t>(ws, c.split) + moe_stream_layer_counter_index(T, k, d, d_ff)
                         : nullptr;
    LAUNCH(mark(0), "event");
    LAUNCH(moe_launch_router(x, (int)dt, Wg, T, d, E, k, idx, gw, nullptr, s, ctr, n_ctr),
           "router");
    LAUNCH(mark(1), "event");
    if (streams) {
        // Decode sizes: the weight-streaming GEMM1 groups the assignments
        // itself, and GEMM2 or the pass after it also combines (dispatch and
        // combine stages empty).
        LAUNCH(mark(2), "event");
        LAUNCH(moe_launch_stream_layer(x, idx, k, gw, residual, W1, W3, W2, T, d, d_ff, E, counts,
                                       offsets, row_of, token_of, hbuf,
                                       (float *)o_perm, y,
                                       c.split_bytes ? at<char>(ws, c.split) : nullptr,
                                       c.split_bytes, ctr, ev ? (hipEvent_t)ev[3] : nullptr, s),
               "expert_ffn");
        LAUNCH(mark(4), "event");
        LAUNCH(mark(5), "event");
        return ok();
    }
    LAUNCH(moe_launch_dispatch_index(idx, A, E, k, counts, offsets, row_of, token_of,
                                     at<int32_t>(ws, c.dsc), s),
           "dispatch");
    // The large-tile and weight-streaming expert kernels read each token's
    // row in place through token_of; the others read rows in expert order,
    // so copy each token's row to its k places first.
    const bool gathers = moe_expert_ffn_gathers((int)dt, A, d, d_ff, E);
    if (!gathers)
        LAUNCH(moe_launch_gather_rows(x, (int)dt, T, d, k, row_of, x_perm, s), "gather");
    LAUNCH(mark(2), "event");
    // The W2 GEMM leaves the expert outputs in fp32; the combine rounds once.
    LAUNCH(moe_launch_expert_ffn(gathers ? x : x_perm, gathers ? token_of : nullptr, offsets, W1,
                                 W3, W2, (int)dt, 1, A, d, d_ff, E, hbuf, o_perm,
                                 c.split_bytes ? at<char>(ws, c.split) : nullptr, c.split_bytes,
                                 ev ? (hipEvent_t)ev[3] : nullptr, s),
           "expert_ffn");
    LAUNCH(mark(4), "event");
    LAUNCH(moe_launch_combine(o_perm, 1, row_of, gw, residual, (int)dt, T, d, k, y, s),
           "combine");
    LAUNCH(mark(5), "event");
    return ok();
}

moe_status moe_forward(const void *x, const float *Wg, const void *W1, const void *W3,
                       const void *W2, moe_dtype dt, int64_t T, int d, int d_ff, int E, int k,
                       void *y, void *ws, size_t ws_bytes, void *stream) {
    CHECK(check_shape(T, d, d_ff, E, k, dt, true));
    if (T == 0) return ok();
    REQUIRE_PTR(x, 16);
    REQUIRE_PTR(Wg, 16);
    REQUIRE_PTR(W1, 16);
    REQUIRE_PTR(W3, 16);
    REQUIRE_PTR(W2, 16);
    REQUIRE_PTR(y, 16);
    const Carve c = carve(T, d, d_ff, E, k, dt);
    if (!ws || ws_bytes < c.total)
        return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, c.total);
    REQUIRE_PTR(ws, kAlign);
    return forward_impl(x, Wg, W1, W3, W2, dt, T, d, d_ff, E, k, nullptr, y, nullptr, nullptr,
                        ws, c, nullptr, (hipStream_t)stream);
}

}  // extern "C"

// ---- the layer without a caller workspace ---------------------------------
//
// The fused layer's scratch (routing, grouping, SwiGLU rows, expert outputs,
// split-tile partial sums) lives in one file-scope device array instead of a
// caller workspace.  Each GPU holds its own copy from the first call on it
// until the process ends.  The array's name is a host-side stand-in in host
// code: its device address comes from hipGetSymbolAddress, once per device,
// and only that address is passed to kernels.  Nothing in it has to start at
// zero: every kernel of the layer writes what a later kernel of the same call
// reads.  Calls that overlap on one GPU share the array and race.
static constexpr size_t kStaticScratchBytes = (size_t)96 << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

moe_status static_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (!p || !aligned(p, kAlign))
            return fail(MOE_ERR_HIP, "scratch array at %p is not %zu-byte aligned", p, kAlign);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_forward_noalloc_max_scratch(void) { return kStaticScratchBytes; }

moe_status moe_forward_noalloc(const void *x, const float *Wg, const void *W1, const void *W3,
                               const void *W2, moe_dtype dt, int64_t T, int d, int d_ff, int E,
                               int k, void *y, void *stream) {
    CHECK(check_shape(T, d, d_ff, E, k, dt, true));
    if (T == 0) return ok();
    REQUIRE_PTR(x, 16);
    REQUIRE_PTR(Wg, 16);
    REQUIRE_PTR(W1, 16);
    REQUIRE_PTR(W3, 16);
    REQUIRE_PTR(W2, 16);
    REQUIRE_PTR(y, 16);
    const Carve c = carve(T, d, d_ff, E, k, dt);
    if (c.total > kStaticScratchBytes)
        return fail(MOE_ERR_WORKSPACE,
                    "this shape needs %zu bytes of scratch; the library's static array holds "
                    "%zu (use moe_forward with a workspace)",
                    c.total, kStaticScratchBytes);
    void *ws = nullptr;
    CHECK(static_scratch(&ws));
    return forward_impl(x, Wg, W1, W3, W2, dt, T, d, d_ff, E, k, nullptr, y, nullptr, nullptr,
                        ws, c, nullptr, (hipStream_t)stream);
}

moe_status moe_forward_profiled(const void *x, const float *Wg, const void *W1, const void *W3,
                                const void *W2, moe_dtype dt, int64_t T, int d, int d_ff, int E,
                                int k, void *y, void *ws, size_t ws_bytes, void *const *events,
                                void *stream) {
    CHECK(check_shape(T, d, d_ff, E, k, dt, true));
    if (T == 0) return ok();
    REQUIRE_PTR(x, 16);
    REQUIRE_PTR(Wg, 16);
    REQUIRE_PTR(W1, 16);
    REQUIRE_PTR(W3, 16);
    REQUIRE_PTR(W2, 16);
    REQUIRE_PTR(y, 16);
    if (!events) return fail(MOE_ERR_INVALID_ARG, "events is NULL");
    const Carve c = carve(T, d, d_ff, E, k, dt);
    if (!ws || ws_bytes < c.total)
        return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, c.total);
    REQUIRE_PTR(ws, kAlign);
    return forward_impl(x, Wg, W1, W3, W2, dt, T, d, d_ff, E, k, nullptr, y, nullptr, nullptr,
                        ws, c, events, (hipStream_t)stream);
}

moe_status moe_rmsnorm(const void *h, moe_dtype dt, int64_t T, int d, float eps, void *out,
                       void *stream) {
    CHECK(check_shape(T, d, 64, 1, 1, dt, false));
    if (!(eps >= 0.0f)) return fail(MOE_ERR_INVALID_ARG, "eps must be >= 0");
    if (T == 0) return ok();
    REQUIRE_PTR(h, 16);
    REQUIRE_PTR(out, 16);
    LAUNCH(moe_launch_rmsnorm(h, (int)dt, T, d, eps, out, (hipStream_t)stream), "rmsnorm");
    return ok();
}

moe_status moe_block_forward(void *h, const float *Wg, const void *W1, const void *W3,
                             const void *W2, moe_dtype dt, int64_t T, int d, int d_ff, int E,
                             int k, float eps, int32_t *topk_idx_or_null,
                             float *topk_w_or_null, void *ws, size_t ws_bytes, void *stream) {
    CHECK(check_shape(T, d, d_ff, E, k, dt, true));
    if (!(eps >= 0.0f)) return fail(MOE_ERR_INVALID_ARG, "eps must be >= 0");
    if (T == 0) return ok();
    REQUIRE_PTR(h, 16);
    REQUIRE_PTR(Wg, 16);
    REQUIRE_PTR(W1, 16);
    REQUIRE_PTR(W3, 16);
    REQUIRE_PTR(W2, 16);
    if (topk_idx_or_null && !aligned(topk_idx_or_null, 4))
        return fail(MOE_ERR_INVALID_ARG, "topk_idx_or_null is not 4-byte aligned");
    if (topk_w_or_null && !aligned(topk_w_or_null, 4))
        return fail(MOE_ERR_INVALID_ARG, "topk_w_or_null is not 4-byte aligned");
    const Carve c = carve(T, d, d_ff, E, k, dt);
    if (!ws || ws_bytes < c.total)
        return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, c.total);
    REQUIRE_PTR(ws, kAlign);
    hipStream_t s = (hipStream_t)stream;
    void *xn = at<char>(ws, c.xn);
    LAUNCH(moe_launch_rmsnorm(h, (int)dt, T, d, eps, xn, s), "rmsnorm");
    // h is both the residual and the output: combine reads each element of h
    // before the same lane overwrites it.
    return forward_impl(xn, Wg, W1, W3, W2, dt, T, d, d_ff, E, k, h, h, topk_idx_or_null,
                        topk_w_or_null, ws, c, nullptr, s);
}

}  // extern "C"
