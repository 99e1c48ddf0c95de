// gemm_common.h — device helpers shared by the expert GEMM kernels
// (expert_gemm.hip, wide_gemm.hip): MFMA steps, output stores, explicit
// waits, the fence-free barrier, global-to-LDS loads and the swizzled LDS
// layout of a stage.
#pragma once

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"

namespace moe {

template <typename T>
struct ElemSize;
template <>
struct ElemSize<float> {
    static constexpr int value = 4;
};
template <>
struct ElemSize<bf16_t> {
    static constexpr int value = 2;
};

typedef float f32x16 __attribute__((ext_vector_type(16)));

// acc += A_frag * B_frag over one 32-byte k-step: 32 rows x 32 cols.
template <typename T>
__device__ __forceinline__ f32x16 mma_step(i32x4 a, i32x4 b, f32x16 c);

template <>
__device__ __forceinline__ f32x16 mma_step<bf16_t>(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16 mma_step<float>(i32x4 a, i32x4 b, f32x16 c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(a.x), __int_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(a.y), __int_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(a.z), __int_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(a.w), __int_as_float(b.w), c, 0, 0, 0);
    return c;
}

// acc += A_frag * B_frag over 32 bf16 k: 16 rows x 16 cols.  Lane l holds
// row l % 16 (A) or column l % 16 (B) at k 8 (l / 16) .. + 8, and D rows
// 4 (l / 16) .. + 4 of column l % 16.  Under random data this form sustains
// about a quarter more throughput on MI355X than the 32 x 32 x 16 one.
__device__ __forceinline__ f32x4 mma16(i32x4 a, i32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// The grouped GEMMs' per-expert table, built by one whole wave (E <= 64):
// lo[i] = expert i's first row, cnt[i] = its rows, first[i] = the tiles of
// the experts before it (first[E] = all tiles), for token tiles of `bt` rows
// times `col_tiles` column tiles.  Every lane loads its two offsets at once
// and a shuffle scan adds the tile counts, so the table costs one memory
// round trip instead of one per expert.  Offsets are clamped to [0, A] so no
// row index leaves the buffers even for a malformed offsets array.  The
// caller syncs the workgroup before the table is read.
__device__ __forceinline__ void build_expert_table(const int32_t *__restrict__ offsets, int E,
                                                   int A, int bt, int col_tiles, int *lo,
                                                   int *cnt, int *first) {
    const int lane = threadIdx.x & (kWave - 1);
    const int o0 = lane < E ? offsets[lane] : 0;
    const int o1 = lane < E ? offsets[lane + 1] : 0;
    const int l = min(max(o0, 0), A);
    const int h = min(max(o1, l), A);
    const int tiles = lane < E ? (h - l + bt - 1) / bt * col_tiles : 0;
    int incl = tiles;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
    }
    if (lane < E) {
        lo[lane] = l;
        cnt[lane] = h - l;
        first[lane] = incl - tiles;
    }
    if (lane == E - 1) first[E] = incl;
}

template <typename T>
__device__ __forceinline__ void store4(T *out, float v0, float v1, float v2, float v3);

template <>
__device__ __forceinline__ void store4<float>(float *out, float v0, float v1, float v2,
                                              float v3) {
    *(float4 *)out = make_float4(v0, v1, v2, v3);
}

template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t *out, float v0, float v1, float v2,
                                               float v3) {
    *(uint2 *)out = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
}

// silu(u) = u / (1 + e^-u) from the hardware base-2 exponential and
// reciprocal (about 1 ulp each, a few ulp together: far inside bf16 and the
// fp32 tolerances, and a fraction of the instructions of expf and an IEEE
// division).  The limits come out right: u -> -inf gives 1 / inf = 0, and
// u -> +inf gives e^-u = 0, so u itself.
__device__ __forceinline__ float silu(float u) {
    const float e = __builtin_amdgcn_exp2f(u * -1.4426950408889634f);  // -u log2(e)
    return u * __builtin_amdgcn_rcpf(1.0f + e);
}

// s_waitcnt constraining vmcnt to N and lgkmcnt to 0 (expcnt free); gfx9
// encoding: vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8].
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier without a memory fence: the explicit waits decide what
// has landed in LDS; the empty asm statements and scheduling barriers keep
// the compiler from moving memory operations across it.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void dma16(const char *g, char *lds) {
    __builtin_amdgcn_global_load_lds((const void *)g,
                                     (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// The same load with the non-temporal hint, for data read once (a weight
// stream): it lifts the sustained HBM read rate on MI355X from about 6.2 to
// about 7 TB/s.
__device__ __forceinline__ void dma16_nt(const char *g, char *lds) {
    __builtin_amdgcn_global_load_lds((const void *)g,
                                     (__attribute__((address_space(3))) void *)lds, 16, 0,
                                     2 /* nt */);
}

// One dword per lane (256 bytes per wave): a load that only keeps a wave's
// count of loads in flight the same from stage to stage (into LDS nothing
// reads, from an address the caches hold).
__device__ __forceinline__ void dma4(const char *g, char *lds) {
    __builtin_amdgcn_global_load_lds((const void *)g,
                                     (__attribute__((address_space(3))) void *)lds, 4, 0, 0);
}

// Byte offset of 16-byte chunk c of 1 KiB row r in a buffer of such rows
// (the weight-streaming kernels' layout): chunk c of row r sits at chunk
// c ^ (r & 15), so sixteen rows read at one chunk hit sixteen bank groups
// while every load instruction still writes one contiguous row piece.
__device__ __forceinline__ int swz1k(int r, int c) { return r * 1024 + ((c ^ (r & 15)) << 4); }

// Activation row of the expert-order rows rb + lane / (64 / ROWS) (the rows
// one load instruction covers), rows past `last` repeating `last`.  With a
// gather map (the token of each expert-order row) the rows are the tokens'
// own rows, read in place instead of from a gathered copy.  The map is read
// with wave-uniform addresses through the scalar cache: those loads count on
// lgkmcnt, so they never wait behind the vector-memory loads of a ring in
// flight (vmcnt retires in issue order).
template <int ROWS>
__device__ __forceinline__ int act_row(const int32_t *__restrict__ gather, int rb, int last,
                                       int lane) {
    const int own = min(rb + lane / (64 / ROWS), last);
    if (!gather) return own;
    int v = 0;
#pragma unroll
    for (int q = 0; q < ROWS; ++q) {
        const int r = __builtin_amdgcn_readfirstlane(min(rb + q, last));
        const int t = __builtin_amdgcn_readfirstlane(gather[r]);
        v = (lane == q) ? t : v;
    }
    return __shfl(v, lane / (64 / ROWS));
}

// Byte offset of 16-byte chunk c of LDS row r within a stage.
__device__ __forceinline__ int lds_off(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

struct TileInfo {
    int e, row0, mrem, n0;
    int mt;  // token tile index within its expert (wide_gemm.hip)
};

// Raises the dynamic LDS limit of kernel KERN, once per device: the runtime
// call is not free, and made before every launch it shows as an idle gap
// ahead of the kernel.  (One flag word per kernel instantiation.)
template <auto KERN>
static inline hipError_t set_lds_limit(int bytes) {
    static std::atomic<unsigned long long> done{0};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const unsigned long long bit = 1ull << (dev & 63);
    if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
    err = hipFuncSetAttribute((const void *)KERN, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (err == hipSuccess) done.fetch_or(bit, std::memory_order_release);
    return err;
}

static inline int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 256;
    return cus;
}

// What the decode path folds into the weight-streaming kernels
// (stream_gemm.hip, stream_cols.hip): no dispatch launch before GEMM1 and
// no separate combine launch.  All NULL / 0: the kernels run alone.
struct StreamFuse {
    // GEMM1 groups the assignments itself: topk_idx [A] holds the expert of
    // every (token, slot), k slots per token; every workgroup derives the
    // same stable grouping, workgroup 0 writes it out (counts [E], offsets
    // [E+1], row_of [A], token_of [A]).
    const int32_t *topk_idx;
    int k;
    int32_t *counts, *offsets, *row_of, *token_of;
    // y[t] = sum_j gw[t][j] o[row_of[t][j]] (+ residual[t]) for the T tokens,
    // formed by the column kernels' GEMM2 or by the pass after the tile
    // kernels' GEMM2.
    const float *gw;
    const bf16_t *residual;
    bf16_t *y;
    int T;
    // GEMM1 of the layer: one counter per tile, zero at the launch; the
    // pieces of split tiles are written through to memory and the last
    // workgroup to count a tile's piece sums them (no pass after GEMM1).
    int32_t *ctr;
};

// Weight-streaming expert GEMMs for decode-sized bf16 batches
// (stream_gemm.hip).
// `partial` (may be NULL) is scratch for the pieces of split tiles at the
// smallest batches, at least stream_partial_bytes() bytes (0: none used).
bool stream_supported(int64_t A, int d, int d_ff, int E);
size_t stream_partial_bytes(int64_t A, int d, int d_ff, int E);
// The layer GEMM1's counters (one per tile, stream_gemm1_tiles_max of them)
// start at int32 index stream_counter_index() of that scratch.
int64_t stream_gemm1_tiles_max(int64_t A, int d_ff, int E);
int64_t stream_counter_index(int64_t A, int d, int d_ff);
hipError_t launch_stream_ffn(const void *act, const int32_t *gather, const int32_t *offsets,
                             const void *W1, const void *W3, const void *W2, int out_f32,
                             int64_t A, int d, int d_ff, int E, void *hbuf, void *out,
                             float *partial, size_t partial_bytes, hipEvent_t mid,
                             hipStream_t s);
// The decode layer's experts with the grouping folded into GEMM1 and the
// combine into GEMM2 or the pass after it (out: fp32 expert outputs; x rows
// read in place; fuse.offsets receives the grouping).  The tile kernels need
// the split scratch (partial, stream_partial_bytes()) here.
hipError_t launch_stream_fused(const void *x, const void *W1, const void *W3, const void *W2,
                               int64_t A, int d, int d_ff, int E, void *hbuf, float *out,
                               float *partial, size_t partial_bytes, const StreamFuse &fuse,
                               hipEvent_t gemm1_done, hipStream_t s);
// The decode layer's experts for one to eight tokens (stream_cols.hip):
// every workgroup streams its own columns of every active expert over the
// whole K; GEMM1 writes h and the grouping (fuse.counts, offsets, row_of,
// token_of), GEMM2 writes y (fuse.gw, residual, y, T, k, topk_idx).
bool stream_cols_supported(int64_t T, int k, int d, int d_ff, int E);
// GEMM2 alone on the column kernel for nine to 32 tokens (16 token rows per
// chunk of an expert's rows), after the tile kernel's GEMM1: hbuf holds h in
// grouped rows; f.topk_idx, k, gw, residual, y and T as for the above.
bool stream_cols_w2_supported(int64_t T, int k, int d, int d_ff, int E);
hipError_t launch_stream_cols_w2(const void *hbuf, const void *W2, int64_t T, int d, int d_ff,
                                 int E, const StreamFuse &f, hipStream_t s);
hipError_t launch_stream_cols(const void *x, const void *W1, const void *W3, const void *W2,
                              int64_t T, int d, int d_ff, int E, void *hbuf,
                              const StreamFuse &f, hipEvent_t gemm1_done, hipStream_t s);

// Wide-tile expert GEMMs (wide_gemm.hip), bf16 only.  `partial` (may be
// NULL) is scratch for split tiles, at least wide_partial_bytes() bytes.
size_t wide_partial_bytes(int64_t A, int E);
// GEMM2 alone on the wide kernels (h in expert order, rows [offsets[0],
// offsets[E]) ), for the mixed path: grouped GEMM1, wide GEMM2.
hipError_t launch_wide_w2(const void *hbuf, const int32_t *offsets, const void *W2, int out_f32,
                          int64_t A, int d, int d_ff, int E, void *out, float *partial,
                          size_t partial_bytes, hipStream_t s);
// Token-tile height (128 or 256) the wide kernels use for A rows over E experts.
int wide_token_tile(int64_t A, int E);
bool wide_supported(int64_t A, int d, int d_ff);
hipError_t launch_wide_ffn(const void *act, const int32_t *gather, const int32_t *offsets,
                           const void *W1, const void *W3, const void *W2, int out_f32, int64_t A,
                           int d, int d_ff, int E, void *hbuf, void *out, float *partial,
                           size_t partial_bytes, hipEvent_t mid, hipStream_t s);

}  // namespace moe
