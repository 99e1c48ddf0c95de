// common.h — device helpers and launcher declarations shared by the HIP
// sources of libmoe.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Element types: fp32 or bf16 held as raw 16-bit patterns.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// fp64 -> bf16, one rounding to nearest even straight from the double (no
// intermediate fp32 rounding).  bf16 keeps 7 explicit mantissa bits, so the
// rounding point of a normal double sits at mantissa bit 45.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double v) {
    uint64_t u = (uint64_t)__double_as_longlong(v);
    uint64_t sign = u >> 63;
    uint64_t mag = u & 0x7fffffffffffffffull;
    if (mag >= 0x7ff0000000000000ull)  // Inf / NaN: the fp32 conversion keeps them
        return f32_to_bf16_bits((float)v);
    double a = __longlong_as_double((long long)mag);
    float f;
    if (a < 0x1p-126) {
        // below the fp32 normal range bf16 steps are 2^-133 apart
        f = (float)(rint(a * 0x1p133) * 0x1p-133);
    } else {
        uint64_t lsb = (mag >> 45) & 1ull;
        mag += 0x00000fffffffffffull + lsb;
        mag &= ~0x00001fffffffffffull;
        double r = __longlong_as_double((long long)mag);
        f = (r >= 0x1p128) ? __builtin_inff() : (float)r;  // exact when finite
    }
    return (__float_as_uint(f) >> 16) | (uint32_t)(sign << 15);
}

}  // namespace moe

// ---- launchers (host side, one per kernel family) -------------------------

// zero [zero_n] (may be NULL): int32 counters that workgroup 0 of the router
// sets to 0, for the launch after it.
hipError_t moe_launch_router(const void *x, int dt, const float *Wg, int64_t T, int d, int E,
                             int k, int32_t *idx, float *gw, float *logits, hipStream_t s,
                             int32_t *zero = nullptr, int zero_n = 0);
// Workgroups of the router launch for T tokens (one statistics row each).
int64_t moe_router_blocks(int64_t T);
// Router plus load statistics: part_p [blocks][E] fp64 and part_c [blocks][E]
// int32 scratch; f, P [E] and laux [1] out (fp32).
hipError_t moe_launch_route_balance(const void *x, int dt, const float *Wg, int64_t T, int d,
                                    int E, int k, int32_t *idx, float *gw, double *part_p,
                                    int32_t *part_c, float *f, float *P, float *laux,
                                    hipStream_t s);
// Grouping of A assignments by expert.  `scratch` holds the chunk counts of
// the two-launch form, at least moe_dispatch_scratch_bytes(A, E) bytes; with
// NULL (or where that is 0) one workgroup does it all.
size_t moe_dispatch_scratch_bytes(int64_t A, int E);
hipError_t moe_launch_dispatch_index(const int32_t *idx, int64_t A, int E, int k,
                                     int32_t *counts, int32_t *offsets, int32_t *row_of,
                                     int32_t *token_of, int32_t *scratch, hipStream_t s);
hipError_t moe_launch_gather_rows(const void *x, int dt, int64_t T, int d, int k,
                                  const int32_t *row_of, void *x_perm, hipStream_t s);
// Grouped expert GEMMs over activations already in expert order (x_perm).
// `mid_event` (may be NULL) is recorded between the W1/W3 GEMM and the W2 GEMM.
// `out_f32` != 0: the W2 GEMM writes fp32 expert outputs instead of dt.
// `scratch` (may be NULL) holds partial sums of split tiles, at least
// moe_expert_ffn_scratch_bytes() bytes to be used.  `gather` NULL: act is
// x_perm (rows in expert order); else act is x and expert-order row r is
// x[gather[r]] (token_of), which the kernels of a shape support only if
// moe_expert_ffn_gathers() says so (else hipErrorInvalidValue).
hipError_t moe_launch_expert_ffn(const void *act, const int32_t *gather, const int32_t *offsets,
                                 const void *W1, const void *W3, const void *W2, int dt,
                                 int out_f32, int64_t A, int d, int d_ff, int E, void *hbuf,
                                 void *out, void *scratch, size_t scratch_bytes,
                                 hipEvent_t mid_event, hipStream_t s);
bool moe_expert_ffn_gathers(int dt, int64_t A, int d, int d_ff, int E);
size_t moe_expert_ffn_scratch_bytes(int dt, int64_t A, int d, int d_ff, int E);
// The decode layer's experts on the weight-streaming kernels
// (moe_expert_ffn_streams()): GEMM1 groups the assignments itself (topk_idx,
// k slots per token; counts, offsets, row_of, token_of written out), and
// GEMM2, or the pass after it, also writes y = sum_j gw o_j (+ residual)
// (bf16; o_perm fp32 in between).  scratch: at least
// moe_expert_ffn_scratch_bytes() of the shape (the split-tile scratch).
bool moe_expert_ffn_streams(int dt, int64_t A, int d, int d_ff, int E);
// `ctr` [moe_stream_layer_counters()] (may be NULL when that is 0): counters
// zeroed by an earlier launch on the stream (the router's), with which GEMM1
// finishes its own K-split tiles; NULL: a pass after GEMM1 does.
hipError_t moe_launch_stream_layer(const void *x, const int32_t *topk_idx, int k, const float *gw,
                                   const void *residual, const void *W1, const void *W3,
                                   const void *W2, int64_t T, int d, int d_ff, int E,
                                   int32_t *counts, int32_t *offsets, int32_t *row_of,
                                   int32_t *token_of, void *hbuf, float *o_perm, void *y,
                                   void *scratch, size_t scratch_bytes, int32_t *ctr,
                                   hipEvent_t gemm1_done, hipStream_t s);
// Counters of the layer's GEMM1 at T tokens (0 where its GEMM1 is not the
// tile kernel) and where they sit in the split-tile scratch (int32 index).
int moe_stream_layer_counters(int dt, int64_t T, int k, int d, int d_ff, int E);
int64_t moe_stream_layer_counter_index(int64_t T, int k, int d, int d_ff);
// Name of the kernel family that runs the experts for this shape.
const char *moe_expert_ffn_kernel_name(int dt, int64_t A, int d, int d_ff, int E);
// The same for the experts of the fused layer (moe_forward and friends) at T
// tokens, which may differ: one to eight tokens take the column kernels.
const char *moe_forward_kernel_name(int dt, int64_t T, int k, int d, int d_ff, int E);
// The same experts for decode-sized batches (few rows per expert).
hipError_t moe_launch_skinny_ffn(const void *x_perm, const int32_t *offsets, const void *W1,
                                 const void *W3, const void *W2, int dt, int out_f32, int64_t A,
                                 int d, int d_ff, int E, void *hbuf, void *out,
                                 hipEvent_t mid_event, hipStream_t s);
// `out_f32` != 0: out_perm holds fp32 expert outputs (y, residual stay dt).
hipError_t moe_launch_combine(const void *out_perm, int out_f32, const int32_t *row_of,
                              const float *gw, const void *residual, int dt, int64_t T, int d,
                              int k, void *y, hipStream_t s);
hipError_t moe_launch_rmsnorm(const void *h, int dt, int64_t T, int d, float eps, void *out,
                              hipStream_t s);
