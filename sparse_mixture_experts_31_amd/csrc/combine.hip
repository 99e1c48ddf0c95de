// combine.hip — the gated sum back in token order, and the block's RMSNorm.
//
// combine_kernel: y = sum_j g_j E_j(x) (tokentrails lineage, step "Two
//   experts per token": y = ga.Ea(x) + gb.Eb(x)), optionally plus a residual
//   (the block's h + moe(...), tokentrails Code listing).  One wave per
//   512-element piece of a token's row, so even a handful of tokens spread
//   over many waves; each lane handles 8 consecutive elements with 16-byte
//   loads, sums in fp32 in slot order and rounds once.
// rmsnorm_kernel: h / sqrt(mean(h^2) + eps) with unit gain (tokentrails Code
//   listing; the block is LLaMA's).  The sum of squares and the scale are
//   fp64 and each output is rounded once from fp64 to the activation dtype,
//   so the bf16 activations the router sees do not depend on reduction order
//   or on fp32 rounding of the scale.
#include "common.h"

namespace moe {

template <typename T>
struct Vec8;

template <>
struct Vec8<bf16_t> {
    static __device__ __forceinline__ void load(const bf16_t *p, float (&v)[8]) {
        const uint4 a = *(const uint4 *)p;
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(bf16_t *p, const float (&v)[8]) {
        *(uint4 *)p = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                 pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    }
};

template <>
struct Vec8<float> {
    static __device__ __forceinline__ void load(const float *p, float (&v)[8]) {
        const float4 a = *(const float4 *)p;
        const float4 b = *(const float4 *)(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    static __device__ __forceinline__ void store(float *p, const float (&v)[8]) {
        *(float4 *)p = make_float4(v[0], v[1], v[2], v[3]);
        *(float4 *)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
};

constexpr int kRowWaves = 4;
constexpr int kCombinePiece = kWave * 8;  // elements of a row per combine wave

// TI: type of the expert outputs (the activation type, or fp32 when the
// fused layer keeps them unrounded); T: residual and output type.
template <typename TI, typename T>
__global__ __launch_bounds__(kRowWaves *kWave) void combine_kernel(
    const TI *__restrict__ out_perm, const int32_t *__restrict__ row_of,
    const float *__restrict__ gw, const T *residual, int64_t T_, int d, int k, T *y) {
    const int lane = threadIdx.x & (kWave - 1);
    const int nch = (d + kCombinePiece - 1) / kCombinePiece;  // pieces per row
    const int64_t wv = (int64_t)blockIdx.x * kRowWaves + threadIdx.x / kWave;
    const int64_t t = wv / nch;
    const int i = (int)(wv - t * nch) * kCombinePiece + lane * 8;
    if (t >= T_ || i >= d) return;
    int rows[8];
    float g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        rows[j] = (j < k) ? row_of[t * k + j] : -1;
        g[j] = (j < k) ? gw[t * k + j] : 0.f;
    }
    {
        float acc[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (rows[j] >= 0) {
                float o[8];
                Vec8<TI>::load(out_perm + (int64_t)rows[j] * d + i, o);
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[c] = fmaf(g[j], o[c], acc[c]);
            }
        }
        if (residual) {
            float r[8];
            Vec8<T>::load(residual + t * d + i, r);
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] += r[c];
        }
        Vec8<T>::store(y + t * d + i, acc);
    }
}

template <typename T>
__device__ __forceinline__ void store8_from_f64(T *p, const double (&v)[8]);

template <>
__device__ __forceinline__ void store8_from_f64<bf16_t>(bf16_t *p, const double (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = f64_to_bf16_bits(v[2 * i]) | (f64_to_bf16_bits(v[2 * i + 1]) << 16);
    *(uint4 *)p = make_uint4(w[0], w[1], w[2], w[3]);
}

template <>
__device__ __forceinline__ void store8_from_f64<float>(float *p, const double (&v)[8]) {
    *(float4 *)p = make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
    *(float4 *)(p + 4) = make_float4((float)v[4], (float)v[5], (float)v[6], (float)v[7]);
}

template <typename T>
__global__ __launch_bounds__(kRowWaves *kWave) void rmsnorm_kernel(const T *h, int64_t T_,
                                                                   int d, double eps, T *out) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * kRowWaves + threadIdx.x / kWave;
    if (t >= T_) return;
    const T *row = h + t * d;
    double ss = 0.0;
    for (int i = lane * 8; i < d; i += kWave * 8) {
        float v[8];
        Vec8<T>::load(row + i, v);
#pragma unroll
        for (int c = 0; c < 8; ++c) ss = fma((double)v[c], (double)v[c], ss);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const double scale = 1.0 / sqrt(ss / d + eps);
    for (int i = lane * 8; i < d; i += kWave * 8) {
        float v[8];
        Vec8<T>::load(row + i, v);
        double o[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] = (double)v[c] * scale;
        store8_from_f64<T>(out + t * d + i, o);
    }
}

}  // namespace moe

hipError_t moe_launch_combine(const void *out_perm, int out_f32, const int32_t *row_of,
                              const float *gw, const void *residual, int dt, int64_t T, int d,
                              int k, void *y, hipStream_t s) {
    using namespace moe;
    const int64_t waves = T * ((d + kCombinePiece - 1) / kCombinePiece);
    const dim3 grid((unsigned)((waves + kRowWaves - 1) / kRowWaves)), block(kRowWaves * kWave);
    if (dt == 0)
        hipLaunchKernelGGL((combine_kernel<float, float>), grid, block, 0, s,
                           (const float *)out_perm, row_of, gw, (const float *)residual, T, d, k,
                           (float *)y);
    else if (out_f32)
        hipLaunchKernelGGL((combine_kernel<float, bf16_t>), grid, block, 0, s,
                           (const float *)out_perm, row_of, gw, (const bf16_t *)residual, T, d, k,
                           (bf16_t *)y);
    else
        hipLaunchKernelGGL((combine_kernel<bf16_t, bf16_t>), grid, block, 0, s,
                           (const bf16_t *)out_perm, row_of, gw, (const bf16_t *)residual, T, d,
                           k, (bf16_t *)y);
    return hipGetLastError();
}

hipError_t moe_launch_rmsnorm(const void *h, int dt, int64_t T, int d, float eps, void *out,
                              hipStream_t s) {
    using namespace moe;
    const dim3 grid((unsigned)((T + kRowWaves - 1) / kRowWaves)), block(kRowWaves * kWave);
    if (dt == 0)
        hipLaunchKernelGGL(rmsnorm_kernel<float>, grid, block, 0, s, (const float *)h, T, d,
                           (double)eps, (float *)out);
    else
        hipLaunchKernelGGL(rmsnorm_kernel<bf16_t>, grid, block, 0, s, (const bf16_t *)h, T, d,
                           (double)eps, (bf16_t *)out);
    return hipGetLastError();
}
