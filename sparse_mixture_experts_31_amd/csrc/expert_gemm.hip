// expert_gemm.hip — the experts as grouped GEMMs on the gfx950 matrix cores.
//
// Every expert is the SwiGLU MLP W2 (silu(W1 x) * W3 x) (fdeinterviews
// breakdown, "The paper in one minute"; tokentrails lineage, Code listing).
// After dispatch the rows of expert e form one contiguous block
// [offsets[e], offsets[e+1]), so the experts are two grouped GEMMs:
//   GEMM1 (SWIGLU=true):  h[r][n] = silu(sum_k X[r][k] W1_e[n][k]) * (sum_k X[r][k] W3_e[n][k])
//   GEMM2 (SWIGLU=false): o[r][n] = sum_k h[r][k] W2_e[n][k]
// Both operands are K-contiguous, the natural layout of the MFMA operands.
//
// Mapping.  A workgroup owns BN weight rows (n) of one expert — for GEMM1 the
// same BN rows of both W1 and W3 — and BM token rows (m) of that expert.
// Weights play the MFMA "A" operand (16 rows x 32 k) and tokens the "B"
// operand (32 k x 16 cols) of v_mfma_f32_16x16x32_bf16 (fp32:
// v_mfma_f32_16x16x4_f32, four per 16-byte fragment), accumulating in fp32.
// An output fragment then holds four consecutive n of one token row, which
// the epilogue writes as one 8-byte (bf16) or 16-byte (fp32) store.  The
// silu(u) * v product is formed in registers from the u and v accumulators of
// the same lane, so GEMM1 never writes u or v.
//
// Pipeline.  K advances in stages of 128 bytes per row (64 bf16 / 32 fp32).
// Each thread loads its share of the next stage with 16-byte global loads
// into registers while the matrix cores work on the current stage from LDS;
// the registers then go to the other LDS buffer (double buffering, one
// barrier per stage).  LDS rows are 128 bytes with the 16-byte chunk index
// XOR-swizzled by (row & 7), so the column of 16-byte reads an MFMA fragment
// needs spreads across banks.
//
// Ragged tiles.  Token rows past the expert's count read a valid clamped row
// and are never stored; weight rows past N are clamped likewise.  A
// workgroup whose tile index lies beyond the experts' total tile count exits
// at once (the grid is sized by an upper bound so the host never reads the
// counts back).
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

// acc += A_frag * B_frag over one 64-byte k-step: 16 rows x 16 cols.
template <typename T>
__device__ __forceinline__ f32x4 mma_step(i32x4 a, i32x4 b, f32x4 c);

template <>
__device__ __forceinline__ f32x4 mma_step<bf16_t>(i32x4 a, i32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4 mma_step<float>(i32x4 a, i32x4 b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a.x), __int_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a.y), __int_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a.z), __int_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a.w), __int_as_float(b.w), c, 0, 0, 0);
    return c;
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

__device__ __forceinline__ float silu(float u) { return u / (1.0f + expf(-u)); }

__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

template <int BN, int BM, int WN, int WM, bool SWIGLU, typename T>
struct GemmShape {
    static constexpr int kThreads = WN * WM * kWave;
    static constexpr int kWRows = SWIGLU ? 2 * BN : BN;  // weight rows staged per stage
    static constexpr int kRows = kWRows + BM;
    static constexpr int kStageBytes = kRows * 128;
    static constexpr int kLdsBytes = 2 * kStageBytes;
    static constexpr int kChunksPerThread = kRows * 8 / kThreads;
    static constexpr int TN = BN / WN / 16;  // 16-row fragments per wave along n
    static constexpr int TM = BM / WM / 16;  // 16-col fragments per wave along m
    static constexpr int kKStep = 128 / ElemSize<T>::value;  // K elements per stage
    static_assert(kRows * 8 % kThreads == 0, "stage must split evenly over threads");
    static_assert(TN >= 1 && TM >= 1, "wave tile too small");
    static_assert(BN % (WN * 16) == 0 && BM % (WM * 16) == 0, "tile shape");
};

template <int BN, int BM, int WN, int WM, bool SWIGLU, typename T>
__global__ __launch_bounds__(WN *WM *kWave) void grouped_gemm_kernel(
    const T *__restrict__ act, const int32_t *__restrict__ gather, int64_t act_ld,
    const T *__restrict__ Wa, const T *__restrict__ Wb, const int32_t *__restrict__ offsets,
    int E, int N, int K, int A, T *__restrict__ out, int n_tiles) {
    using S = GemmShape<BN, BM, WN, WM, SWIGLU, T>;
    constexpr int CPT = S::kChunksPerThread;
    constexpr int TN = S::TN, TM = S::TM;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int bx = blockIdx.x % n_tiles;
    const int by = blockIdx.x / n_tiles;

    // Which expert and which of its token tiles this workgroup owns.  The
    // offsets are clamped to [0, A] so that no row index leaves the buffers
    // even for a malformed offsets array.
    int e = -1, mt = 0, before = 0, lo = 0, hi = 0;
    for (int i = 0; i < E; ++i) {
        lo = min(max(offsets[i], 0), A);
        hi = min(max(offsets[i + 1], lo), A);
        const int tiles = (hi - lo + BM - 1) / BM;
        if (by < before + tiles) {
            e = i;
            mt = by - before;
            break;
        }
        before += tiles;
    }
    if (e < 0) return;  // uniform over the workgroup
    const int row0 = lo + mt * BM;
    const int mrem = min(BM, hi - row0);
    const int n0 = bx * BN;

    // This thread's chunks of every stage: fixed rows, fixed 16-byte columns.
    const char *src[CPT];
    int dst[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int q = i * S::kThreads + tid;
        const int r = q >> 3, c = q & 7;
        dst[i] = swz(r, c);
        if (r < S::kWRows) {
            const T *W = (SWIGLU && r >= BN) ? Wb : Wa;
            const int nr = min(n0 + (SWIGLU ? r % BN : r), N - 1);
            src[i] = (const char *)(W + ((int64_t)e * N + nr) * K) + c * 16;
        } else {
            const int m = min(r - S::kWRows, mrem - 1);
            const int64_t arow = gather ? (int64_t)gather[row0 + m] : (int64_t)(row0 + m);
            src[i] = (const char *)(act + arow * act_ld) + c * 16;
        }
    }

    f32x4 accu[TN][TM];
    f32x4 accv[SWIGLU ? TN : 1][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            accu[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (SWIGLU) accv[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    i32x4 regs[CPT];
    const int n_stages = K / S::kKStep;
    const int wn = wave % WN, wm = wave / WN;
    const int wrow0 = wn * (BN / WN);  // this wave's first weight row (u block)
    const int xrow0 = wm * (BM / WM);  // this wave's first token row

#pragma unroll
    for (int i = 0; i < CPT; ++i) regs[i] = *(const i32x4 *)src[i];
#pragma unroll
    for (int i = 0; i < CPT; ++i) *(i32x4 *)(smem + dst[i]) = regs[i];
    __syncthreads();

    for (int s = 0; s < n_stages; ++s) {
        const int buf = s & 1;
        if (s + 1 < n_stages) {
#pragma unroll
            for (int i = 0; i < CPT; ++i)
                regs[i] = *(const i32x4 *)(src[i] + (int64_t)(s + 1) * 128);
        }
        const char *sW = smem + buf * S::kStageBytes;
        const char *sX = sW + S::kWRows * 128;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int c = ks * 4 + (lane >> 4);
            i32x4 xf[TM];
#pragma unroll
            for (int j = 0; j < TM; ++j) {
                const int r = xrow0 + j * 16 + (lane & 15);
                xf[j] = *(const i32x4 *)(sX + swz(r, c));
            }
#pragma unroll
            for (int i = 0; i < TN; ++i) {
                const int r = wrow0 + i * 16 + (lane & 15);
                const i32x4 wf = *(const i32x4 *)(sW + swz(r, c));
#pragma unroll
                for (int j = 0; j < TM; ++j) accu[i][j] = mma_step<T>(wf, xf[j], accu[i][j]);
                if constexpr (SWIGLU) {
                    const i32x4 vf = *(const i32x4 *)(sW + swz(BN + r, c));
#pragma unroll
                    for (int j = 0; j < TM; ++j) accv[i][j] = mma_step<T>(vf, xf[j], accv[i][j]);
                }
            }
        }
        if (s + 1 < n_stages) {
            char *nb = smem + (buf ^ 1) * S::kStageBytes;
#pragma unroll
            for (int i = 0; i < CPT; ++i) *(i32x4 *)(nb + dst[i]) = regs[i];
        }
        __syncthreads();
    }

    // Epilogue: fragment (i, j) element q is D[n = 4*(lane/16) + q][m = lane % 16].
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        const int n = n0 + wrow0 + i * 16 + 4 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int m = xrow0 + j * 16 + (lane & 15);
            if (m < mrem && n < N) {
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[q] = accu[i][j][q];
                    if constexpr (SWIGLU) v[q] = silu(v[q]) * accv[i][j][q];
                }
                store4<T>(out + (int64_t)(row0 + m) * N + n, v[0], v[1], v[2], v[3]);
            }
        }
    }
}

template <int BN, int BM, int WN, int WM, bool SWIGLU, typename T>
static hipError_t launch_grouped(const void *act, const int32_t *gather, int64_t act_ld,
                                 const void *Wa, const void *Wb, const int32_t *offsets, int E,
                                 int N, int K, int64_t A, void *out, hipStream_t s) {
    using S = GemmShape<BN, BM, WN, WM, SWIGLU, T>;
    auto kern = grouped_gemm_kernel<BN, BM, WN, WM, SWIGLU, T>;
    // LDS beyond the 64 KiB default must be requested per kernel (the call
    // is cheap and keeps the library free of cached per-device state).
    hipError_t err = hipFuncSetAttribute((const void *)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         S::kLdsBytes);
    if (err != hipSuccess) return err;
    const int n_tiles = (N + BN - 1) / BN;
    // sum_e ceil(c_e / BM) <= ceil(A / BM) + E - 1
    const int64_t m_bound = (A + BM - 1) / BM + E - 1;
    const int64_t blocks = (int64_t)n_tiles * m_bound;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(S::kThreads), S::kLdsBytes, s,
                       (const T *)act, gather, act_ld, (const T *)Wa, (const T *)Wb, offsets,
                       E, N, K, (int)A, (T *)out, n_tiles);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_ffn_typed(const void *act, const int32_t *gather,
                                   const int32_t *offsets, const void *W1, const void *W3,
                                   const void *W2, int64_t A, int d, int d_ff, int E,
                                   void *hbuf, void *out, hipEvent_t mid, hipStream_t s) {
    hipError_t err;
    // Few rows per expert (decode): narrow token tiles so the weights stream
    // once.  Many rows (prefill): wide tiles for operand reuse.
    const bool few = A < 64LL * E;
    if (few) {
        err = launch_grouped<64, 32, 4, 1, true, T>(act, gather, d, W1, W3, offsets, E, d_ff, d,
                                                     A, hbuf, s);
        if (err == hipSuccess && mid) err = hipEventRecord(mid, s);
        if (err != hipSuccess) return err;
        return launch_grouped<128, 32, 4, 1, false, T>(hbuf, nullptr, d_ff, W2, nullptr,
                                                        offsets, E, d, d_ff, A, out, s);
    }
    err = launch_grouped<128, 128, 4, 2, true, T>(act, gather, d, W1, W3, offsets, E, d_ff, d,
                                                   A, hbuf, s);
    if (err == hipSuccess && mid) err = hipEventRecord(mid, s);
    if (err != hipSuccess) return err;
    return launch_grouped<256, 128, 4, 2, false, T>(hbuf, nullptr, d_ff, W2, nullptr, offsets,
                                                     E, d, d_ff, A, out, s);
}

}  // namespace moe

hipError_t moe_launch_expert_ffn(const void *act, const int32_t *gather, const int32_t *offsets,
                                 const void *W1, const void *W3, const void *W2, int dt,
                                 int64_t A, int d, int d_ff, int E, void *hbuf, void *out,
                                 hipEvent_t mid, hipStream_t s) {
    if (dt == 0)
        return moe::launch_ffn_typed<float>(act, gather, offsets, W1, W3, W2, A, d, d_ff, E,
                                            hbuf, out, mid, s);
    return moe::launch_ffn_typed<moe::bf16_t>(act, gather, offsets, W1, W3, W2, A, d, d_ff, E,
                                              hbuf, out, mid, s);
}
