// skinny_gemm.hip — the expert GEMMs when every expert holds only a few rows
// (decode-sized batches).
//
// Same arithmetic as expert_gemm.hip (SwiGLU experts, fdeinterviews
// breakdown "The paper in one minute"; tokentrails lineage, Code listing),
// but here the work is a stream over the active experts' weights: at T = 32
// each expert sees ~8 rows, so every weight byte feeds only a handful of
// multiply-adds and HBM bandwidth is the bound.  The kernel is shaped for
// memory-level parallelism rather than matrix-core reuse:
//   - one workgroup per tile of BN weight rows (W1 and W3 rows for GEMM1) by
//     BM tokens of one expert; a decode batch has at most one token tile per
//     expert, so each weight row is read exactly once;
//   - K advances 128 bytes per stage; each thread loads its share of the next
//     stage with 16-byte loads into registers while the current stage is
//     consumed from LDS (double buffer, one barrier per stage).  Eight
//     consecutive lanes cover one 128-byte row segment, so every load
//     instruction moves whole cache lines;
//   - small tiles and 40 KiB of LDS let several workgroups share a CU, which
//     keeps many loads in flight;
//   - v_mfma_f32_16x16x32_bf16 (fp32 data: v_mfma_f32_16x16x4_f32) with the
//     weights as the 16-row "A" operand and up to 32 tokens as two 16-column
//     "B" operands; fragments wholly past the expert's rows are skipped.
// LDS rows are 128 bytes with the 16-byte chunk index XOR (row >> 1) & 7,
// which keeps the column reads of an MFMA operand conflict-free.
#include "common.h"

namespace moe {

template <typename T>
struct SkinnyElem;
template <>
struct SkinnyElem<float> {
    static constexpr int size = 4;
};
template <>
struct SkinnyElem<bf16_t> {
    static constexpr int size = 2;
};

// acc += A_frag * B_frag over one 64-byte k-step: 16 rows x 16 cols.
template <typename T>
__device__ __forceinline__ f32x4 mma16(i32x4 a, i32x4 b, f32x4 c);

template <>
__device__ __forceinline__ f32x4 mma16<bf16_t>(i32x4 a, i32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4 mma16<float>(i32x4 a, i32x4 b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a.x), __int_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a.y), __int_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a.z), __int_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a.w), __int_as_float(b.w), c, 0, 0, 0);
    return c;
}

template <typename T>
__device__ __forceinline__ void put4(T *out, float v0, float v1, float v2, float v3);

template <>
__device__ __forceinline__ void put4<float>(float *out, float v0, float v1, float v2, float v3) {
    *(float4 *)out = make_float4(v0, v1, v2, v3);
}

template <>
__device__ __forceinline__ void put4<bf16_t>(bf16_t *out, float v0, float v1, float v2,
                                             float v3) {
    *(uint2 *)out = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
}

__device__ __forceinline__ float silu_f(float u) { return u / (1.0f + expf(-u)); }

__device__ __forceinline__ int swz128(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

template <int BN, int BM, int WN, int WM, bool SWIGLU, typename T>
struct SkinnyCfg {
    static constexpr int kThreads = WN * WM * kWave;
    static constexpr int kWRows = SWIGLU ? 2 * BN : BN;  // weight rows staged per stage
    static constexpr int kRows = kWRows + BM;
    static constexpr int kStageBytes = kRows * 128;
    static constexpr int kLdsBytes = 2 * kStageBytes;
    static constexpr int CPT = kRows * 8 / kThreads;  // 16-byte chunks per thread per stage
    static constexpr int TN = BN / WN / 16;            // 16-row weight fragments per wave
    static constexpr int TM = BM / WM / 16;            // 16-col token fragments per wave
    static constexpr int kKStep = 128 / SkinnyElem<T>::size;  // K elements per stage
    static_assert(kRows * 8 % kThreads == 0, "stage must split evenly over threads");
    static_assert(TN >= 1 && TM >= 1, "wave tile too small");
    static_assert(BN % (WN * 16) == 0 && BM % (WM * 16) == 0, "tile shape");
    static_assert(kLdsBytes <= 64 * 1024, "static LDS");
    static_assert(kWRows * 8 % kThreads == 0, "a thread's chunk i is all weight or all token rows");
    // chunks [0, NW) of every thread hold weight rows, the rest token rows
    static constexpr int NW = kWRows * 8 / kThreads;
};

// Weight chunks are read once per call: non-temporal loads stream them past
// the caches, which lifts the sustained HBM read rate (measured on MI355X:
// about 7 TB/s against about 6.2 TB/s for plain loads).  Token rows are
// shared by every tile of an expert and keep the default policy.
template <int CPT, int NW>
__device__ __forceinline__ void load_stage(i32x4 (&regs)[CPT], const char *const (&src)[CPT],
                                           int64_t off) {
#pragma unroll
    for (int i = 0; i < NW; ++i) regs[i] = __builtin_nontemporal_load((const i32x4 *)(src[i] + off));
#pragma unroll
    for (int i = NW; i < CPT; ++i) regs[i] = *(const i32x4 *)(src[i] + off);
}

// T: activation and weight type; TO: output type (T, or fp32 for the expert
// outputs the fused layer combines).
template <int BN, int BM, int WN, int WM, bool SWIGLU, typename T, typename TO>
__global__ __launch_bounds__(WN *WM *kWave) void skinny_gemm_kernel(
    const T *__restrict__ act, int64_t act_ld, const T *__restrict__ Wa,
    const T *__restrict__ Wb, const int32_t *__restrict__ offsets, int E, int N, int K, int A,
    TO *__restrict__ out) {
    using C = SkinnyCfg<BN, BM, WN, WM, SWIGLU, T>;
    constexpr int CPT = C::CPT, TN = C::TN, TM = C::TM;
    __shared__ __attribute__((aligned(16))) char smem[C::kLdsBytes];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int n_tiles = (N + BN - 1) / BN;

    // Tile numbering as in the grouped kernel: eight contiguous ranges, one
    // per XCD (workgroup b runs on XCD b % 8), token tiles fastest.  Offsets
    // are clamped to [0, A] so that no row index leaves the buffers.
    int total = 0;
    for (int i = 0; i < E; ++i) {
        const int lo = min(max(offsets[i], 0), A);
        const int hi = min(max(offsets[i + 1], lo), A);
        total += (hi - lo + BM - 1) / BM * n_tiles;
    }
    const int per_xcd = (total + 7) / 8;
    const int tile = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (tile >= total) return;  // uniform over the workgroup
    int rem = tile, e = 0, lo = 0, hi = 0;
    for (int i = 0; i < E; ++i) {
        lo = min(max(offsets[i], 0), A);
        hi = min(max(offsets[i + 1], lo), A);
        const int mtiles = (hi - lo + BM - 1) / BM;
        if (rem < mtiles * n_tiles) {
            e = i;
            break;
        }
        rem -= mtiles * n_tiles;
    }
    const int mtiles = (hi - lo + BM - 1) / BM;
    const int row0 = lo + (rem % mtiles) * BM;
    const int mrem = min(BM, hi - row0);
    const int n0 = (rem / mtiles) * BN;

    // This thread's chunks of every stage: fixed rows, fixed 16-byte columns.
    const char *src[CPT];
    int dst[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int q = i * C::kThreads + tid;
        const int r = q >> 3, c = q & 7;
        dst[i] = swz128(r, c);
        if (r < C::kWRows) {
            const T *W = (SWIGLU && r >= BN) ? Wb : Wa;
            const int nr = min(n0 + (SWIGLU ? r % BN : r), N - 1);
            src[i] = (const char *)(W + ((int64_t)e * N + nr) * K) + c * 16;
        } else {
            const int m = min(r - C::kWRows, mrem - 1);
            src[i] = (const char *)(act + (int64_t)(row0 + m) * act_ld) + c * 16;
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

    const int wn = wave % WN, wm = wave / WN;
    const int wrow0 = wn * (BN / WN);
    const int xrow0 = wm * (BM / WM);
    // token fragments of this wave holding at least one real row (wave-uniform)
    const int live = __builtin_amdgcn_readfirstlane(min(TM, max(0, (mrem - xrow0 + 15) / 16)));
    const int n_stages = K / C::kKStep;

    i32x4 regs[CPT];
    load_stage<CPT, C::NW>(regs, src, 0);
#pragma unroll
    for (int i = 0; i < CPT; ++i) *(i32x4 *)(smem + dst[i]) = regs[i];
    __syncthreads();

    for (int s = 0; s < n_stages; ++s) {
        const int buf = s & 1;
        if (s + 1 < n_stages) load_stage<CPT, C::NW>(regs, src, (int64_t)(s + 1) * 128);
        const char *sW = smem + buf * C::kStageBytes;
        const char *sX = sW + C::kWRows * 128;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int c = ks * 4 + (lane >> 4);
            i32x4 xf[TM];
#pragma unroll
            for (int j = 0; j < TM; ++j)
                xf[j] = *(const i32x4 *)(sX + swz128(xrow0 + j * 16 + (lane & 15), c));
#pragma unroll
            for (int i = 0; i < TN; ++i) {
                const int r = wrow0 + i * 16 + (lane & 15);
                const i32x4 wf = *(const i32x4 *)(sW + swz128(r, c));
                i32x4 vf;
                if constexpr (SWIGLU) vf = *(const i32x4 *)(sW + swz128(BN + r, c));
#pragma unroll
                for (int j = 0; j < TM; ++j) {
                    if (j < live) {
                        accu[i][j] = mma16<T>(wf, xf[j], accu[i][j]);
                        if constexpr (SWIGLU) accv[i][j] = mma16<T>(vf, xf[j], accv[i][j]);
                    }
                }
            }
        }
        if (s + 1 < n_stages) {
            char *nb = smem + (buf ^ 1) * C::kStageBytes;
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
                    if constexpr (SWIGLU) v[q] = silu_f(v[q]) * accv[i][j][q];
                }
                put4<TO>(out + (int64_t)(row0 + m) * N + n, v[0], v[1], v[2], v[3]);
            }
        }
    }
}

template <int BN, int BM, int WN, int WM, bool SWIGLU, typename T, typename TO = T>
static hipError_t launch_skinny(const void *act, int64_t act_ld, const void *Wa, const void *Wb,
                                const int32_t *offsets, int E, int N, int K, int64_t A, void *out,
                                hipStream_t s) {
    using C = SkinnyCfg<BN, BM, WN, WM, SWIGLU, T>;
    const int64_t n_tiles = (N + BN - 1) / BN;
    // sum_e ceil(c_e / BM) <= ceil(A / BM) + E - 1; the XCD numbering can
    // reach 7 past the total.
    const int64_t bound = n_tiles * ((A + BM - 1) / BM + E - 1);
    const int64_t blocks = (bound + 7) / 8 * 8 + 8;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((skinny_gemm_kernel<BN, BM, WN, WM, SWIGLU, T, TO>),
                       dim3((unsigned)blocks), dim3(C::kThreads), 0, s, (const T *)act, act_ld,
                       (const T *)Wa, (const T *)Wb, offsets, E, N, K, (int)A, (TO *)out);
    return hipGetLastError();
}

template <typename T, typename TO>
static hipError_t skinny_ffn_typed(const void *x_perm, const int32_t *offsets, const void *W1,
                                   const void *W3, const void *W2, int64_t A, int d, int d_ff,
                                   int E, void *hbuf, void *out, hipEvent_t mid, hipStream_t s) {
    hipError_t err = launch_skinny<64, 32, 4, 1, true, T>(x_perm, d, W1, W3, offsets, E, d_ff, d,
                                                          A, hbuf, s);
    if (err == hipSuccess && mid) err = hipEventRecord(mid, s);
    if (err != hipSuccess) return err;
    // W2 has only d rows per expert: 32-row tiles give 8x more workgroups
    // (more loads in flight) than GEMM1's tiles would.
    return launch_skinny<32, 32, 2, 2, false, T, TO>(hbuf, d_ff, W2, nullptr, offsets, E, d,
                                                     d_ff, A, out, s);
}

}  // namespace moe

hipError_t moe_launch_skinny_ffn(const void *x_perm, const int32_t *offsets, const void *W1,
                                 const void *W3, const void *W2, int dt, int out_f32, int64_t A,
                                 int d, int d_ff, int E, void *hbuf, void *out, hipEvent_t mid,
                                 hipStream_t s) {
    using moe::bf16_t;
    if (dt == 0)
        return moe::skinny_ffn_typed<float, float>(x_perm, offsets, W1, W3, W2, A, d, d_ff, E,
                                                   hbuf, out, mid, s);
    if (out_f32)
        return moe::skinny_ffn_typed<bf16_t, float>(x_perm, offsets, W1, W3, W2, A, d, d_ff, E,
                                                    hbuf, out, mid, s);
    return moe::skinny_ffn_typed<bf16_t, bf16_t>(x_perm, offsets, W1, W3, W2, A, d, d_ff, E,
                                                 hbuf, out, mid, s);
}
