// stream_gemm.hip — the expert GEMMs of decode-sized bf16 batches as one
// continuous weight stream.
//
// Same experts as expert_gemm.hip (the SwiGLU MLP W2 (silu(W1 x) * W3 x):
// fdeinterviews breakdown, "The paper in one minute"; tokentrails lineage,
// Code listing), but at decode sizes every expert holds only a few rows
// (about 8 at T = 32), so each weight byte feeds a handful of multiply-adds
// and the kernel is a read of the active experts' weights at the HBM rate.
// What it takes to stay at that rate:
//  * bytes in flight: one persistent workgroup per CU runs a ring of P = 6
//    LDS stages filled by global_load_lds, so ~120 KiB per CU are always on
//    their way (a plain register double buffer keeps one stage in flight);
//  * no drain between tiles: the ring runs across the tiles of a workgroup,
//    the next tile's first stages load while the current one finishes;
//  * non-temporal weight loads: weights are read once, and the nt hint lifts
//    the sustained read rate (about 7 TB/s against about 6.2 on MI355X);
//    token rows, shared by all tiles of an expert, keep the default policy.
//
// Tile: 128 weight rows (GEMM1: 64 rows of W1 and the same 64 rows of W3)
// by 64 token rows of one expert, K in stages of 64 bf16.  A stage holds the
// 128 weight rows and the 64 token rows (rows past the expert's count repeat
// its last row and are not stored), 128 bytes each: every load instruction
// moves eight whole 128-byte lines (with half lines per stage, the nt hint
// can drop a line before the next stage reads its other half).  In LDS the
// 16-byte chunk c of row r sits at chunk c ^ ((r >> 1) & 7), which keeps the
// 32-row operand reads free of bank conflicts.  Four waves in a 2 x 2 grid:
// wave (wn, wm) multiplies the weight fragments of half wn (GEMM1: one W1
// and the matching W3 fragment) with token fragment wm on
// v_mfma_f32_32x32x16_bf16, two MFMAs per 16-wide k-step -- the matrix cores
// idle almost always, by design.
#include "gemm_common.h"

namespace moe {

namespace {

constexpr int kSBW = 128, kSBT = 64, kSWaves = 4;
constexpr int kSP = 6;                                // stages in the ring
constexpr int kSRows = kSBW + kSBT;                   // LDS rows per stage
constexpr int kSLPW = kSRows / 8 / kSWaves;           // 8-row loads per wave per stage
constexpr int kSWLoads = kSBW / 8 / kSWaves;          // of which weight rows
constexpr int kSStageBytes = kSRows * 128;
constexpr int kSLds = kSP * kSStageBytes;
constexpr int kSKStep = 64;                           // bf16 K elements per stage
static_assert(kSRows % (8 * kSWaves) == 0 && kSBW % (8 * kSWaves) == 0, "load split");

__device__ __forceinline__ int swz128(int r, int c) {
    return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
}
static_assert(kSLPW * (kSP - 2) < 64, "vmcnt range");
static_assert(kSLds <= 160 * 1024 - 1024, "LDS capacity");

}  // namespace

template <bool SWIGLU, typename TO>
__global__ __launch_bounds__(256) void stream_gemm_kernel(
    const bf16_t *__restrict__ act, int64_t act_ld, const int32_t *__restrict__ gather,
    const bf16_t *__restrict__ Wa, const bf16_t *__restrict__ Wb,
    const int32_t *__restrict__ offsets, int E, int N, int K, int A, TO *__restrict__ out) {
    constexpr int P = kSP, LPW = kSLPW, BW = kSBW, BT = kSBT;
    constexpr int kCols = SWIGLU ? BW / 2 : BW;  // output columns per tile
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    __shared__ int s_lo[64], s_cnt[64], s_first[65];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int col_tiles = (N + kCols - 1) / kCols;
    const int n_k = K / kSKStep;  // >= P - 1, checked by the launcher

    // Per-expert tile table (token tiles fastest, then column tiles); offsets
    // clamped to [0, A] so no row index leaves the buffers.
    if (tid == 0) {
        int f = 0;
        for (int i = 0; i < E; ++i) {
            const int lo = min(max(offsets[i], 0), A);
            const int hi = min(max(offsets[i + 1], lo), A);
            s_lo[i] = lo;
            s_cnt[i] = hi - lo;
            s_first[i] = f;
            f += (hi - lo + BT - 1) / BT * col_tiles;
        }
        s_first[E] = f;
    }
    __syncthreads();
    const int total = s_first[E];
    const int G = gridDim.x;
    const int my_tiles = (total > (int)blockIdx.x) ? (total - (int)blockIdx.x + G - 1) / G : 0;
    if (my_tiles == 0) return;  // uniform over the workgroup

    auto tile_info = [&](int k) {
        const int t = (int)blockIdx.x + k * G;
        int i = 0;
        while (i + 1 < E && s_first[i + 1] <= t) ++i;
        const int rem = t - s_first[i];
        const int mtiles = (s_cnt[i] + BT - 1) / BT;
        TileInfo ti;
        ti.e = i;
        ti.row0 = s_lo[i] + (rem % mtiles) * BT;
        ti.mrem = min(BT, s_lo[i] + s_cnt[i] - ti.row0);
        ti.n0 = (rem / mtiles) * kCols;
        return ti;
    };

    // Lane pointers of this wave's LPW 8-row loads: load i covers stage rows
    // (wave + 4 i) * 8 .. + 8, lane l the chunk that belongs at LDS offset
    // 16 l; loads [0, kSWLoads) are weight rows, the rest token rows (act
    // rows, through `gather` if set).
    auto sources = [&](const TileInfo &ti, const char *(&src)[LPW]) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int r = (wave + kSWaves * i) * 8 + (lane >> 3);
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            if (i < kSWLoads) {
                const bf16_t *W = Wa;
                int nr;
                if constexpr (SWIGLU) {
                    W = (r < BW / 2) ? Wa : Wb;
                    nr = ti.n0 + (r % (BW / 2));
                } else {
                    nr = ti.n0 + r;
                }
                nr = min(nr, N - 1);
                src[i] = (const char *)(W + ((int64_t)ti.e * N + nr) * K) + c * 16;
            } else {
                const int row = act_row<8>(gather, ti.row0 + (wave + kSWaves * i) * 8 - BW,
                                           ti.row0 + ti.mrem - 1, lane);
                src[i] = (const char *)(act + (int64_t)row * act_ld) + c * 16;
            }
        }
    };
    auto issue = [&](int slot, const char *const (&src)[LPW], int stage) {
        char *dst = smem + slot * kSStageBytes;
        const int64_t off = (int64_t)stage * 128;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            if (i < kSWLoads)
                dma16_nt(src[i] + off, dst + (wave + kSWaves * i) * 1024);
            else
                dma16(src[i] + off, dst + (wave + kSWaves * i) * 1024);
        }
    };

    const int wn = wave & 1, wm = wave >> 1;
    const int lrow = lane & 31, lhalf = lane >> 5;
    // LDS rows of the wave's two weight fragments and its token fragment
    const int wr0 = SWIGLU ? wn * 32 : wn * 64;
    const int wr1 = SWIGLU ? BW / 2 + wn * 32 : wn * 64 + 32;
    const int tr = BW + wm * 32;

    const char *sc[LPW], *sn[LPW];  // sources of the current and the next tile
    TileInfo nxt = tile_info(0);
    sources(nxt, sn);
#pragma unroll
    for (int g = 0; g < P - 1; ++g) issue(g, sn, g);

    int g = 0;  // stages consumed so far = ring cursor
    for (int c_k = 0; c_k < my_tiles; ++c_k) {
        const TileInfo cur = nxt;
#pragma unroll
        for (int i = 0; i < LPW; ++i) sc[i] = sn[i];
        if (c_k + 1 < my_tiles) {
            nxt = tile_info(c_k + 1);
            sources(nxt, sn);
        }
        // (past the last tile sn == sc: the refills reload stages of this
        // tile, which nothing reads)
        f32x16 acc0 = {}, acc1 = {};
        for (int s = 0; s < n_k; ++s, ++g) {
            // stage g landed (this wave's loads, then everyone's); every wave
            // is done reading the slot of stage g - 1
            wait_vmcnt_lgkm0<LPW * (P - 2)>();
            stage_barrier();
            const int q = s + P - 1;
            if (q < n_k)
                issue((g + P - 1) % P, sc, q);
            else
                issue((g + P - 1) % P, sn, q - n_k);
            const char *base = smem + (g % P) * kSStageBytes;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int c = 2 * t + lhalf;
                const i32x4 w0 = *(const i32x4 *)(base + swz128(wr0 + lrow, c));
                const i32x4 w1 = *(const i32x4 *)(base + swz128(wr1 + lrow, c));
                const i32x4 x = *(const i32x4 *)(base + swz128(tr + lrow, c));
                acc0 = mma_step<bf16_t>(w0, x, acc0);
                acc1 = mma_step<bf16_t>(w1, x, acc1);
            }
        }
        // Epilogue: element q of a fragment is D[n = 8 (q / 4) + 4 lhalf + q % 4][m = lrow].
        const int m = wm * 32 + lrow;
        if (m < cur.mrem) {
            TO *orow = out + (int64_t)(cur.row0 + m) * N;
#pragma unroll
            for (int f = 0; f < (SWIGLU ? 1 : 2); ++f) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int n = cur.n0 + (SWIGLU ? wn * 32 : wn * 64 + f * 32) + 8 * gq + 4 * lhalf;
                    if (n < N) {
                        float r[4];
#pragma unroll
                        for (int qq = 0; qq < 4; ++qq) {
                            if constexpr (SWIGLU)
                                r[qq] = silu(acc0[4 * gq + qq]) * acc1[4 * gq + qq];
                            else
                                r[qq] = (f == 0 ? acc0 : acc1)[4 * gq + qq];
                        }
                        store4<TO>(orow + n, r[0], r[1], r[2], r[3]);
                    }
                }
            }
        }
    }
    wait_vmcnt_lgkm0<0>();  // the trailing reloads land before the wave ends
}

namespace {

template <bool SWIGLU, typename TO>
hipError_t launch_stream(const void *act, int64_t act_ld, const int32_t *gather, const void *Wa,
                         const void *Wb, const int32_t *offsets, int E, int N, int K, int64_t A,
                         void *out, hipStream_t s) {
    auto kern = stream_gemm_kernel<SWIGLU, TO>;
    hipError_t err = set_lds_limit<stream_gemm_kernel<SWIGLU, TO>>(kSLds);
    if (err != hipSuccess) return err;
    // one workgroup per CU, never more than there are tiles:
    // sum_e ceil(c_e / BT) <= ceil(A / BT) + E - 1
    const int64_t cols = SWIGLU ? kSBW / 2 : kSBW;
    const int64_t tile_bound = (N + cols - 1) / cols * ((A + kSBT - 1) / kSBT + E - 1);
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(device_cus(), tile_bound));
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), kSLds, s, (const bf16_t *)act, act_ld,
                       gather, (const bf16_t *)Wa, (const bf16_t *)Wb, offsets, E, N, K, (int)A,
                       (TO *)out);
    return hipGetLastError();
}

}  // namespace

bool stream_supported(int d, int d_ff) {
    return d >= (kSP - 1) * kSKStep && d_ff >= (kSP - 1) * kSKStep;
}

hipError_t launch_stream_ffn(const void *act, const int32_t *gather, const int32_t *offsets,
                             const void *W1, const void *W3, const void *W2, int out_f32,
                             int64_t A, int d, int d_ff, int E, void *hbuf, void *out,
                             hipEvent_t mid, hipStream_t s) {
    hipError_t err =
        launch_stream<true, bf16_t>(act, d, gather, W1, W3, offsets, E, d_ff, d, A, hbuf, s);
    if (err == hipSuccess && mid) err = hipEventRecord(mid, s);
    if (err != hipSuccess) return err;
    if (out_f32)
        return launch_stream<false, float>(hbuf, d_ff, nullptr, W2, nullptr, offsets, E, d, d_ff,
                                           A, out, s);
    return launch_stream<false, bf16_t>(hbuf, d_ff, nullptr, W2, nullptr, offsets, E, d, d_ff, A,
                                        out, s);
}

}  // namespace moe
