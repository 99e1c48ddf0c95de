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
// Tiles.  A tile is BW weight rows by BT token rows of one expert (for GEMM1
// the BW rows are BW/2 rows of W1 and the same BW/2 rows of W3).  Weights
// play the "A" operand and tokens the "B" operand of
// v_mfma_f32_32x32x16_bf16 (fp32 data: four v_mfma_f32_32x32x2_f32 per
// 16-byte fragment), accumulating in fp32.  On gfx950 the 32x32x16 form runs
// at the full dense bf16 rate, twice the 16x16x32 form.  A lane of an output
// fragment holds four runs of four consecutive n of one token row, each
// written as one 8-byte (bf16) or 16-byte (fp32) store.  silu(u) * v is
// formed in registers from the u and v accumulators of the same lane, so
// GEMM1 never writes u or v.
//
// LDS layout.  K advances 64 bytes per stage (32 bf16 / 16 fp32).  A stage
// holds BW + BT rows of 64 bytes; the four 16-byte chunks of row r sit at
// chunk ^ ((r >> 2) & 3).  An MFMA operand read (32 rows, one chunk per
// half-wave) then touches 16 distinct 16-byte bank groups in every group of
// 16 lanes: no bank conflicts.
//
// Pipeline.  Rows move from global memory straight into LDS with
// global_load_lds_dwordx4: one instruction moves 16 rows x 64 bytes, lane i
// fetching the chunk that belongs at LDS offset 16 i.  No registers hold
// tiles in flight.  A ring of P stages keeps P-1 stages in flight while one
// is consumed: wait (vmcnt) for this wave's share of the stage, barrier,
// issue the stage P-1 ahead into the slot every wave finished reading before
// the barrier, then run the MFMAs.  The waits are explicit; the barrier
// carries no memory fence (a fence would wait for every load in flight) but
// compiler barriers keep the code order.
//
// Persistent tiles.  The grid is a fixed number of resident workgroups; each
// walks a list of tiles, and the load ring runs across tile boundaries, so
// the next tile's first stages are in flight while the current one finishes
// and writes its output.  Workgroup b runs on XCD b % 8.  The tiles are cut
// into eight contiguous ranges, one per XCD (token tiles fastest, then
// weight tiles, then experts), and the workgroups of an XCD take consecutive
// tiles of its range in lock step, so they share weight and token tiles in
// that XCD's L2.
//
// Ragged tiles.  Token rows past the expert's count load a clamped valid row
// and are never stored; 32-row fragments wholly past the count skip their
// MFMAs.  Weight rows past N are clamped likewise.  The tile list is derived
// on the device from the offsets, so the host never reads the counts back.
#include "gemm_common.h"

namespace moe {

template <int BW, int BT, int WN, int WM, int P, bool SWIGLU, typename T>
struct GemmCfg {
    static constexpr int kWaves = WN * WM;
    static constexpr int kThreads = kWaves * kWave;
    static constexpr int kRows = BW + BT;               // LDS rows per stage
    static constexpr int LPW = kRows / 16 / kWaves;     // 16-row loads per wave per stage
    static constexpr int kStageBytes = kRows * 64;
    static constexpr int kLdsBytes = P * kStageBytes;
    static constexpr int kCols = SWIGLU ? BW / 2 : BW;  // output columns per tile
    static constexpr int WU = kCols / 32 / WN;          // 32-row weight fragments per wave (u)
    static constexpr int WT = BT / 32 / WM;             // 32-row token fragments per wave
    static constexpr int kKStep = 64 / ElemSize<T>::value;  // K elements per stage
    static_assert(kRows % (16 * kWaves) == 0, "stage rows must split evenly over waves");
    static_assert(WU >= 1 && WT >= 1, "wave tile too small");
    static_assert(kCols % (32 * WN) == 0 && BT % (32 * WM) == 0, "tile shape");
    static_assert(P >= 3, "ring needs at least three stages");
    static_assert(LPW * (P - 2) < 64, "vmcnt range");
    static_assert(kLdsBytes <= 160 * 1024, "LDS capacity");
};


// T: activation and weight type; TO: output type (T, or fp32 for the expert
// outputs the fused layer combines).
template <int BW, int BT, int WN, int WM, int P, bool SWIGLU, typename T, typename TO>
__global__ __launch_bounds__(WN *WM *kWave) void grouped_gemm_kernel(
    const T *__restrict__ act, int64_t act_ld, const T *__restrict__ Wa,
    const T *__restrict__ Wb, const int32_t *__restrict__ offsets, int E, int N, int K, int A,
    TO *__restrict__ out) {
    using C = GemmCfg<BW, BT, WN, WM, P, SWIGLU, T>;
    constexpr int WU = C::WU, WT = C::WT, LPW = C::LPW;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    // per expert: first row, row count, first tile number (tiles before it)
    __shared__ int s_lo[64], s_cnt[64], s_first[65];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int n_tiles = (N + C::kCols - 1) / C::kCols;

    if (wave == 0) build_expert_table(offsets, E, A, BT, n_tiles, s_lo, s_cnt, s_first);
    __syncthreads();
    const int total = s_first[E];

    // This workgroup's tiles: XCD range, then round robin inside the XCD.
    const int G8 = gridDim.x / 8;  // workgroups per XCD (grid is a multiple of 8)
    const int xcd = blockIdx.x % 8, wj = blockIdx.x / 8;
    const int range = (total + 7) / 8;
    const int range_lo = xcd * range;
    const int range_n = max(0, min(range, total - range_lo));
    const int my_tiles = (range_n > wj) ? (range_n - wj + G8 - 1) / G8 : 0;
    const int n_k = K / C::kKStep;  // stages per tile
    const int n_stages = my_tiles * n_k;
    if (n_stages == 0) return;  // uniform over the workgroup

    auto tile_info = [&](int k) {
        const int t = range_lo + wj + k * G8;
        int i = 0;
        while (i + 1 < E && s_first[i + 1] <= t) ++i;
        const int rem = t - s_first[i];
        const int mtiles = (s_cnt[i] + BT - 1) / BT;
        TileInfo ti;
        ti.e = i;
        ti.row0 = s_lo[i] + (rem % mtiles) * BT;
        ti.mrem = min(BT, s_lo[i] + s_cnt[i] - ti.row0);
        ti.n0 = (rem / mtiles) * C::kCols;
        return ti;
    };

    // Producer.  Row r of a stage is loaded by wave (r / 16) % waves, lane
    // 4 (r % 16) + chunk slot; the lane fetches the chunk that belongs in that
    // slot.  Inside the loop the only vector-memory instructions are these
    // loads (and the output stores), so the explicit waits stay exact.
    const char *src[LPW];
    auto set_sources = [&](const TileInfo &ti) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int r = (wave + C::kWaves * i) * 16 + (lane >> 2);  // LDS row
            const int c = (lane & 3) ^ ((r >> 2) & 3);                // global chunk it holds
            if (r < BW) {
                const T *W = Wa;
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
                const int m = min(r - BW, ti.mrem - 1);
                src[i] = (const char *)(act + (int64_t)(ti.row0 + m) * act_ld) + c * 16;
            }
        }
    };
    int p_k = 0, p_s = 0;  // producer cursor: tile, stage
    auto issue_next = [&](int g) {
        if (p_s == 0) set_sources(tile_info(p_k));
        char *slot = smem + (g % P) * C::kStageBytes;
#pragma unroll
        for (int i = 0; i < LPW; ++i)
            dma16(src[i] + (int64_t)p_s * 64, slot + (wave + C::kWaves * i) * 1024);
        if (++p_s == n_k) {
            p_s = 0;
            ++p_k;
        }
    };

    f32x16 accu[WU][WT];
    f32x16 accv[SWIGLU ? WU : 1][WT];
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < WU; ++i)
#pragma unroll
            for (int j = 0; j < WT; ++j) {
                accu[i][j] = f32x16{};
                if constexpr (SWIGLU) accv[i][j] = f32x16{};
            }
    };
    zero_acc();

    const int wn = wave % WN, wm = wave / WN;
    const int ur0 = wn * WU * 32;        // first u (or plain weight) row of this wave
    const int tr0 = BW + wm * WT * 32;   // first token LDS row of this wave
    const int lrow = lane & 31, lhalf = lane >> 5;

    // MFMAs of one stage over the first `live` token fragments of the wave.
    auto compute = [&](const char *slot, int live) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int c = 2 * t + lhalf;
            i32x4 tf[WT];
#pragma unroll
            for (int j = 0; j < WT; ++j) tf[j] = *(const i32x4 *)(slot + lds_off(tr0 + j * 32 + lrow, c));
#pragma unroll
            for (int i = 0; i < WU; ++i) {
                const int r = ur0 + i * 32 + lrow;
                const i32x4 wf = *(const i32x4 *)(slot + lds_off(r, c));
                i32x4 vf;
                if constexpr (SWIGLU) vf = *(const i32x4 *)(slot + lds_off(BW / 2 + r, c));
#pragma unroll
                for (int j = 0; j < WT; ++j) {
                    if (j < live) {
                        accu[i][j] = mma_step<T>(wf, tf[j], accu[i][j]);
                        if constexpr (SWIGLU) accv[i][j] = mma_step<T>(vf, tf[j], accv[i][j]);
                    }
                }
            }
        }
    };

#pragma unroll
    for (int g = 0; g < P - 1; ++g)
        if (g < n_stages) issue_next(g);

    TileInfo cur = tile_info(0);
    // token fragments of this wave holding at least one real row (wave-uniform)
    int live_t = __builtin_amdgcn_readfirstlane(min(WT, max(0, (cur.mrem - wm * WT * 32 + 31) / 32)));
    int c_s = 0, c_k = 0;  // consumer cursor: stage within tile, tile
    for (int g = 0; g < n_stages; ++g) {
        if (g + P - 2 < n_stages)
            wait_vmcnt_lgkm0<LPW * (P - 2)>();
        else
            wait_vmcnt_lgkm0<0>();
        stage_barrier();
        if (g + P - 1 < n_stages) issue_next(g + P - 1);

        const char *slot = smem + (g % P) * C::kStageBytes;
        compute(slot, live_t);

        if (++c_s == n_k) {
            // Epilogue of the tile: element q of fragment (i, j) is
            // D[n = 8 (q / 4) + 4 lhalf + q % 4][m = lrow].
#pragma unroll
            for (int i = 0; i < WU; ++i) {
#pragma unroll
                for (int j = 0; j < WT; ++j) {
                    const int m = wm * WT * 32 + j * 32 + lrow;
                    if (m < cur.mrem) {
                        TO *orow = out + (int64_t)(cur.row0 + m) * N;
#pragma unroll
                        for (int gq = 0; gq < 4; ++gq) {
                            const int n = cur.n0 + ur0 + i * 32 + 8 * gq + 4 * lhalf;
                            if (n < N) {
                                float v[4];
#pragma unroll
                                for (int q = 0; q < 4; ++q) {
                                    v[q] = accu[i][j][4 * gq + q];
                                    if constexpr (SWIGLU) v[q] = silu(v[q]) * accv[i][j][4 * gq + q];
                                }
                                store4<TO>(orow + n, v[0], v[1], v[2], v[3]);
                            }
                        }
                    }
                }
            }
            zero_acc();
            c_s = 0;
            if (++c_k < my_tiles) {
                cur = tile_info(c_k);
                live_t = __builtin_amdgcn_readfirstlane(
                    min(WT, max(0, (cur.mrem - wm * WT * 32 + 31) / 32)));
            }
        }
    }
}


template <int BW, int BT, int WN, int WM, int P, bool SWIGLU, typename T, typename TO = T>
static hipError_t launch_grouped(const void *act, int64_t act_ld, const void *Wa, const void *Wb,
                                 const int32_t *offsets, int E, int N, int K, int64_t A,
                                 void *out, int wg_per_cu, hipStream_t s) {
    using C = GemmCfg<BW, BT, WN, WM, P, SWIGLU, T>;
    auto kern = grouped_gemm_kernel<BW, BT, WN, WM, P, SWIGLU, T, TO>;
    // LDS beyond the 64 KiB default must be requested per kernel
    hipError_t err =
        set_lds_limit<grouped_gemm_kernel<BW, BT, WN, WM, P, SWIGLU, T, TO>>(C::kLdsBytes);
    if (err != hipSuccess) return err;
    // Resident workgroups, a multiple of 8 (one share per XCD), and never
    // more than the tile count can use: sum_e ceil(c_e / BT) <= ceil(A / BT) + E - 1.
    const int64_t n_tiles = (N + C::kCols - 1) / C::kCols;
    const int64_t tile_bound = n_tiles * ((A + BT - 1) / BT + E - 1);
    int64_t grid = (int64_t)device_cus() * wg_per_cu;
    grid = std::min<int64_t>(grid, (tile_bound + 7) / 8 * 8);
    grid = std::max<int64_t>(8, grid / 8 * 8);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::kThreads), C::kLdsBytes, s,
                       (const T *)act, act_ld, (const T *)Wa, (const T *)Wb, offsets, E, N, K,
                       (int)A, (TO *)out);
    return hipGetLastError();
}

// Which kernels run the experts: decode-sized batches stream the weights
// (stream_gemm.hip for bf16, skinny_gemm.hip for fp32 or small d), mid-sized
// ones use 8-wave grouped tiles, large bf16 ones the wide tiles
// (wide_gemm.hip).
enum class FfnPath { kStream, kSkinny, kGroupedSmall, kGroupedLarge, kWide, kMixed };

// Which kernels run the experts, by the average rows per expert (measured on
// MI355X at d = 4096, d_ff = 14336, E = 8, k = 2; layer times in us):
//   T        96    128   192   256   512   1024
//   stream   459   815  1145  1300  2056  3676
//   grouped  605   615   632   867  1254  1892
//   wide     653   659   669   690   722   954
// The weight stream wins while one 32-row token tile holds nearly every
// expert's rows (an expert with more streams its weights twice; with the even
// K split balancing the tiles, the stream ran the layer in 0.443 ms at 26
// rows per expert on average, 0.549 at 27 against 0.550 for the kernels
// below, and lost from 29 on); the large tiles win from about 56 rows per
// expert on, since smaller tiles re-read the weights for every token tile.
// (Those wide figures are 256-row token tiles.  At 25-48 rows per expert the
// wide kernels' GEMM2 with 128-row token tiles beats the grouped one by a
// quarter, 181-186 against 251-264 us at T = 100-195, while their GEMM1,
// whose 128-row tiles are mostly padding there, loses to the grouped 64-row
// tiles, 367-378 against 335-358 us: bf16 takes the grouped GEMM1 and the
// wide GEMM2 there, the wide kernels for both from 49 on.)
static FfnPath ffn_path(int dt, int64_t A, int d, int d_ff, int E) {
    const int64_t per_expert = A / E;
    const bool stream = dt == 1 && stream_supported(A, d, d_ff, E);
    if (stream && per_expert <= 26) return FfnPath::kStream;
    if (dt == 1 && per_expert > 24 && wide_supported(A, d, d_ff))
        return per_expert <= 48 ? FfnPath::kMixed : FfnPath::kWide;
    if (per_expert <= 32 && !stream) return FfnPath::kSkinny;
    if (per_expert <= 256) return FfnPath::kGroupedSmall;
    return FfnPath::kGroupedLarge;
}

static bool path_gathers(FfnPath p) { return p == FfnPath::kStream || p == FfnPath::kWide; }

template <typename T, typename TO>
static hipError_t launch_ffn_typed(const void *act, const int32_t *gather,
                                   const int32_t *offsets, const void *W1, const void *W3,
                                   const void *W2, int64_t A, int d, int d_ff, int E, void *hbuf,
                                   void *out, void *scratch, size_t scratch_bytes,
                                   hipEvent_t mid, hipStream_t s) {
    hipError_t err;
    const int dt = ElemSize<T>::value == 4 ? 0 : 1;
    const FfnPath path = ffn_path(dt, A, d, d_ff, E);
    if (gather && !path_gathers(path)) return hipErrorInvalidValue;
    switch (path) {
        case FfnPath::kStream:
            return launch_stream_ffn(act, gather, offsets, W1, W3, W2, ElemSize<TO>::value == 4,
                                     A, d, d_ff, E, hbuf, out, (float *)scratch, scratch_bytes,
                                     mid, s);
        case FfnPath::kSkinny:
            return moe_launch_skinny_ffn(act, offsets, W1, W3, W2, dt, ElemSize<TO>::value == 4, A,
                                         d, d_ff, E, hbuf, out, mid, s);
        case FfnPath::kGroupedSmall:
            err = launch_grouped<128, 64, 2, 2, 6, true, T>(act, d, W1, W3, offsets, E, d_ff, d,
                                                             A, hbuf, 2, s);
            if (err == hipSuccess && mid) err = hipEventRecord(mid, s);
            if (err != hipSuccess) return err;
            return launch_grouped<128, 64, 2, 2, 6, false, T, TO>(hbuf, d_ff, W2, nullptr,
                                                                   offsets, E, d, d_ff, A, out, 2,
                                                                   s);
        case FfnPath::kWide:
            return launch_wide_ffn(act, gather, offsets, W1, W3, W2, ElemSize<TO>::value == 4, A,
                                   d, d_ff, E, hbuf, out, (float *)scratch, scratch_bytes, mid,
                                   s);
        case FfnPath::kMixed:
            err = launch_grouped<128, 64, 2, 2, 6, true, T>(act, d, W1, W3, offsets, E, d_ff, d,
                                                             A, hbuf, 2, s);
            if (err == hipSuccess && mid) err = hipEventRecord(mid, s);
            if (err != hipSuccess) return err;
            return launch_wide_w2(hbuf, offsets, W2, ElemSize<TO>::value == 4, A, d, d_ff, E, out,
                                  (float *)scratch, scratch_bytes, s);
        case FfnPath::kGroupedLarge:
            break;
    }
    err = launch_grouped<256, 256, 4, 2, 4, true, T>(act, d, W1, W3, offsets, E, d_ff, d, A,
                                                      hbuf, 1, s);
    if (err == hipSuccess && mid) err = hipEventRecord(mid, s);
    if (err != hipSuccess) return err;
    return launch_grouped<256, 256, 4, 2, 4, false, T, TO>(hbuf, d_ff, W2, nullptr, offsets, E,
                                                            d, d_ff, A, out, 1, s);
}

}  // namespace moe

bool moe_expert_ffn_gathers(int dt, int64_t A, int d, int d_ff, int E) {
    return moe::path_gathers(moe::ffn_path(dt, A, d, d_ff, E));
}

bool moe_expert_ffn_streams(int dt, int64_t A, int d, int d_ff, int E) {
    return moe::ffn_path(dt, A, d, d_ff, E) == moe::FfnPath::kStream;
}


hipError_t moe_launch_stream_layer(const void *x, const int32_t *topk_idx, int k, const float *gw,
                                   const void *residual, const void *W1, const void *W3,
                                   const void *W2, int64_t T, int d, int d_ff, int E,
                                   int32_t *counts, int32_t *offsets, int32_t *row_of,
                                   int32_t *token_of, void *hbuf, float *o_perm, void *y,
                                   void *scratch, size_t scratch_bytes, int32_t *ctr,
                                   hipEvent_t gemm1_done, hipStream_t s) {
    const int64_t A = T * k;
    moe::StreamFuse f{};
    f.ctr = ctr;
    f.topk_idx = topk_idx;
    f.k = k;
    f.counts = counts;
    f.offsets = offsets;
    f.row_of = row_of;
    f.token_of = token_of;
    f.gw = gw;
    f.residual = (const moe::bf16_t *)residual;
    f.y = (moe::bf16_t *)y;
    f.T = (int)T;
    return moe::launch_stream_fused(x, W1, W3, W2, A, d, d_ff, E, hbuf, o_perm, (float *)scratch,
                                    scratch_bytes, f, gemm1_done, s);
}

int moe_stream_layer_counters(int dt, int64_t T, int k, int d, int d_ff, int E) {
    if (!moe_expert_ffn_streams(dt, T * k, d, d_ff, E) ||
        moe::stream_cols_supported(T, k, d, d_ff, E))
        return 0;
    return (int)moe::stream_gemm1_tiles_max(T * k, d_ff, E);
}

int64_t moe_stream_layer_counter_index(int64_t T, int k, int d, int d_ff) {
    return moe::stream_counter_index(T * k, d, d_ff);
}

const char *moe_expert_ffn_kernel_name(int dt, int64_t A, int d, int d_ff, int E) {
    switch (moe::ffn_path(dt, A, d, d_ff, E)) {
        case moe::FfnPath::kStream:
            return "stream_gemm_kernel";
        case moe::FfnPath::kSkinny:
            return "skinny_gemm_kernel";
        case moe::FfnPath::kGroupedSmall:
            return "grouped_gemm_kernel (128 x 64 tiles)";
        case moe::FfnPath::kGroupedLarge:
            return "grouped_gemm_kernel (256 x 256 tiles)";
        case moe::FfnPath::kWide:
            return moe::wide_token_tile(A, E) == 128 ? "wide_gemm_kernel (128-row token tiles)"
                                                     : "wide_gemm_kernel (256-row token tiles)";
        case moe::FfnPath::kMixed:
            return "grouped_gemm_kernel (128 x 64 tiles) + wide_gemm_kernel (128-row token tiles) "
                   "(W2)";
    }
    return "";
}

const char *moe_forward_kernel_name(int dt, int64_t T, int k, int d, int d_ff, int E) {
    if (moe::ffn_path(dt, T * k, d, d_ff, E) == moe::FfnPath::kStream) {
        if (moe::stream_cols_supported(T, k, d, d_ff, E)) return "stream_cols_kernel";
        if (moe::stream_cols_w2_supported(T, k, d, d_ff, E))
            return "stream_gemm_kernel + stream_cols_kernel (W2)";
    }
    return moe_expert_ffn_kernel_name(dt, T * k, d, d_ff, E);
}

size_t moe_expert_ffn_scratch_bytes(int dt, int64_t A, int d, int d_ff, int E) {
    switch (moe::ffn_path(dt, A, d, d_ff, E)) {
        case moe::FfnPath::kWide:
        case moe::FfnPath::kMixed:
            return moe::wide_partial_bytes(A, E);
        case moe::FfnPath::kStream:
            return moe::stream_partial_bytes(A, d, d_ff, E);
        default:
            return 0;
    }
}

hipError_t moe_launch_expert_ffn(const void *act, const int32_t *gather, const int32_t *offsets,
                                 const void *W1, const void *W3, const void *W2, int dt,
                                 int out_f32, int64_t A, int d, int d_ff, int E, void *hbuf,
                                 void *out, void *scratch, size_t scratch_bytes, hipEvent_t mid,
                                 hipStream_t s) {
    using moe::bf16_t;
    if (dt == 0)
        return moe::launch_ffn_typed<float, float>(act, gather, offsets, W1, W3, W2, A, d, d_ff,
                                                   E, hbuf, out, scratch, scratch_bytes, mid, s);
    if (out_f32)
        return moe::launch_ffn_typed<bf16_t, float>(act, gather, offsets, W1, W3, W2, A, d, d_ff,
                                                    E, hbuf, out, scratch, scratch_bytes, mid, s);
    return moe::launch_ffn_typed<bf16_t, bf16_t>(act, gather, offsets, W1, W3, W2, A, d, d_ff, E,
                                                 hbuf, out, scratch, scratch_bytes, mid, s);
}
