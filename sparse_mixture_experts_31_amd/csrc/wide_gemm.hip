// wide_gemm.hip — the expert GEMMs of large bf16 batches on wide tiles.
//
// The experts are the SwiGLU MLP W2 (silu(W1 x) * W3 x) (fdeinterviews
// breakdown, "The paper in one minute"; tokentrails lineage, Code listing);
// with the rows of each expert contiguous after dispatch they are two grouped
// GEMMs (see expert_gemm.hip for the tile, operand and LDS conventions).
//
// Tiles.  256 weight rows x 256 token rows; for GEMM1 the weight rows are
// 128 rows of W1 and the same 128 rows of W3.  Four waves in a 2 x 2 grid,
// each owning 128 x 128 outputs in 256 accumulator registers (one wave per
// SIMD).  Per 16-wide k-step a wave reads four weight and four token
// fragments and issues 16 v_mfma_f32_32x32x16_bf16: half the LDS reads per
// MFMA of the 8-wave tiles, whose 64 x 128 wave tiles keep the LDS port as
// busy as the matrix cores.
//
// k-loop.  The stage ring of expert_gemm.hip (global_load_lds straight into
// swizzled LDS, explicit vmcnt waits, fence-free barrier) with three changes
// that keep the single wave per SIMD issuing MFMAs:
//  * fragment double buffering: the second k-half of a stage is read under
//    the MFMAs of the first, the next stage's first half under the second
//    half's, and the reads and loads are interleaved one by one with the
//    MFMAs (scheduling groups), so no memory instruction waits at issue
//    behind a full queue while the matrix core idles;
//  * no branches: the slot a stage frees is refilled with the stage P ahead
//    in this segment or the next (a select), and past the last segment with
//    a reload of the same segment that nothing reads, so every stage issues
//    the same loads and every vmcnt wait is a constant;
//  * a ragged token tile runs all MFMAs (rows past the count hold a clamped
//    valid row and are not stored): every wave meets every barrier, so
//    skipping a dead wave's MFMAs would not shorten the tile.
//
// Schedule.  Workgroup b runs on XCD b % 8.  The tiles (token tiles fastest,
// then weight tiles, then experts) are cut into eight contiguous ranges, one
// per XCD; the G8 workgroups of an XCD take its tiles round robin, so the
// tiles in flight on an XCD at any time are neighbours that share weight and
// token rows in its L2.  When the round robin would leave a last round at
// most half full, that round is instead split along K: its tiles' stages are
// divided evenly (in multiples of P stages) over all G8 workgroups.  A
// workgroup whose share covers a tile only in part writes its fp32
// accumulators to a scratch slot; wide_fixup_kernel then sums each split
// tile's parts in workgroup order (a fixed order: the result is
// deterministic) and applies the epilogue.
#include "gemm_common.h"

namespace moe {

namespace {

constexpr int kWideBW = 256, kWideBT = 256, kWideWaves = 4;
constexpr int kWideP = 4;  // stages in the ring
constexpr int kWideRows = kWideBW + kWideBT;
constexpr int kWideLPW = kWideRows / 16 / kWideWaves;  // 16-row loads per wave per stage
constexpr int kWideStageBytes = kWideRows * 64;
constexpr int kWideLds = kWideP * kWideStageBytes;
constexpr int kWideKStep = 32;                   // bf16 K elements per stage
constexpr int kSlotFloats = kWideWaves * kWave * 256;  // accumulators of one workgroup
static_assert(kWideLPW * (kWideP - 1) < 64, "vmcnt range");
static_assert(kWideLds <= 160 * 1024 - 1024, "LDS capacity");

// Per-expert tile table in LDS: first row, row count, first tile number.
struct TileTable {
    int *lo, *cnt, *first;
    int E;
    // Offsets are clamped to [0, A] so no row index leaves the buffers even
    // for a malformed offsets array.  Called by one thread; the caller syncs.
    __device__ void build(const int32_t *offsets, int A, int col_tiles) {
        int f = 0;
        for (int i = 0; i < E; ++i) {
            const int l = min(max(offsets[i], 0), A);
            const int h = min(max(offsets[i + 1], l), A);
            lo[i] = l;
            cnt[i] = h - l;
            first[i] = f;
            f += (h - l + kWideBT - 1) / kWideBT * col_tiles;
        }
        first[E] = f;
    }
    __device__ int total() const { return first[E]; }
    __device__ TileInfo info(int t, int cols) const {
        int i = 0;
        while (i + 1 < E && first[i + 1] <= t) ++i;
        const int rem = t - first[i];
        const int mtiles = (cnt[i] + kWideBT - 1) / kWideBT;
        TileInfo ti;
        ti.e = i;
        ti.row0 = lo[i] + (rem % mtiles) * kWideBT;
        ti.mrem = min(kWideBT, lo[i] + cnt[i] - ti.row0);
        ti.n0 = (rem / mtiles) * cols;
        return ti;
    }
};

// One XCD's share of the tiles and how its last round is handled.
struct XcdShare {
    int lo, n;     // tiles [lo, lo + n)
    int rounds;    // full round-robin rounds
    int left;      // tiles of the last round (split along K when `split`)
    bool split;
    int sk_total;  // stages of the split round
    __device__ XcdShare(int total, int xcd, int G8, int n_k, bool can_split) {
        const int range = (total + 7) / 8;
        lo = xcd * range;
        n = max(0, min(range, total - lo));
        rounds = n / G8;
        left = n - rounds * G8;
        split = can_split && left > 0 && 2 * left <= G8;
        sk_total = split ? left * n_k : 0;
    }
    // First split stage of workgroup w of the XCD (w = G8 gives the end);
    // boundaries are multiples of P stages.
    __device__ int bound(int w, int G8) const {
        return kWideP * (int)((int64_t)w * (sk_total / kWideP) / G8);
    }
};

// A piece of work of a workgroup: stages [sb, se) of one tile; `slot` is -1
// for a whole tile, else which of the workgroup's two scratch slots (its
// first or its last split piece) receives the partial accumulators.
struct Segment {
    int tile, sb, se, slot;
};

// Store fragment (i, j) of a wave's 128 x 128 block: element q of a fragment
// is D[n = 8 (q / 4) + 4 lhalf + q % 4][m = lrow].  GEMM1 passes the u
// fragment and the matching v fragment and stores silu(u) * v.
template <bool SWIGLU, typename TO>
__device__ __forceinline__ void store_fragment(TO *__restrict__ out, int N, const TileInfo &ti,
                                               int wn, int wm, int lane, int i, int j,
                                               const f32x16 &u, const f32x16 &v) {
    const int lrow = lane & 31, lhalf = lane >> 5;
    const int m = wm * 128 + j * 32 + lrow;
    if (m >= ti.mrem) return;
    TO *orow = out + (int64_t)(ti.row0 + m) * N;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
        const int n = ti.n0 + (SWIGLU ? wn * 64 : wn * 128) + i * 32 + 8 * gq + 4 * lhalf;
        if (n < N) {
            float r[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                r[q] = u[4 * gq + q];
                if constexpr (SWIGLU) r[q] = silu(r[q]) * v[4 * gq + q];
            }
            store4<TO>(orow + n, r[0], r[1], r[2], r[3]);
        }
    }
}

// Scratch slot layout: float4 number p (0..63) of thread t at 4 (p * 256 + t),
// p = 4 (4 i + j) + gq, so every store and load of a wave is 1 KiB contiguous.
__device__ __forceinline__ float *slot_ptr(float *partial, int slot) {
    return partial + (size_t)slot * kSlotFloats;
}

}  // namespace

template <bool SWIGLU, typename TO>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void wide_gemm_kernel(
    const bf16_t *__restrict__ act, int64_t act_ld, const int32_t *__restrict__ gather,
    const bf16_t *__restrict__ Wa, const bf16_t *__restrict__ Wb,
    const int32_t *__restrict__ offsets, int E, int N, int K, int A, TO *__restrict__ out,
    float *__restrict__ partial) {
    constexpr int P = kWideP, LPW = kWideLPW, BW = kWideBW;
    constexpr int kCols = SWIGLU ? BW / 2 : BW;  // output columns per tile
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    __shared__ int s_lo[64], s_cnt[64], s_first[65];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    // wave-uniform by construction; saying so keeps the LDS destinations of
    // the loads (M0) in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int n_k = K / kWideKStep;  // >= P, checked by the launcher

    TileTable tt{s_lo, s_cnt, s_first, E};
    if (tid == 0) tt.build(offsets, A, (N + kCols - 1) / kCols);
    __syncthreads();

    const int G8 = gridDim.x / 8;  // workgroups per XCD (grid is a multiple of 8)
    const int xcd = blockIdx.x % 8, wj = blockIdx.x / 8;
    const XcdShare xs(tt.total(), xcd, G8, n_k, partial != nullptr && n_k % P == 0);
    // this workgroup's whole tiles, then its split stages [sk_lo, sk_hi)
    const int n_rr = xs.split ? xs.rounds : (xs.n > wj ? (xs.n - wj + G8 - 1) / G8 : 0);
    const int sk_lo = xs.split ? xs.bound(wj, G8) : 0;
    const int sk_hi = xs.split ? xs.bound(wj + 1, G8) : 0;
    const int n_sk = sk_hi > sk_lo ? (sk_hi - 1) / n_k - sk_lo / n_k + 1 : 0;
    const int n_seg = n_rr + n_sk;
    if (n_seg == 0) return;  // uniform over the workgroup

    auto segment = [&](int k) {
        Segment sg;
        if (k < n_rr) {
            sg.tile = xs.lo + k * G8 + wj;
            sg.sb = 0;
            sg.se = n_k;
            sg.slot = -1;
        } else {
            const int j = k - n_rr;
            const int tr = sk_lo / n_k + j;  // tile within the split round
            sg.tile = xs.lo + xs.rounds * G8 + tr;
            sg.sb = (j == 0) ? sk_lo - tr * n_k : 0;
            sg.se = min(n_k, sk_hi - tr * n_k);
            sg.slot = (sg.sb == 0 && sg.se == n_k) ? -1 : (j == 0 ? 0 : 1);
        }
        return sg;
    };

    // Lane pointers of this wave's LPW 16-row loads of a tile: row r of a
    // stage is loaded by wave (r / 16) % 4, lane 4 (r % 16) + chunk slot,
    // fetching the chunk that belongs at that slot.  Loads [0, LPW / 2) are
    // weight rows, the rest token rows (act rows, through `gather` if set).
    auto sources = [&](const TileInfo &ti, const char *(&src)[LPW]) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int r = (wave + kWideWaves * i) * 16 + (lane >> 2);
            const int c = (lane & 3) ^ ((r >> 2) & 3);
            if (i < LPW / 2) {
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
                const int row = act_row<16>(gather, ti.row0 + (wave + kWideWaves * i) * 16 - BW,
                                            ti.row0 + ti.mrem - 1, lane);
                src[i] = (const char *)(act + (int64_t)row * act_ld) + c * 16;
            }
        }
    };

    const int wn = wave & 1, wm = wave >> 1;
    const int lrow = lane & 31, lhalf = lane >> 5;
    // LDS row of weight fragment i (GEMM1: 0,1 are W1 rows, 2,3 the same W3 rows)
    auto wrow = [&](int i) {
        if constexpr (SWIGLU)
            return (i < 2 ? 0 : BW / 2) + wn * 64 + (i & 1) * 32;
        else
            return wn * 128 + i * 32;
    };
    const int trow0 = BW + wm * 128;

    f32x16 acc[4][4];
    i32x4 a0[4], b0[4], a1[4], b1[4];
    auto load_frags = [&](i32x4 (&a)[4], i32x4 (&b)[4], int slot, int t) {
        const char *base = smem + slot * kWideStageBytes;
        const int c = 2 * t + lhalf;
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *(const i32x4 *)(base + lds_off(wrow(i) + lrow, c));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            b[j] = *(const i32x4 *)(base + lds_off(trow0 + j * 32 + lrow, c));
    };
    auto mma = [&](const i32x4 (&a)[4], const i32x4 (&b)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mma_step<bf16_t>(a[i], b[j], acc[i][j]);
    };

    // The producer runs P stages ahead of the consumer with its own cursor:
    // pp are its lane pointers into the next stage to load, p_left the
    // stages left in its segment.  Every segment holds at least P stages
    // (whole tiles n_k >= P, split pieces multiples of P).  Past the last
    // segment it reloads the first stages of that segment, which nothing
    // reads, so every stage issues the same loads.
    const char *pp[LPW];
    int p_left;
    auto produce_from = [&](int k) {
        const Segment sg = segment(min(k, n_seg - 1));
        sources(tt.info(sg.tile, kCols), pp);
#pragma unroll
        for (int i = 0; i < LPW; ++i) pp[i] += (int64_t)sg.sb * 64;
        p_left = (k < n_seg) ? sg.se - sg.sb : 0x7fffffff;
    };
    int p_seg = 0;
    produce_from(0);
#pragma unroll
    for (int g = 0; g < P; ++g) {
        char *dst = smem + g * kWideStageBytes;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            dma16(pp[i], dst + (wave + kWideWaves * i) * 1024);
            pp[i] += 64;
        }
    }
    p_left -= P;
    if (p_left == 0) produce_from(++p_seg);
    wait_vmcnt_lgkm0<LPW * (P - 1)>();
    stage_barrier();
    load_frags(a0, b0, 0, 0);

    int g = 0;  // stages consumed so far = ring cursor
    for (int c_k = 0; c_k < n_seg; ++c_k) {
        const Segment cur = segment(c_k);
        const TileInfo ti = tt.info(cur.tile, kCols);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
        // Only fragment reads are pending inside the k-loop; a clean count
        // here lets the compiler's own waits stay exact.
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)

        for (int s = cur.sb; s < cur.se; ++s, ++g) {
            const int slot = g % P;
            // Second k-half of this stage, under the MFMAs of the first.
            __builtin_amdgcn_sched_barrier(0);
            load_frags(a1, b1, slot, 1);
            mma(a0, b0);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            __builtin_amdgcn_sched_barrier(0);
            // Next stage landed (this wave's loads, then everyone's), and
            // every wave is done reading this slot.
            wait_vmcnt_lgkm0<LPW * (P - 2)>();
            stage_barrier();
            // Refill this slot P stages ahead; read the next stage's first
            // k-half; both under the MFMAs of this stage's second half.
            char *dst = smem + slot * kWideStageBytes;
            load_frags(a0, b0, (g + 1) % P, 0);
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                dma16(pp[i], dst + (wave + kWideWaves * i) * 1024);
                pp[i] += 64;
            }
            mma(a1, b1);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // one global->LDS load
            }
            __builtin_amdgcn_sched_barrier(0);
            // The reads above were issued before eight MFMAs and have landed;
            // saying so keeps the compiler's next wait at the next eight.
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
            if (--p_left == 0) produce_from(++p_seg);  // the producer's next segment
        }

        if (cur.slot < 0) {
            // Epilogue.  Each fragment is pinned in accumulator registers up
            // to its turn, so they are moved out one at a time and not all
            // 256 at the loop exit.
            constexpr int NI = SWIGLU ? 2 : 4;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    asm volatile("" : "+a"(acc[i][j]));
                    if constexpr (SWIGLU) asm volatile("" : "+a"(acc[i + 2][j]));
                    store_fragment<SWIGLU, TO>(out, N, ti, wn, wm, lane, i, j, acc[i][j],
                                               acc[SWIGLU ? i + 2 : i][j]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
            float *dst = slot_ptr(partial, blockIdx.x * 2 + cur.slot);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    asm volatile("" : "+a"(acc[i][j]));
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int p = 4 * (4 * i + j) + gq;
                        *(float4 *)(dst + 4 * (p * 256 + tid)) =
                            make_float4(acc[i][j][4 * gq], acc[i][j][4 * gq + 1],
                                        acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }
    wait_vmcnt_lgkm0<0>();  // the trailing reloads land before the wave ends
}

// Sums the parts of every split tile in workgroup order and applies the
// epilogue.  Block b handles fragment b % 16 (GEMM1: u/v pair b % 8; the
// other eight blocks exit) of tile b / 128 of the split round of XCD
// (b / 16) % 8: one fragment per block keeps many loads in flight.
template <bool SWIGLU, typename TO>
__global__ __launch_bounds__(256) void wide_fixup_kernel(const int32_t *__restrict__ offsets,
                                                         int E, int N, int K, int A, int G8,
                                                         TO *__restrict__ out,
                                                         const float *__restrict__ partial) {
    constexpr int kCols = SWIGLU ? kWideBW / 2 : kWideBW;
    __shared__ int s_lo[64], s_cnt[64], s_first[65];
    __shared__ int s_slots[64], s_nparts, s_tile;  // G8 <= 64: one part per workgroup at most
    const int tid = threadIdx.x;
    const int n_k = K / kWideKStep;
    TileTable tt{s_lo, s_cnt, s_first, E};
    const int frag = blockIdx.x % 16, xcd = (blockIdx.x / 16) % 8, jr = blockIdx.x / 128;
    if (SWIGLU && frag >= 8) return;
    if (tid == 0) {
        tt.build(offsets, A, (N + kCols - 1) / kCols);
        const XcdShare xs(tt.total(), xcd, G8, n_k, n_k % kWideP == 0);
        int np = 0;
        if (xs.split && jr < xs.left) {
            const int t_lo = jr * n_k, t_hi = t_lo + n_k;
            for (int w = 0; w < G8 && np >= 0; ++w) {
                const int b_lo = xs.bound(w, G8), b_hi = xs.bound(w + 1, G8);
                if (b_hi <= t_lo || b_lo >= t_hi || b_hi <= b_lo) continue;
                if (b_lo <= t_lo && b_hi >= t_hi) {
                    np = -1;  // one workgroup did the whole tile and stored it
                    break;
                }
                // its first split tile went to slot 0, a later one to slot 1
                s_slots[np++] = (w * 8 + xcd) * 2 + (jr == b_lo / n_k ? 0 : 1);
            }
            s_tile = xs.lo + xs.rounds * G8 + jr;
        }
        s_nparts = np;
    }
    __syncthreads();
    const int np = s_nparts;
    if (np <= 0) return;
    const TileInfo ti = tt.info(s_tile, kCols);
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int wn = wave & 1, wm = wave >> 1;
    auto load_sum = [&](int i, int j) {
        f32x16 r{};
#pragma unroll 4
        for (int k = 0; k < np; ++k) {
            const float *src = partial + (size_t)s_slots[k] * kSlotFloats;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int p = 4 * (4 * i + j) + gq;
                const float4 v = *(const float4 *)(src + 4 * (p * 256 + tid));
                r[4 * gq] += v.x;
                r[4 * gq + 1] += v.y;
                r[4 * gq + 2] += v.z;
                r[4 * gq + 3] += v.w;
            }
        }
        return r;
    };
    // GEMM1: u/v fragment pair (i, j), i < 2; GEMM2: fragment (i, j)
    const int i = frag / 4, j = frag % 4;
    const f32x16 u = load_sum(i, j);
    const f32x16 v = SWIGLU ? load_sum(i + 2, j) : u;
    store_fragment<SWIGLU, TO>(out, N, ti, wn, wm, lane, i, j, u, v);
}

namespace {

// one workgroup per CU, a multiple of 8 (one share per XCD), at most 64 per XCD
int wide_grid() { return std::max(8, std::min(device_cus(), 512) / 8 * 8); }

template <bool SWIGLU, typename TO>
hipError_t launch_wide(const void *act, int64_t act_ld, const int32_t *gather, const void *Wa,
                       const void *Wb, const int32_t *offsets, int E, int N, int K, int64_t A,
                       void *out, float *partial, hipStream_t s) {
    auto kern = wide_gemm_kernel<SWIGLU, TO>;
    hipError_t err = hipFuncSetAttribute((const void *)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, kWideLds);
    if (err != hipSuccess) return err;
    const int grid = wide_grid();
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), kWideLds, s, (const bf16_t *)act, act_ld,
                       gather, (const bf16_t *)Wa, (const bf16_t *)Wb, offsets, E, N, K, (int)A,
                       (TO *)out, partial);
    if ((err = hipGetLastError()) != hipSuccess || !partial) return err;
    hipLaunchKernelGGL((wide_fixup_kernel<SWIGLU, TO>), dim3(grid * 16), dim3(256), 0, s, offsets,
                       E, N, K, (int)A, grid / 8, (TO *)out, (const float *)partial);
    return hipGetLastError();
}

}  // namespace

size_t wide_partial_bytes() { return (size_t)2 * wide_grid() * kSlotFloats * sizeof(float); }

bool wide_supported(int d, int d_ff) {
    return d >= kWideP * kWideKStep && d_ff >= kWideP * kWideKStep;
}

hipError_t launch_wide_ffn(const void *act, const int32_t *gather, const int32_t *offsets,
                           const void *W1, const void *W3, const void *W2, int out_f32, int64_t A,
                           int d, int d_ff, int E, void *hbuf, void *out, float *partial,
                           size_t partial_bytes, hipEvent_t mid, hipStream_t s) {
    if (partial && partial_bytes < wide_partial_bytes()) partial = nullptr;  // no splits
    hipError_t err = launch_wide<true, bf16_t>(act, d, gather, W1, W3, offsets, E, d_ff, d, A,
                                               hbuf, partial, s);
    if (err == hipSuccess && mid) err = hipEventRecord(mid, s);
    if (err != hipSuccess) return err;
    if (out_f32)
        return launch_wide<false, float>(hbuf, d_ff, nullptr, W2, nullptr, offsets, E, d, d_ff,
                                         A, out, partial, s);
    return launch_wide<false, bf16_t>(hbuf, d_ff, nullptr, W2, nullptr, offsets, E, d, d_ff, A,
                                      out, partial, s);
}

}  // namespace moe
