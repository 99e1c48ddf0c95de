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
// SIMD) as 8 x 8 fragments of v_mfma_f32_16x16x32_bf16, the MFMA form that
// sustains the most throughput on random data.  Per 32-wide k-step a wave
// reads eight weight and eight token fragments and issues 64 MFMAs.  When
// the experts hold about 100 rows or fewer, a second instantiation uses
// 128-row token tiles (128 x 64 per wave, 8 x 4 fragments), so less of
// each tile is padding.
//
// k-loop.  A stage is 64 k: one whole 128-byte line of every weight and token
// row, fetched by global_load_lds (eight lines per instruction) into a
// swizzled two-slot LDS ring, with explicit vmcnt waits and a fence-free
// barrier.  Fragments are double buffered: step 0 of a stage runs under the
// reads of step 1, then one barrier frees the slot (its reads have landed),
// and step 1 runs under the reads of the next stage's step 0 and the loads
// that refill the slot two stages ahead, spread over the step so the
// load path never backs up into the MFMA issue.  Scheduling groups fix the
// interleaving; the loop has no branches (the slot a stage frees is refilled
// with the stage two ahead in this segment or the next, and past the last
// segment with a reload that nothing reads), so every vmcnt wait is a
// constant.  A ragged token tile runs all MFMAs (rows past the count hold a
// clamped valid row and are not stored): every wave meets every barrier, and
// a second fragment count in the same kernel costs the full one registers.
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

constexpr int kWideBW = 256, kWideWaves = 4;
constexpr int kWideP = 2;  // stages in the ring (double buffer)
constexpr int kWidePfBytes = 256;  // where the L2 prefetches land (never read)
// The token-tile height BT: 256, or 128 when the experts hold about 100 rows
// or fewer (most of a 256-row tile would be padding).
template <int BT>
struct WideTile {
    static constexpr int kRows = kWideBW + BT;
    static constexpr int kLPW = kRows / 8 / kWideWaves;  // 8-row loads per wave per stage
    static constexpr int kStageBytes = kRows * 128;
    static constexpr int kLds = kWideP * kStageBytes + kWidePfBytes;
    static constexpr int kNJ = BT / 32;  // token fragments per wave
    static constexpr int kFW = 8 * kNJ;  // fragments per wave
    // a scratch slot: the accumulators of one workgroup
    static constexpr int kSlotFloats = kWideWaves * kWave * 4 * kFW;
    static_assert(kLPW * (kWideP - 1) < 64, "vmcnt range");
    static_assert(kLds <= 160 * 1024 - 1024, "LDS capacity");
};
constexpr int kWidePfAhead = 2;   // stages past the one being loaded
constexpr int kWideKStep = 64;                   // bf16 K elements per stage

// Byte offset of 16-byte chunk c of row r in a stage of 128-byte rows: the
// chunk sits at c ^ ((r >> 1) & 7), so a 32-row operand read (16 lanes per
// LDS cycle on 16 rows of one chunk) hits 16 distinct bank groups.
__device__ __forceinline__ int swz128(int r, int c) {
    return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
}

// Per-expert tile table in LDS: first row, row count, first tile number.
template <int BT>
struct TileTable {
    int *lo, *cnt, *first;
    int E;
    // Called by one whole wave; the caller syncs.
    __device__ void build(const int32_t *offsets, int A, int col_tiles) {
        build_expert_table(offsets, E, A, BT, col_tiles, lo, cnt, first);
    }
    // The table is the same for every lane: reading it through
    // readfirstlane keeps the tile and segment arithmetic in scalar
    // registers, away from the vector registers the k-loop needs.
    __device__ static int u(int v) { return __builtin_amdgcn_readfirstlane(v); }
    __device__ int total() const { return u(first[E]); }
    __device__ TileInfo info(int t, int cols) const {
        int i = 0;
        while (i + 1 < E && u(first[i + 1]) <= t) ++i;
        const int rem = t - u(first[i]);
        const int c = u(cnt[i]), l = u(lo[i]);
        const int mtiles = (c + BT - 1) / BT;
        TileInfo ti;
        ti.e = i;
        ti.mt = rem % mtiles;
        ti.row0 = l + ti.mt * BT;
        ti.mrem = min(BT, l + c - ti.row0);
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

// Store fragment (i, j) of a wave's 128 x 128 block: lane l holds the
// outputs of token row m = 32 j + 16 wm + l % 16 and weight rows
// 16 i + 4 (l / 16) .. + 4.  GEMM1 passes the u fragment and the matching v
// fragment and stores silu(u) * v.
template <bool SWIGLU, typename TO>
__device__ __forceinline__ void store_fragment(TO *__restrict__ out, int N, const TileInfo &ti,
                                               int wn, int wm, int lane, int i, int j,
                                               const f32x4 &u, const f32x4 &v) {
    const int m = (2 * j + wm) * 16 + (lane & 15);
    if (m >= ti.mrem) return;
    const int n = ti.n0 + (SWIGLU ? wn * 64 : wn * 128) + i * 16 + 4 * (lane >> 4);
    if (n >= N) return;
    float r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        r[q] = u[q];
        if constexpr (SWIGLU) r[q] = silu(r[q]) * v[q];
    }
    store4<TO>(out + (int64_t)(ti.row0 + m) * N + n, r[0], r[1], r[2], r[3]);
}

// Says that every accumulator is in an accumulator register here.
template <int NJ>
__device__ __forceinline__ void pin_accumulators(f32x4 (&acc)[8][NJ]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// Scratch slot layout: fragment p = NJ i + j of thread t at float4
// p * 256 + t, so every store and load of a wave is 1 KiB contiguous.
template <int BT>
__device__ __forceinline__ float *slot_ptr(float *partial, int slot) {
    return partial + (size_t)slot * WideTile<BT>::kSlotFloats;
}

}  // namespace

template <bool SWIGLU, typename TO, int BT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void wide_gemm_kernel(
    const bf16_t *__restrict__ act, int64_t act_ld, const int32_t *__restrict__ gather,
    const bf16_t *__restrict__ Wa, const bf16_t *__restrict__ Wb,
    const int32_t *__restrict__ offsets, int E, int N, int K, int A, TO *__restrict__ out,
    float *__restrict__ partial) {
    using C = WideTile<BT>;
    constexpr int P = kWideP, LPW = C::kLPW, BW = kWideBW, NJ = C::kNJ, FW = C::kFW;
    constexpr int kWideStageBytes = C::kStageBytes;
    constexpr int kCols = SWIGLU ? BW / 2 : BW;  // output columns per tile
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    __shared__ int s_lo[64], s_cnt[64], s_first[65];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    // wave-uniform by construction; saying so keeps the LDS destinations of
    // the loads (M0) in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int n_k = K / kWideKStep;  // >= P, checked by the launcher

    TileTable<BT> tt{s_lo, s_cnt, s_first, E};
    if (wave == 0) tt.build(offsets, A, (N + kCols - 1) / kCols);
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

    // Sources of this wave's LPW 8-row loads of a tile: row r of a stage is
    // loaded by wave (r / 8) % 4, lane 8 (r % 8) + chunk slot, fetching the
    // chunk that belongs at that slot; every load instruction moves eight
    // whole 128-byte lines.  Loads [0, LPW / 4) read base[0] (GEMM1: W1
    // rows), [LPW / 4, LPW / 2) base[1] (the same W3 rows), the rest base[2]
    // (token rows: act rows, through `gather` if set).  A load's address is a
    // wave-uniform base plus a 32-bit lane offset, so the bases advance in
    // scalar registers and the loads take the scalar-base address form.
    auto sources = [&](const TileInfo &ti, const char *(&base)[3], uint32_t (&off)[LPW]) {
        const bf16_t *W = Wa + ((int64_t)ti.e * N + ti.n0) * K;
        base[0] = (const char *)W;
        base[1] = SWIGLU ? (const char *)(Wb + ((int64_t)ti.e * N + ti.n0) * K) : base[0];
        base[2] = (const char *)(act + (gather ? 0 : (int64_t)ti.row0 * act_ld));
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int r = (wave + kWideWaves * i) * 8 + (lane >> 3);
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            if (i < BW / 32) {
                const int rr = SWIGLU ? r % (BW / 2) : r;  // row within the tile's rows of W
                off[i] = (uint32_t)(min(ti.n0 + rr, N - 1) - ti.n0) * (uint32_t)(K * 2) + c * 16;
            } else {
                const int row = act_row<8>(gather, ti.row0 + (wave + kWideWaves * i) * 8 - BW,
                                           ti.row0 + ti.mrem - 1, lane);
                off[i] = (uint32_t)(gather ? row : row - ti.row0) * (uint32_t)(act_ld * 2) + c * 16;
            }
        }
    };

    const int wn = wave & 1, wm = wave >> 1;
    // LDS row of weight fragment i (GEMM1: 0..3 are W1 rows, 4..7 the same
    // W3 rows)
    auto wrow = [&](int i) {
        if constexpr (SWIGLU)
            return (i < 4 ? 0 : BW / 2) + wn * 64 + (i & 3) * 16;
        else
            return wn * 128 + i * 16;
    };
    // LDS row of token fragment j: the two wave rows interleave 16-row
    // fragments, so the first 32 j + 32 token rows sit in fragments <= j.
    auto trow = [&](int j) { return BW + (2 * j + wm) * 16; };
    // Lane part of a fragment read for k-step s of a stage: row l % 16 of the
    // fragment, 16-byte chunk 4 s + l / 16 (fragment rows start at multiples
    // of 16, so the swizzle depends on the lane only).
    const int lr = lane & 15, lq = lane >> 4, lx = (lr >> 1) & 7;
    const int roff[2] = {lr * 128 + ((lq ^ lx) << 4), lr * 128 + (((4 + lq) ^ lx) << 4)};

    f32x4 acc[8][NJ];
    i32x4 a0[8], b0[NJ], a1[8], b1[NJ];
    // Fragment read k of k-step s (k < 8: weight fragment k, else token
    // fragment k - 8) from a slot.
    auto read_frag = [&](i32x4 (&a)[8], i32x4 (&b)[NJ], int slot, int s, int k)
        __attribute__((always_inline)) {
        const char *base = smem + slot * kWideStageBytes + roff[s];
        if (k < 8)
            a[k] = *(const i32x4 *)(base + wrow(k) * 128);
        else
            b[k - 8] = *(const i32x4 *)(base + trow(k - 8) * 128);
    };
    // MFMAs [m0, m1) of a k-step, fragment (m / NJ, m % NJ) for MFMA m.
    auto mma_part = [&](const i32x4 (&a)[8], const i32x4 (&b)[NJ], int m0, int m1)
        __attribute__((always_inline)) {
#pragma unroll
        for (int m = m0; m < m1; ++m)
            acc[m / NJ][m % NJ] = mma16(a[m / NJ], b[m % NJ], acc[m / NJ][m % NJ]);
    };

    // The producer runs P stages ahead of the consumer with its own cursor:
    // pp are its lane pointers into the next stage to load, p_left the
    // stages left in its segment.  Every segment holds at least P stages
    // (whole tiles n_k >= P, split pieces multiples of P).  Past the last
    // segment it reloads the first stages of that segment, which nothing
    // reads, so every stage issues the same loads.
    const char *pb[3];   // wave-uniform bases of the producer's next stage
    uint32_t po[LPW];    // lane offsets from them
    int p_left;
    // L2 prefetch.  The four workgroups of an XCD that share a weight tile
    // (its four token tiles, neighbours in the round robin) each touch a
    // quarter of its rows kWidePfAhead stages before they are loaded, so the
    // loads that follow hit in L2 instead of waiting on HBM.  Lane l covers
    // half l / 16 % 2 of weight row 64 (mt % 4) + 16 wave + l % 16 (rows of
    // one of W1 and W3 per wave).
    const char *pfb;     // wave-uniform base of the stage the last loads went to
    uint32_t pfo;
    int pf_rem;          // stages of the producer's segment from pfb on
    auto produce_from = [&](int k) __attribute__((always_inline)) {
        const Segment sg = segment(min(k, n_seg - 1));
        const TileInfo ti = tt.info(sg.tile, kCols);
        sources(ti, pb, po);
#pragma unroll
        for (int b = 0; b < 3; ++b) pb[b] += (int64_t)sg.sb * 128;
        p_left = (k < n_seg) ? sg.se - sg.sb : 0x7fffffff;
        const int r0 = 64 * (ti.mt & 3) + 16 * wave;  // wave-uniform; r0 % 16 == 0
        const int r = r0 + (lane & 15);
        const int rr = SWIGLU ? r % (BW / 2) : r;
        pfb = (SWIGLU && r0 >= BW / 2) ? pb[1] : pb[0];
        pfo = (uint32_t)(min(ti.n0 + rr, N - 1) - ti.n0) * (uint32_t)(K * 2) +
              ((lane >> 4) & 1) * 64;
        pf_rem = sg.se - sg.sb;
    };
    // The loads of one stage into LDS slot dst, then the bases move on.
    auto load_stage = [&](char *dst, int i) __attribute__((always_inline)) {
        dma16(pb[i < BW / 64 ? 0 : i < BW / 32 ? 1 : 2] + po[i], dst + (wave + kWideWaves * i) * 1024);
    };
    auto advance = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < 3; ++b) pb[b] += 128;
    };
    // One prefetch per wave, after the loads of a stage (pfb is that
    // stage): kWidePfAhead stages further, within the producer's segment
    // (past the last segment the reloads stay within its first P stages).
    auto prefetch = [&]() __attribute__((always_inline)) {
        const int ahead = max(0, min(kWidePfAhead, pf_rem - 1));
        --pf_rem;
        __builtin_amdgcn_global_load_lds((const void *)(pfb + ahead * 128 + pfo),
                                         (__attribute__((address_space(3))) void *)(smem + kWideP * kWideStageBytes),
                                         4, 0, 0);
        pfb += 128;
    };
    int p_seg = 0;
    produce_from(0);
#pragma unroll
    for (int g = 0; g < P; ++g) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) load_stage(smem + g * kWideStageBytes, i);
        advance();
        prefetch();
        --p_left;
    }
    if (p_left == 0) produce_from(++p_seg);
    // stage 0 has landed (stage 1's loads and prefetch may be in flight)
    wait_vmcnt_lgkm0<(LPW + 1) * (P - 1)>();
    stage_barrier();

    int g = 0;  // stages consumed so far = ring cursor
    for (int c_k = 0; c_k < n_seg; ++c_k) {
        const Segment cur = segment(c_k);
        const TileInfo ti = tt.info(cur.tile, kCols);
        // Accumulators start at zero, and are held in the accumulator
        // registers (said at the start and at the end of every stage, so
        // the allocator never parks one in a vector register).
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{};
        pin_accumulators(acc);
        // The k-loop of one segment.  Each step is cut into chunks by
        // scheduling barriers, so every read and load issues between the
        // MFMAs it is placed among.
        // Step 0 of the segment's first stage (the previous segment read it
        // too, but the ring may have moved on since).
#pragma unroll
        for (int k = 0; k < 8 + NJ; ++k) read_frag(a0, b0, g % P, 0, k);
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        for (int s = cur.sb; s < cur.se; ++s, ++g) {
            const int slot = g % P;
            // Step 0 under the reads of step 1, one per MFMA, so the last
            // read has FW - 8 - NJ MFMAs to land under.
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < FW; ++m) {
                if (m < 8 + NJ) read_frag(a1, b1, slot, 1, m);
                mma_part(a0, b0, m, m + 1);
                __builtin_amdgcn_sched_barrier(0);
            }
            // Every read of this slot has landed and the next stage's loads
            // too (this wave's, then everyone's): free the slot.
            // (the last prefetch may still be in flight: it was issued after
            // those loads)
            wait_vmcnt_lgkm0<(LPW + 1) * (P - 2) + 1>();
            stage_barrier();
            // Step 1 under the reads of the next stage's step 0 (one per two
            // MFMAs) and the loads refilling this slot P stages ahead (spread
            // evenly over the whole step, one per four MFMAs for 256-row
            // tiles, so the load path never backs up into the issue).
            char *dst = smem + slot * kWideStageBytes;
#pragma unroll
            for (int m = 0; m < FW; ++m) {
                if (m % 2 == 0 && m / 2 < 8 + NJ) read_frag(a0, b0, (g + 1) % P, 0, m / 2);
#pragma unroll
                for (int l = 0; l < LPW; ++l)
                    if ((l * FW) / LPW == m) load_stage(dst, l);
                if (m == FW - 1) {
                    advance();
                    prefetch();
                }
                mma_part(a1, b1, m, m + 1);
                __builtin_amdgcn_sched_barrier(0);
            }
            // The reads above have landed by now; saying so keeps the
            // compiler's next wait exact.
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
            if (--p_left == 0) produce_from(++p_seg);  // the producer's next segment
            pin_accumulators(acc);
        }

        if (cur.slot < 0) {
            // Epilogue.  Each fragment is pinned in accumulator registers up
            // to its turn, so they are moved out a few at a time and not all
            // 256 at the loop exit.
            constexpr int NI = SWIGLU ? 4 : 8;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    asm volatile("" : "+a"(acc[i][j]));
                    if constexpr (SWIGLU) asm volatile("" : "+a"(acc[i + 4][j]));
                    store_fragment<SWIGLU, TO>(out, N, ti, wn, wm, lane, i, j, acc[i][j],
                                               acc[SWIGLU ? i + 4 : i][j]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
            float *dst = slot_ptr<BT>(partial, blockIdx.x * 2 + cur.slot);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    asm volatile("" : "+a"(acc[i][j]));
                    const int p = NJ * i + j;
                    *(f32x4 *)(dst + 4 * (p * 256 + tid)) = acc[i][j];
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }
    wait_vmcnt_lgkm0<0>();  // the trailing reloads land before the wave ends
}

// Sums the parts of every split tile in workgroup order and applies the
// epilogue.  With FB = FW / 4 blocks per tile (16 for 256-row tiles), block b
// handles fragments 4 (b % FB) .. + 4 of every wave (GEMM1: u fragments,
// with their v fragments FW / 2 further; the other half of the blocks exit)
// of tile b / (8 FB) of the split round of XCD (b / FB) % 8: a few fragments
// per block keep many loads in flight.
template <bool SWIGLU, typename TO, int BT>
__global__ __launch_bounds__(256) void wide_fixup_kernel(const int32_t *__restrict__ offsets,
                                                         int E, int N, int K, int A, int G8,
                                                         TO *__restrict__ out,
                                                         const float *__restrict__ partial) {
    constexpr int kCols = SWIGLU ? kWideBW / 2 : kWideBW;
    __shared__ int s_lo[64], s_cnt[64], s_first[65];
    __shared__ int s_slots[64], s_nparts;  // G8 <= 64: one part per workgroup at most
    const int tid = threadIdx.x;
    const int n_k = K / kWideKStep;
    constexpr int NJ = WideTile<BT>::kNJ, FW = WideTile<BT>::kFW, FB = FW / 4;
    TileTable<BT> tt{s_lo, s_cnt, s_first, E};
    const int frag = blockIdx.x % FB, xcd = (blockIdx.x / FB) % 8, jr = blockIdx.x / (8 * FB);
    if (SWIGLU && frag >= FB / 2) return;
    if (tid < kWave) tt.build(offsets, A, (N + kCols - 1) / kCols);
    __syncthreads();
    const XcdShare xs(tt.total(), xcd, G8, n_k, n_k % kWideP == 0);
    if (!xs.split || jr >= xs.left) return;  // uniform over the workgroup
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    if (wave == 0) {
        // lane w < G8: does workgroup w's share of the split stages cover
        // this tile in part (a partial in one of its slots) or whole (it
        // stored the tile itself)?  Parts are taken in workgroup order.
        const int t_lo = jr * n_k, t_hi = t_lo + n_k;
        bool part = false, whole = false;
        int slot = 0;
        if (lane < G8) {
            const int b_lo = xs.bound(lane, G8), b_hi = xs.bound(lane + 1, G8);
            const bool overlap = !(b_hi <= t_lo || b_lo >= t_hi || b_hi <= b_lo);
            whole = overlap && b_lo <= t_lo && b_hi >= t_hi;
            part = overlap && !whole;
            // its first split tile went to slot 0, a later one to slot 1
            slot = (lane * 8 + xcd) * 2 + (jr == b_lo / n_k ? 0 : 1);
        }
        const uint64_t wm = __ballot(whole), pm = __ballot(part);
        const uint64_t lower_lanes = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        if (part && !wm) s_slots[__popcll(pm & lower_lanes)] = slot;
        if (lane == 0) s_nparts = wm ? -1 : __popcll(pm);
    }
    __syncthreads();
    const int np = s_nparts;
    if (np <= 0) return;
    const TileInfo ti = tt.info(xs.lo + xs.rounds * G8 + jr, kCols);
    const int wn = wave & 1, wm = wave >> 1;
    auto load_sum = [&](int p) {
        f32x4 r{};
#pragma unroll 4
        for (int k = 0; k < np; ++k)
            r += *(const f32x4 *)(partial + (size_t)s_slots[k] * WideTile<BT>::kSlotFloats +
                                  4 * (p * 256 + tid));
        return r;
    };
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int p = 4 * frag + q;  // GEMM1: u fragment (p < FW / 2); GEMM2: any fragment
        const f32x4 u = load_sum(p);
        const f32x4 v = SWIGLU ? load_sum(p + FW / 2) : u;
        store_fragment<SWIGLU, TO>(out, N, ti, wn, wm, lane, p / NJ, p % NJ, u, v);
    }
}

namespace {

// one workgroup per CU, a multiple of 8 (one share per XCD), at most 64 per XCD
int wide_grid() { return std::max(8, std::min(device_cus(), 512) / 8 * 8); }

// `after`, if set, is recorded right after the GEMM kernel, before the fixup.
template <bool SWIGLU, typename TO, int BT>
hipError_t launch_wide_bt(const void *act, int64_t act_ld, const int32_t *gather, const void *Wa,
                          const void *Wb, const int32_t *offsets, int E, int N, int K, int64_t A,
                          void *out, float *partial, hipStream_t s, hipEvent_t after) {
    using C = WideTile<BT>;
    auto kern = wide_gemm_kernel<SWIGLU, TO, BT>;
    hipError_t err = set_lds_limit<wide_gemm_kernel<SWIGLU, TO, BT>>(C::kLds);
    if (err != hipSuccess) return err;
    const int grid = wide_grid();
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), C::kLds, s, (const bf16_t *)act, act_ld,
                       gather, (const bf16_t *)Wa, (const bf16_t *)Wb, offsets, E, N, K, (int)A,
                       (TO *)out, partial);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (after && (err = hipEventRecord(after, s)) != hipSuccess) return err;
    if (!partial) return err;
    hipLaunchKernelGGL((wide_fixup_kernel<SWIGLU, TO, BT>), dim3(grid * (C::kFW / 4)), dim3(256),
                       0, s, offsets, E, N, K, (int)A, grid / 8, (TO *)out,
                       (const float *)partial);
    return hipGetLastError();
}

// 128-row token tiles up to 100 rows per expert on average (measured on
// MI355X with d = 4096, d_ff = 14336, E = 8: 16 % faster at 57-96 rows, 10 %
// slower from 128 on, where 256-row tiles are fuller), else 256.
template <bool SWIGLU, typename TO>
hipError_t launch_wide(const void *act, int64_t act_ld, const int32_t *gather, const void *Wa,
                       const void *Wb, const int32_t *offsets, int E, int N, int K, int64_t A,
                       void *out, float *partial, hipStream_t s, hipEvent_t after = nullptr) {
    if (wide_token_tile(A, E) == 128)
        return launch_wide_bt<SWIGLU, TO, 128>(act, act_ld, gather, Wa, Wb, offsets, E, N, K, A,
                                               out, partial, s, after);
    return launch_wide_bt<SWIGLU, TO, 256>(act, act_ld, gather, Wa, Wb, offsets, E, N, K, A, out,
                                           partial, s, after);
}

}  // namespace

int wide_token_tile(int64_t A, int E) { return A <= 100 * (int64_t)E ? 128 : 256; }

size_t wide_partial_bytes(int64_t A, int E) {
    const size_t slot = wide_token_tile(A, E) == 128 ? WideTile<128>::kSlotFloats
                                                     : WideTile<256>::kSlotFloats;
    return (size_t)2 * wide_grid() * slot * sizeof(float);
}

bool wide_supported(int64_t A, int d, int d_ff) {
    // load addresses are 32-bit offsets from a tile's bases: token rows are
    // found anywhere in x (at most A rows of d), weight rows within a tile
    constexpr int64_t kOff = (int64_t)1 << 32;
    return d >= kWideP * kWideKStep && d_ff >= kWideP * kWideKStep &&
           A * d * 2 < kOff && (int64_t)kWideBW * std::max(d, d_ff) * 2 < kOff;
}

hipError_t launch_wide_ffn(const void *act, const int32_t *gather, const int32_t *offsets,
                           const void *W1, const void *W3, const void *W2, int out_f32, int64_t A,
                           int d, int d_ff, int E, void *hbuf, void *out, float *partial,
                           size_t partial_bytes, hipEvent_t mid, hipStream_t s) {
    if (partial && partial_bytes < wide_partial_bytes(A, E)) partial = nullptr;  // no splits
    hipError_t err = launch_wide<true, bf16_t>(act, d, gather, W1, W3, offsets, E, d_ff, d, A,
                                               hbuf, partial, s, mid);
    if (err != hipSuccess) return err;
    if (out_f32)
        return launch_wide<false, float>(hbuf, d_ff, nullptr, W2, nullptr, offsets, E, d, d_ff,
                                         A, out, partial, s);
    return launch_wide<false, bf16_t>(hbuf, d_ff, nullptr, W2, nullptr, offsets, E, d, d_ff, A,
                                      out, partial, s);
}

hipError_t launch_wide_w2(const void *hbuf, const int32_t *offsets, const void *W2, int out_f32,
                          int64_t A, int d, int d_ff, int E, void *out, float *partial,
                          size_t partial_bytes, hipStream_t s) {
    if (partial && partial_bytes < wide_partial_bytes(A, E)) partial = nullptr;  // no splits
    if (out_f32)
        return launch_wide<false, float>(hbuf, d_ff, nullptr, W2, nullptr, offsets, E, d, d_ff,
                                         A, out, partial, s);
    return launch_wide<false, bf16_t>(hbuf, d_ff, nullptr, W2, nullptr, offsets, E, d, d_ff, A,
                                      out, partial, s);
}

}  // namespace moe
