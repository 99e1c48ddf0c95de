// stream_gemm.hip — the expert GEMMs of decode-sized bf16 batches as one
// continuous weight stream.
//
// Same experts as expert_gemm.hip (the SwiGLU MLP W2 (silu(W1 x) * W3 x):
// fdeinterviews breakdown, "The paper in one minute"; tokentrails lineage,
// Code listing), but at decode sizes every expert holds only a few rows
// (about 8 at T = 32), so each weight byte feeds a handful of multiply-adds
// and the kernel is a read of the active experts' weights at the HBM rate.
// What it takes to stay near that rate on MI355X:
//  * few rows at a time, long pieces: HBM delivers 6.8-7.0 TB/s when a
//    workgroup streams 16 weight rows in 1 KiB pieces, against 5.6-5.9 TB/s
//    for 128-byte pieces of 128 rows (a probe of this ring's access
//    pattern); so a stage is 16 rows x 1 KiB, one row per global_load_lds;
//  * bytes in flight: one persistent workgroup per CU runs a 5-slot ring of
//    those stages (64 KiB of weights always on their way) across tile
//    boundaries, weight loads non-temporal (read once);
//  * tokens reused, not re-streamed: a tile is 128 weight rows x 32 token
//    rows walked as 512-wide K ranges, each K range as 8 stages of 16 rows
//    (row group minor), so the token rows of a K range (32 x 1 KiB) are
//    loaded once into one of two LDS buffers and read by all 8 stages.
//    They are loaded with the weight loads of the previous K range's last
//    four stages, when no stage still reads the buffer they go to.
//
// Per stage each wave issues its 4 of the 16 weight rows (and, in the
// second half of a K range, 2 of the next K range's token rows).  The load
// counts follow the row group, so the loop body is unrolled over the 8 row
// groups and every vmcnt wait is a compile-time constant.  A stage is
// computed by the two waves of its row-group parity, one 16-token fragment
// each, on v_mfma_f32_16x16x32_bf16: 16 MFMAs per stage per wave -- the
// matrix cores idle almost always, by design.  In LDS the 16-byte chunk c
// of a 1 KiB row r sits at chunk c ^ (r & 15), so the 16 rows of a fragment
// read hit 16 distinct bank groups, and every load instruction is still one
// contiguous row piece.
//
// Token rows are read in place (GEMM1 through `gather` = token_of): the map
// is copied to LDS at the start, so a token row's address is one LDS read,
// never a memory round trip in the middle of the ring.
#include "gemm_common.h"

namespace moe {

namespace {

constexpr int kSRowsT = 128;   // weight rows per tile (GEMM1: 64 of W1 + the same 64 of W3)
constexpr int kSBT = 32;       // token rows per tile
constexpr int kSGrp = 16;      // weight rows per stage
constexpr int kSGroups = kSRowsT / kSGrp;  // stages per K range
constexpr int kSKRange = 512;  // bf16 K elements per row piece (1 KiB)
constexpr int kSP = 5;         // weight stages in the ring
constexpr int kSWStage = kSGrp * 1024;
constexpr int kSTokBuf = kSBT * 1024;
constexpr int kSMapMax = 33 * 64;  // token_of entries: A < 33 E on this path, E <= 64
constexpr int kSLds = kSP * kSWStage + 2 * kSTokBuf + kSMapMax * 4;
constexpr int kSPartHdr = 64;  // header ints of `part`: [0] split taken, [1] the grid
constexpr int kSSlot = kSBT * kSRowsT;  // floats in a slot: one tile's 32 x 128 fp32 sums
static_assert(kSLds <= 160 * 1024 - 3 * 1024, "LDS capacity (3 KiB of static tables)");
static_assert(kSGrp == 16 && kSGroups == 8, "one 16-row MFMA fragment per stage, 8 per K range");
static_assert(kSP - 1 <= kSGroups / 2, "prologue stages carry no token loads");

// Four fp32 partial sums of a split tile's piece, as two 64-bit stores:
// written through to memory when another workgroup of the same launch will
// read them (agent-coherent), else plain.
__device__ __forceinline__ void put_piece(float *p, const f32x4 &v, bool coherent) {
    if (coherent) {
        uint64_t *q = (uint64_t *)p;
        __hip_atomic_store(q, ((uint64_t)__float_as_uint(v[1]) << 32) | __float_as_uint(v[0]),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(q + 1, ((uint64_t)__float_as_uint(v[3]) << 32) | __float_as_uint(v[2]),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        *(f32x4 *)p = v;
    }
}

// A piece written by another workgroup of this launch (agent-coherent loads).
__device__ __forceinline__ f32x4 get_piece(const float *p) {
    const uint64_t *q = (const uint64_t *)p;
    const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x4{__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)),
                 __uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32))};
}

// Loads a wave issues along with stage row group rg: 4 weight rows, and in
// the second half of a K range 2 token rows of the next one.
constexpr int loads_of(int rg) { return 4 + (rg >= kSGroups / 2 ? 2 : 0); }
// Loads that may still be in flight once stage rg's weights have landed:
// the token loads issued with them and all loads of the next P - 2 stages.
constexpr int vm_allow(int rg) {
    int n = loads_of(rg) - 4;
    for (int j = 1; j <= kSP - 2; ++j) n += loads_of((rg + j) % kSGroups);
    return n;
}
static_assert(vm_allow(4) < 64, "vmcnt range");

}  // namespace

template <bool SWIGLU, typename TO>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void stream_gemm_kernel(
    const bf16_t *__restrict__ act, int64_t act_ld, const int32_t *__restrict__ gather,
    const bf16_t *__restrict__ Wa, const bf16_t *__restrict__ Wb,
    const int32_t *__restrict__ offsets, int E, int N, int K, int A, TO *__restrict__ out,
    int max_pieces, float *__restrict__ part, const StreamFuse fz) {
    constexpr int P = kSP, G = kSGroups;
    constexpr int kCols = SWIGLU ? kSRowsT / 2 : kSRowsT;  // output columns per tile
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    char *const wring = smem;
    char *const tbuf = smem + P * kSWStage;
    int32_t *const s_map = (int32_t *)(smem + P * kSWStage + 2 * kSTokBuf);
    __shared__ int s_lo[64], s_cnt[64], s_first[65];
    __shared__ int s_goff[65], s_gbase[64], s_gwc[4][64];  // grouping (fz.topk_idx)
    // Stable grouping of the A assignments by expert, as the dispatch
    // kernel does it (dispatch.hip), by one workgroup: an LDS histogram and
    // its scan give every expert's first row; then 256 assignments a round,
    // a lane's rank among the lanes of its wave with the same expert (one
    // ballot per expert) plus the earlier waves' and rounds' counts give its
    // row, so rows inside an expert follow ascending assignment index.  The
    // experts are staged in `se` (the ring, idle until the prologue); the
    // map row -> token goes to `map`; workgroup 0 writes the grouping out.
    auto group_assignments = [&](const StreamFuse &f, int A_, int E_, int32_t *se, int32_t *map) {
        const int t = threadIdx.x, ln = t & (kWave - 1), wv = t / kWave;
        const bool writer = blockIdx.x == 0;
        for (int a = t; a < A_; a += 256) se[a] = f.topk_idx[a];
        if (t < 64) s_gbase[t] = 0;
        __syncthreads();
        for (int a = t; a < A_; a += 256) {
            const int e = se[a];
            if ((unsigned)e < (unsigned)E_) atomicAdd(&s_gbase[e], 1);
        }
        __syncthreads();
        if (wv == 0) {
            const int c = ln < E_ ? s_gbase[ln] : 0;
            int incl = c;
#pragma unroll
            for (int dd = 1; dd < kWave; dd <<= 1) {
                const int v = __shfl_up(incl, dd);
                if (ln >= dd) incl += v;
            }
            if (ln < E_) {
                s_goff[ln] = incl - c;
                s_gbase[ln] = incl - c;
                if (writer) {
                    f.counts[ln] = c;
                    f.offsets[ln] = incl - c;
                }
            }
            if (ln == E_ - 1) {
                s_goff[E_] = incl;
                if (writer) f.offsets[E_] = incl;
            }
        }
        __syncthreads();
        const uint64_t lower = (ln == 0) ? 0ull : (~0ull >> (64 - ln));
        for (int r0 = 0; r0 < A_; r0 += 256) {
            const int a = r0 + t;
            const int e = a < A_ ? se[a] : -1;
            const bool valid = (unsigned)e < (unsigned)E_;
            int rank = 0, cnt = 0;
            for (int ex = 0; ex < E_; ++ex) {
                const uint64_t m = __ballot(e == ex);
                if (e == ex) rank = __popcll(m & lower);
                if (ln == ex) cnt = __popcll(m);
            }
            s_gwc[wv][ln] = cnt;
            __syncthreads();
            if (valid) {
                int row = s_gbase[e] + rank;
                for (int w = 0; w < wv; ++w) row += s_gwc[w][e];
                map[row] = a / f.k;
                if (writer) {
                    f.row_of[a] = row;
                    f.token_of[row] = a / f.k;
                }
            } else if (writer && a < A_) {
                f.row_of[a] = -1;
            }
            __syncthreads();
            if (t < E_) s_gbase[t] += s_gwc[0][t] + s_gwc[1][t] + s_gwc[2][t] + s_gwc[3][t];
            __syncthreads();
        }
    };

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    // wave-uniform by construction; saying so keeps the load bases scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int col_tiles = (N + kCols - 1) / kCols;
    const int n_kr = K / kSKRange;  // >= 1, checked by the launcher

    // Per-expert tile table (token tiles fastest, then column tiles) by wave
    // 0; meanwhile the other three copy the token map, four loads in flight
    // per lane, so the whole set-up is about one memory round trip.  With
    // fz.topk_idx (GEMM1 of the decode layer) the workgroup first groups the
    // assignments itself and the table and map come from that.
    if (SWIGLU && fz.topk_idx) {
        group_assignments(fz, A, E, (int32_t *)wring, s_map);
        if (wave == 0) build_expert_table(s_goff, E, A, kSBT, col_tiles, s_lo, s_cnt, s_first);
    } else if (wave == 0) {
        build_expert_table(offsets, E, A, kSBT, col_tiles, s_lo, s_cnt, s_first);
    } else if (gather) {
        const int32_t *src = gather;
        constexpr int kStride = 256 - kWave;
        for (int i0 = tid - kWave; i0 < A; i0 += 4 * kStride) {
            int v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = i0 + q * kStride < A ? src[i0 + q * kStride] : 0;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (i0 + q * kStride < A) s_map[i0 + q * kStride] = v[q];
        }
    }
    __syncthreads();
    auto u = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
    // Work split.  Whole tiles, workgroup b taking the run of tiles
    // [b tiles / NG, (b + 1) tiles / NG) (a run of neighbouring column tiles
    // of one expert streams 3 % faster on MI355X than tiles dealt round
    // robin); or, where the launcher allows it (max_pieces > 1: scratch for the
    // partial sums is there) and whole tiles would leave CUs idle for much of
    // the kernel (few tiles, or a last round mostly empty), an even split of all
    // R = tiles x n_kr K ranges in tile order: workgroup b of the NGe used
    // walks ranges [b R / NGe, (b + 1) R / NGe), cut at tile boundaries into
    // items.  A tile's pieces (at most max_pieces: NGe is kept small enough that
    // every workgroup gets at least (n_kr - 1) / (max_pieces - 1) ranges) leave
    // fp32 partial sums, summed in K order by stream_reduce_kernel.  The
    // split is taken when it cuts the K ranges of the busiest workgroup by
    // at least 10 % (the partial sums and the extra pass cost a few
    // percent).  Every workgroup makes the same choice; it is recorded in
    // the header of `part` for the reduce pass.
    const int NG = gridDim.x;
    const int tiles = u(s_first[E]);
    const int64_t R = (int64_t)tiles * n_kr;
    bool split = false;
    int NGe = NG;
    if (max_pieces > 1 && tiles > 0) {
        const int s_need = n_kr > 1 ? (n_kr - 2) / (max_pieces - 1) + 1 : 1;
        NGe = (int)max<int64_t>(1, min<int64_t>(NG, R / s_need));
        const int64_t whole = (int64_t)((tiles + NG - 1) / NG) * n_kr;
        split = 10 * ((R + NGe - 1) / NGe) <= 9 * whole;
        if (!split) NGe = NG;
    }
    if (max_pieces > 1 && blockIdx.x == 0 && tid == 0) {
        ((int *)part)[0] = split ? 1 : 0;
        ((int *)part)[1] = NG;
    }
    // A piece of a split tile is always the first or the last item of its
    // workgroup (the items between are whole tiles), so the pieces go to two
    // slots per workgroup: slot 2 b for its first item, 2 b + 1 for its last.
    // info[r * col_tiles + c] describes the tile holding row r and column
    // tile c: r's row in the tile (bits 0-4), the tile's pieces (bits 5-8)
    // and the slot of its first piece (from bit 9); the next pieces are in
    // the first slots of the next workgroups.
    float *const slots = part + kSPartHdr;
    int32_t *const info = split ? (int32_t *)(slots + (int64_t)2 * NG * kSSlot) : nullptr;
    // (R < 2^31: tiles <= 33 x 224 x 64 experts, n_kr <= K / 512)
    const int g0 = split ? (int)((int64_t)blockIdx.x * R / NGe) : 0;
    const int g1 = split ? (int)(((int64_t)blockIdx.x + 1) * R / NGe) : 0;
    const int t_first = g0 / n_kr;
    int my_items = 0;
    if (split)
        my_items = ((int)blockIdx.x < NGe) ? (g1 - 1) / n_kr - t_first + 1 : 0;
    // Whole tiles: workgroup b runs on XCD b % 8, so the runs are numbered
    // XCD by XCD (bx) and each XCD's L2 holds one stretch of tiles, whose
    // token rows and expert are mostly shared, rather than every eighth run.
    const int bx = (NG % 8 == 0) ? ((int)blockIdx.x % 8) * (NG / 8) + (int)blockIdx.x / 8
                                 : (int)blockIdx.x;
    const int tw0 = (int)((int64_t)bx * tiles / NG);
    const int tw1 = (int)(((int64_t)bx + 1) * tiles / NG);
    if (!split)
        my_items = tw1 - tw0;
    if (my_items == 0) return;  // uniform over the workgroup
    // workgroup whose ranges hold global K range g
    auto wg_of = [&](int g) { return (int)((((int64_t)g + 1) * NGe - 1) / R); };

    struct Item {
        TileInfo ti;
        int kr0, kr1;  // K ranges [kr0, kr1) of the tile
        int t;         // the tile
    };
    auto item_info = [&](int k) {
        Item it;
        int t;
        if (split) {
            t = t_first + k;
            const int t0 = t * n_kr;
            it.kr0 = max(g0, t0) - t0;
            it.kr1 = min(g1, t0 + n_kr) - t0;
        } else {
            t = tw0 + k;
            it.kr0 = 0;
            it.kr1 = n_kr;
        }
        it.t = t;
        int i = 0;
        while (i + 1 < E && u(s_first[i + 1]) <= t) ++i;
        const int rem = t - u(s_first[i]);
        const int c = u(s_cnt[i]), l = u(s_lo[i]);
        const int mtiles = (c + kSBT - 1) / kSBT;
        TileInfo &ti = it.ti;
        ti.e = i;
        ti.mt = rem % mtiles;
        ti.row0 = l + ti.mt * kSBT;
        ti.mrem = min(kSBT, l + c - ti.row0);
        ti.n0 = (rem / mtiles) * kCols;
        return it;
    };
    // Weight row r of a tile (GEMM1: r < 64 rows of W1, else the same rows of
    // W3), clamped to the matrix.
    auto weight_row = [&](const TileInfo &ti, int r) -> const char * {
        const bf16_t *W = Wa;
        int nr = ti.n0 + r;
        if constexpr (SWIGLU) {
            W = (r < kSRowsT / 2) ? Wa : Wb;
            nr = ti.n0 + (r % (kSRowsT / 2));
        }
        nr = min(nr, N - 1);
        return (const char *)(W + ((int64_t)ti.e * N + nr) * K);
    };
    // Token rows of a tile, one per lane: lane j < 32 holds the address of
    // the tile's token row j (rows past the count repeat the last one), so a
    // load of row j takes it with one readlane.
    auto token_rows = [&](const TileInfo &ti) -> uint64_t {
        const int r = ti.row0 + min(lane & (kSBT - 1), ti.mrem - 1);
        const int row = gather ? s_map[r] : r;
        return (uint64_t)(act + (int64_t)row * act_ld);
    };
    auto token_row = [&](uint64_t rows, int j) -> const char * {
        return (const char *)(((uint64_t)__builtin_amdgcn_readlane((int)(rows >> 32), j) << 32) |
                              (uint32_t)__builtin_amdgcn_readlane((int)rows, j));
    };
    // One 1 KiB row piece of K range kr into LDS row dst (swizzle key `key`):
    // lane l fetches the chunk that belongs at LDS chunk l.
    auto piece = [&](const char *row, int kr, char *dst, int key, bool nt) {
        const char *src = row + (int64_t)kr * 1024 + ((lane ^ key) << 4);
        if (nt)
            dma16_nt(src, dst);
        else
            dma16(src, dst);
    };

    // ---- producer: runs P - 1 stages ahead; stage pq goes to slot pq % P.
    // (pk, pkr) are its tile and K range; past the last stage it keeps the
    // last addresses, reloading into slots nothing reads.
    // (pk, pkr): the producer's item and K range; pr counts the K ranges it
    // has entered (token buffer pr % 2).
    Item pit = item_info(0);
    Item pnext = my_items > 1 ? item_info(1) : pit;
    int pk = 0, pkr = pit.kr0, pr = 0;
    uint64_t prows = token_rows(pit.ti), pnext_rows = token_rows(pnext.ti);
    auto issue = [&](int pq, int rg) __attribute__((always_inline)) {
        char *slot = wring + (pq % P) * kSWStage;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * wave + i;  // row within the stage
            piece(weight_row(pit.ti, rg * kSGrp + r), pkr, slot + r * 1024, r, true);
        }
        if (rg >= G / 2) {
            // token rows of the next K range (this item's, or the next
            // item's first) into the other buffer
            const bool last = (pkr + 1 == pit.kr1);
            const uint64_t rows = last ? pnext_rows : prows;
            const int nkr = last ? pnext.kr0 : pkr + 1;
            char *tb = tbuf + ((pr + 1) & 1) * kSTokBuf;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int j = 8 * (rg - G / 2) + 2 * wave + i;
                piece(token_row(rows, j), nkr, tb + j * 1024, j & 15, false);
            }
        }
    };
    // after the loads of a row group G - 1 stage: the next K range (past
    // the last one the producer stays, reloading it into slots nothing reads)
    auto next_range = [&]() __attribute__((always_inline)) {
        if (pkr + 1 < pit.kr1) {
            ++pkr;
            ++pr;
        } else if (pk + 1 < my_items) {
            ++pk;
            ++pr;
            pit = pnext;
            pkr = pit.kr0;
            prows = pnext_rows;
            pnext = (pk + 1 < my_items) ? item_info(pk + 1) : pit;
            pnext_rows = token_rows(pnext.ti);
        }
    };

    // prologue: the first K range's token rows, then stages 0 .. P - 2
#pragma unroll
    for (int i = 0; i < kSBT / 4; ++i) {
        const int j = 8 * wave + i;
        piece(token_row(prows, j), pit.kr0, tbuf + j * 1024, j & 15, false);
    }
    static_assert(P - 1 < G, "the prologue stays in the first K range");
#pragma unroll
    for (int q = 0; q < P - 1; ++q) issue(q, q);
    int pq = P - 1;  // next stage the producer loads

    // ---- consumer ----
    const int par = wave >> 1, jfrag = wave & 1;  // row-group parity, token fragment
    const int lr = lane & 15, lq = lane >> 4;
    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{};

    int cr = 0;  // K ranges consumed (token buffer cr % 2, ring stage G cr + rg)
    for (int ck = 0; ck < my_items; ++ck) {
        const Item cit = item_info(ck);
        const TileInfo &cti = cit.ti;
        for (int ckr = cit.kr0; ckr < cit.kr1; ++ckr, ++cr) {
            const char *tb = tbuf + (cr & 1) * kSTokBuf;
            const int s0 = cr * G;
            // the G stages of one K range, unrolled: every wait is a constant
            auto stage = [&](auto rgc) __attribute__((always_inline)) {
                constexpr int RG = decltype(rgc)::value;
                constexpr int QRG = (RG + P - 1) % G;  // row group of the stage loaded now
                // stage s0 + RG landed (this wave's loads, then everyone's),
                // and every wave is done with the slot of the previous stage
                wait_vmcnt_lgkm0<vm_allow(RG)>();
                stage_barrier();
                issue(pq, QRG);
                if (QRG == G - 1) next_range();
                ++pq;
                // the two waves of this row group's parity, one token fragment
                // each (the fragment reads run RD k-steps ahead of the MFMAs,
                // which alternate between two accumulators); a fragment past
                // the tile's rows would only multiply padding, so its wave
                // skips the reads and MFMAs (its outputs are never stored)
                if ((RG & 1) == par && 16 * jfrag < cti.mrem) {
                    constexpr int NT = kSKRange / 32, RD = 3;
                    const char *wslot = wring + ((s0 + RG) % P) * kSWStage;
                    i32x4 w[NT], x[NT];
                    auto rd = [&](int t) __attribute__((always_inline)) {
                        const int c = 4 * t + lq;
                        w[t] = *(const i32x4 *)(wslot + swz1k(lr, c));
                        x[t] = *(const i32x4 *)(tb + swz1k(16 * jfrag + lr, c));
                    };
#pragma unroll
                    for (int t = 0; t < RD; ++t) rd(t);
                    f32x4 ab[2] = {acc[RG >> 1], f32x4{}};
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        if (t + RD < NT) rd(t + RD);
                        ab[t & 1] = mma16(w[t], x[t], ab[t & 1]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    acc[RG >> 1] = ab[0] + ab[1];
                }
            };
            stage(std::integral_constant<int, 0>{});
            stage(std::integral_constant<int, 1>{});
            stage(std::integral_constant<int, 2>{});
            stage(std::integral_constant<int, 3>{});
            stage(std::integral_constant<int, 4>{});
            stage(std::integral_constant<int, 5>{});
            stage(std::integral_constant<int, 6>{});
            stage(std::integral_constant<int, 7>{});
        }

        // Epilogue of the item.  Wave (par, jfrag) holds row groups par + 2 h
        // (h = 0..3) for tokens 16 jfrag .. + 16: lane l has weight rows
        // 4 (l / 16) .. + 4 of a group, for token l % 16.  GEMM1: groups
        // par, par + 2 are W1 rows, par + 4, par + 6 the same W3 rows.  A
        // piece of a split tile leaves its raw fp32 sums in its slot for
        // stream_reduce_kernel (GEMM1: u at column c of the tile, v at
        // 64 + c); the workgroup of a tile's first piece describes the tile
        // in `info` for each of its rows.
        const int m = 16 * jfrag + lr;
        if (m < cti.mrem) {
            const int64_t row = cti.row0 + m;
            int first = (int)blockIdx.x, np = 1;  // the tile's first workgroup and pieces
            if (split) {
                first = wg_of(cit.t * n_kr);
                np = wg_of(cit.t * n_kr + n_kr - 1) - first + 1;
            }
            const int slot = 2 * (int)blockIdx.x + (ck == 0 ? 0 : 1);
            if (split && !fz.ctr && first == (int)blockIdx.x && par == 0 && lq == 0)
                info[row * col_tiles + cti.n0 / kCols] = m | (np << 5) | (slot << 9);
#pragma unroll
            for (int h = 0; h < (SWIGLU ? 2 : 4); ++h) {
                const int c = 16 * (par + 2 * h) + 4 * lq;  // column in the tile
                const int n = cti.n0 + c;
                if (n < N) {
                    if (np > 1) {
                        float *sl = slots + (int64_t)slot * kSSlot + m * kSRowsT + c;
                        put_piece(sl, acc[h], fz.ctr != nullptr);
                        if constexpr (SWIGLU)
                            put_piece(sl + kSRowsT / 2, acc[h + 2], fz.ctr != nullptr);
                    } else {
                        float r[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            r[q] = acc[h][q];
                            if constexpr (SWIGLU) r[q] = silu(r[q]) * acc[h + 2][q];
                        }
                        store4<TO>(out + row * N + n, r[0], r[1], r[2], r[3]);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = f32x4{};
    }
    wait_vmcnt_lgkm0<0>();  // the trailing reloads land before the wave ends

    // With counters (the layer's GEMM1) the kernel finishes its split tiles
    // itself.  Only a workgroup's first and last items can be pieces; once
    // every wave's stores are done (the wait above) it counts each of them
    // on its tile, and the workgroup that completes a tile's count adds the
    // pieces in K order and applies the epilogue, as stream_reduce_kernel
    // does (the same sums in the same order).  The pieces were written
    // through to memory and are read with agent-coherent loads: no cache
    // flush or invalidation, which would stall the XCD's workgroups still
    // streaming.
    if (split && fz.ctr) {
        __shared__ int s_last;
        constexpr int kC4 = kCols / 4;
        for (int j = 0; j < 2 && j < my_items; ++j) {
            const Item it = item_info(j == 0 ? 0 : my_items - 1);
            const int first = wg_of(it.t * n_kr);
            const int np = wg_of(it.t * n_kr + n_kr - 1) - first + 1;
            if (np <= 1) continue;  // a whole tile, stored above
            __syncthreads();        // s_last of the previous tile has been read
            if (tid == 0)
                s_last = __hip_atomic_fetch_add(&fz.ctr[it.t], 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT) == np - 1;
            __syncthreads();
            if (!s_last) continue;
            // piece 0 is workgroup `first`'s last item, or its first if the
            // tile is where its ranges start; piece p > 0 is the first item
            // of workgroup first + p
            const int t_of_first = (int)(((int64_t)first * R / NGe) / n_kr);
            const int s0 = 2 * first + (t_of_first == it.t ? 0 : 1);
            for (int q = tid; q < kSBT * kC4; q += 256) {
                const int m = q / kC4, c = (q - m * kC4) * 4;
                const int n = it.ti.n0 + c;
                if (m >= it.ti.mrem || n >= N) continue;
                const float *p0 = slots + (int64_t)s0 * kSSlot + m * kSRowsT + c;
                f32x4 uu = get_piece(p0), vv = {};
                if constexpr (SWIGLU) vv = get_piece(p0 + kSRowsT / 2);
                for (int pc = 1; pc < np; ++pc) {
                    const float *pq = slots + (int64_t)(2 * (first + pc)) * kSSlot + m * kSRowsT + c;
                    uu += get_piece(pq);
                    if constexpr (SWIGLU) vv += get_piece(pq + kSRowsT / 2);
                }
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = SWIGLU ? silu(uu[i]) * vv[i] : uu[i];
                store4<TO>(out + (int64_t)(it.ti.row0 + m) * N + n, o[0], o[1], o[2], o[3]);
            }
        }
    }
}

// The pieces of split tiles added in K order (so the sum is the same on
// every run), then the epilogue: GEMM2 out[r][n] = sum_p o_p[r][n]; GEMM1
// out[r][n] = silu(sum_p u_p[r][n]) * sum_p v_p[r][n].  Nothing to do when
// the GEMM kernel kept whole tiles, or for the rows of tiles it did not
// split (it stored those itself).  Only the rows the experts own,
// [offsets[0], offsets[E]) clamped to [0, A) as the tile table clamps them,
// are looked at: rows outside belong to no tile.
template <bool SWIGLU, typename TO>
__global__ __launch_bounds__(256) void stream_reduce_kernel(const float *__restrict__ part,
                                                            const int32_t *__restrict__ offsets,
                                                            int E, int64_t A, int N,
                                                            TO *__restrict__ out) {
    const int *hdr = (const int *)part;
    if (hdr[0] == 0) return;
    const float *slots = part + kSPartHdr;
    constexpr int kCols = SWIGLU ? kSRowsT / 2 : kSRowsT;  // output columns per tile
    const int col_tiles = (N + kCols - 1) / kCols;
    const int32_t *info = (const int32_t *)(slots + (int64_t)2 * hdr[1] * kSSlot);
    const int64_t lo = min<int64_t>(max(offsets[0], 0), A);
    const int64_t hi = min<int64_t>(max<int64_t>(offsets[E], lo), A);
    const int64_t n4 = hi * N / 4;  // N is a multiple of 512
    for (int64_t i = lo * N / 4 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * 256) {
        const int64_t r = (4 * i) / N, n = (4 * i) % N;
        const int v = info[r * col_tiles + n / kCols];
        const int np = (v >> 5) & 15;
        if (np <= 1) continue;  // a whole tile: stored by the GEMM kernel
        const int m = v & 31, s0 = v >> 9, c = (int)(n % kCols);
        const float *p = slots + (int64_t)s0 * kSSlot + m * kSRowsT + c;
        f32x4 uu = *(const f32x4 *)p, vv = {};
        if constexpr (SWIGLU) vv = *(const f32x4 *)(p + kSRowsT / 2);
        for (int q = 1; q < np; ++q) {
            // piece q: the first slot of workgroup s0 / 2 + q
            const float *pq = slots + (int64_t)(2 * (s0 / 2 + q)) * kSSlot + m * kSRowsT + c;
            uu += *(const f32x4 *)pq;
            if constexpr (SWIGLU) vv += *(const f32x4 *)(pq + kSRowsT / 2);
        }
        float o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = SWIGLU ? silu(uu[q]) * vv[q] : uu[q];
        store4<TO>(out + 4 * i, o[0], o[1], o[2], o[3]);
    }
}

// GEMM2 of the decode layer where its tiles may be split: its expert
// outputs (the pieces' sums as stream_reduce_kernel forms them for split
// tiles, `o` itself for the others) go straight into the combine, y[t] =
// residual[t] + sum_j g_j o[row_of[t][j]] with one fused multiply-add per
// slot in slot order, as combine_kernel forms it, rounded once to bf16.
__global__ __launch_bounds__(256) void stream_reduce_combine_kernel(
    const float *__restrict__ part, const float *__restrict__ o,
    const int32_t *__restrict__ row_of, const float *__restrict__ gw,
    const bf16_t *__restrict__ residual, int64_t T, int k, int N, bf16_t *__restrict__ y) {
    const int *hdr = (const int *)part;
    const bool split = hdr[0] != 0;
    const float *slots = part + kSPartHdr;
    const int col_tiles = (N + kSRowsT - 1) / kSRowsT;
    const int32_t *info = (const int32_t *)(slots + (int64_t)2 * hdr[1] * kSSlot);
    const int n8 = N / 8;  // N is a multiple of 512
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < T * n8;
         i += (int64_t)gridDim.x * 256) {
        const int64_t t = i / n8;
        const int n = (int)(i - t * n8) * 8;
        float acc[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = 0.f;
        for (int j = 0; j < k; ++j) {
            const int r = row_of[t * k + j];
            if (r < 0) continue;
            const float g = gw[t * k + j];
            const int v = split ? info[(int64_t)r * col_tiles + n / kSRowsT] : 0;
            const int np = (v >> 5) & 15;
            f32x4 a, b;
            if (np <= 1) {
                const float *p = o + (int64_t)r * N + n;
                a = *(const f32x4 *)p;
                b = *(const f32x4 *)(p + 4);
            } else {
                const int m = v & 31, s0 = v >> 9, c0 = n % kSRowsT;
                const float *p = slots + (int64_t)s0 * kSSlot + m * kSRowsT + c0;
                a = *(const f32x4 *)p;
                b = *(const f32x4 *)(p + 4);
                for (int q = 1; q < np; ++q) {
                    const float *pq =
                        slots + (int64_t)(2 * (s0 / 2 + q)) * kSSlot + m * kSRowsT + c0;
                    a += *(const f32x4 *)pq;
                    b += *(const f32x4 *)(pq + 4);
                }
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc[c] = fmaf(g, a[c], acc[c]);
                acc[4 + c] = fmaf(g, b[c], acc[4 + c]);
            }
        }
        if (residual) {
            const uint4 rv = *(const uint4 *)(residual + t * N + n);
            const uint32_t w4[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += bf16_bits_to_f32(w4[q] & 0xffffu);
                acc[2 * q + 1] += bf16_bits_to_f32(w4[q] >> 16);
            }
        }
        *(uint4 *)(y + t * N + n) =
            make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                       pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    }
}

namespace {

// Most pieces a tile may be split into (the kernel decides whether to split).
constexpr int kSMaxPieces = 8;

// `reduce`: also launch the pass that sums split tiles' pieces (the decode
// layer's GEMM1 sums them itself, with counters, and its GEMM2 leaves that
// to stream_reduce_combine_kernel).  `after`, if set, is recorded right
// after the GEMM kernel, before that pass.
template <bool SWIGLU, typename TO>
hipError_t launch_stream(const void *act, int64_t act_ld, const int32_t *gather, const void *Wa,
                         const void *Wb, const int32_t *offsets, int E, int N, int K, int64_t A,
                         void *out, int max_pieces, float *part, hipStream_t s,
                         const StreamFuse &fz = StreamFuse{}, bool reduce = true,
                         hipEvent_t after = nullptr) {
    hipError_t err = set_lds_limit<stream_gemm_kernel<SWIGLU, TO>>(kSLds);
    if (err != hipSuccess) return err;
    // one workgroup per CU, never more than there can be items:
    // sum_e ceil(c_e / BT) <= ceil(A / BT) + E - 1 tiles, max_pieces items each
    const int64_t cols = SWIGLU ? kSRowsT / 2 : kSRowsT;
    const int64_t item_bound = (N + cols - 1) / cols * ((A + kSBT - 1) / kSBT + E - 1) * max_pieces;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(device_cus(), item_bound));
    hipLaunchKernelGGL((stream_gemm_kernel<SWIGLU, TO>), dim3(grid), dim3(256), kSLds, s,
                       (const bf16_t *)act, act_ld, gather, (const bf16_t *)Wa,
                       (const bf16_t *)Wb, offsets, E, N, K, (int)A, (TO *)out, max_pieces, part, fz);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (after && (err = hipEventRecord(after, s)) != hipSuccess) return err;
    if (max_pieces == 1 || !reduce) return err;
    const int64_t n4 = A * N / 4;  // N is a multiple of 512
    const int rgrid = (int)std::max<int64_t>(1, std::min<int64_t>(1024, (n4 + 255) / 256));
    hipLaunchKernelGGL((stream_reduce_kernel<SWIGLU, TO>), dim3(rgrid), dim3(256), 0, s,
                       (const float *)part, offsets, E, A, N, (TO *)out);
    return hipGetLastError();
}

}  // namespace

// GEMM1's tiles at most (one counter each when the layer's GEMM1 finishes its
// own split tiles): ceil(c_e / BT) token tiles per expert sum to at most
// ceil(A / BT) + E - 1.
int64_t stream_gemm1_tiles_max(int64_t A, int d_ff, int E) {
    const int64_t cols = (d_ff + kSRowsT / 2 - 1) / (kSRowsT / 2);
    return cols * ((std::max<int64_t>(A, 0) + kSBT - 1) / kSBT + E - 1);
}

// int32 index in the split scratch where those counters start: past the
// header, two slots per workgroup (at most one per CU) and the tile
// description per row and column tile (the larger of GEMM1's and GEMM2's;
// the two launches run one after the other).
int64_t stream_counter_index(int64_t A, int d, int d_ff) {
    const int64_t col_tiles = std::max((d_ff + kSRowsT / 2 - 1) / (kSRowsT / 2),
                                       (d + kSRowsT - 1) / kSRowsT);
    return (int64_t)kSPartHdr + (int64_t)2 * device_cus() * kSSlot +
           std::max<int64_t>(A, 0) * col_tiles;
}

size_t stream_partial_bytes(int64_t A, int d, int d_ff, int E) {
    return sizeof(int32_t) *
           (size_t)(stream_counter_index(A, d, d_ff) + stream_gemm1_tiles_max(A, d_ff, E));
}

bool stream_supported(int64_t A, int d, int d_ff, int E) {
    // whole 1 KiB row pieces, and the token map fits its LDS area
    return d % kSKRange == 0 && d_ff % kSKRange == 0 && d >= kSKRange && d_ff >= kSKRange &&
           A <= kSMapMax && E <= 64;
}


hipError_t launch_stream_fused(const void *x, const void *W1, const void *W3, const void *W2,
                               int64_t A, int d, int d_ff, int E, void *hbuf, float *out,
                               float *partial, size_t partial_bytes, const StreamFuse &fuse,
                               hipEvent_t gemm1_done, hipStream_t s) {
    if (!fuse.y) return hipErrorInvalidValue;
    // one to eight tokens: each workgroup streams its own columns of every
    // active expert (stream_cols.hip), no split tiles, GEMM2 forms y
    if (stream_cols_supported(fuse.T, fuse.k, d, d_ff, E))
        return launch_stream_cols(x, W1, W3, W2, fuse.T, d, d_ff, E, hbuf, fuse, gemm1_done, s);
    // The tile kernels may always split: each launch takes the even K split
    // when it cuts its busiest workgroup's K ranges by 10 % (few tiles, or a
    // round a few tiles past the CUs when an expert needs a second token
    // tile), and the pass after GEMM2 forms y from the pieces or the whole
    // tiles' outputs.
    if (!partial || partial_bytes < stream_partial_bytes(A, d, d_ff, E)) return hipErrorInvalidValue;
    // nine to 32 tokens: GEMM2 on the column kernel, which forms y itself
    const bool w2_cols = stream_cols_w2_supported(fuse.T, fuse.k, d, d_ff, E);
    // GEMM1 reads token rows through the map it builds
    StreamFuse f1 = fuse;
    f1.gw = nullptr;
    f1.residual = nullptr;
    f1.y = nullptr;
    // with counters GEMM1 finishes its split tiles itself (no pass after it)
    hipError_t err = launch_stream<true, bf16_t>(x, d, fuse.token_of, W1, W3, fuse.offsets, E,
                                                 d_ff, d, A, hbuf, kSMaxPieces, partial, s, f1,
                                                 fuse.ctr == nullptr, gemm1_done);
    if (err != hipSuccess) return err;
    if (w2_cols) return launch_stream_cols_w2(hbuf, W2, fuse.T, d, d_ff, E, fuse, s);
    err = launch_stream<false, float>(hbuf, d_ff, nullptr, W2, nullptr, fuse.offsets, E, d, d_ff,
                                      A, out, kSMaxPieces, partial, s, StreamFuse{}, false);
    if (err != hipSuccess) return err;
    const int64_t T = fuse.T, n8 = T * d / 8;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(1024, (n8 + 255) / 256));
    hipLaunchKernelGGL(stream_reduce_combine_kernel, dim3(grid), dim3(256), 0, s,
                       (const float *)partial, (const float *)out, fuse.row_of, fuse.gw,
                       fuse.residual, T, fuse.k, d, fuse.y);
    return hipGetLastError();
}

hipError_t launch_stream_ffn(const void *act, const int32_t *gather, const int32_t *offsets,
                             const void *W1, const void *W3, const void *W2, int out_f32,
                             int64_t A, int d, int d_ff, int E, void *hbuf, void *out,
                             float *partial, size_t partial_bytes, hipEvent_t mid,
                             hipStream_t s) {
    // split tiles only when the scratch for their partial sums is there
    int pieces = kSMaxPieces;
    if (!partial || partial_bytes < stream_partial_bytes(A, d, d_ff, E)) pieces = 1;
    hipError_t err = launch_stream<true, bf16_t>(act, d, gather, W1, W3, offsets, E, d_ff, d, A,
                                                 hbuf, pieces, partial, s, StreamFuse{}, true,
                                                 mid);
    if (err != hipSuccess) return err;
    if (out_f32)
        return launch_stream<false, float>(hbuf, d_ff, nullptr, W2, nullptr, offsets, E, d, d_ff,
                                           A, out, pieces, partial, s);
    return launch_stream<false, bf16_t>(hbuf, d_ff, nullptr, W2, nullptr, offsets, E, d, d_ff, A,
                                        out, pieces, partial, s);
}

}  // namespace moe
