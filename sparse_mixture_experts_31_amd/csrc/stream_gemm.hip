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
constexpr int kSPartHdr = 64;  // floats before the chunk slices (the chosen chunk count)
static_assert(kSLds <= 160 * 1024 - 1024, "LDS capacity");
static_assert(kSGrp == 16 && kSGroups == 8, "one 16-row MFMA fragment per stage, 8 per K range");
static_assert(kSP - 1 <= kSGroups / 2, "prologue stages carry no token loads");

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

// Byte offset of 16-byte chunk c of 1 KiB row r in a buffer of such rows.
__device__ __forceinline__ int swz1k(int r, int c) { return r * 1024 + ((c ^ (r & 15)) << 4); }

}  // namespace

template <bool SWIGLU, typename TO>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void stream_gemm_kernel(
    const bf16_t *__restrict__ act, int64_t act_ld, const int32_t *__restrict__ gather,
    const bf16_t *__restrict__ Wa, const bf16_t *__restrict__ Wb,
    const int32_t *__restrict__ offsets, int E, int N, int K, int A, TO *__restrict__ out,
    int kc_max, float *__restrict__ part) {
    constexpr int P = kSP, G = kSGroups;
    constexpr int kCols = SWIGLU ? kSRowsT / 2 : kSRowsT;  // output columns per tile
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    char *const wring = smem;
    char *const tbuf = smem + P * kSWStage;
    int32_t *const s_map = (int32_t *)(smem + P * kSWStage + 2 * kSTokBuf);
    __shared__ int s_lo[64], s_cnt[64], s_first[65];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    // wave-uniform by construction; saying so keeps the load bases scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int col_tiles = (N + kCols - 1) / kCols;
    const int n_kr = K / kSKRange;  // >= 1, checked by the launcher

    // Per-expert tile table (token tiles fastest, then column tiles) by wave
    // 0; meanwhile the other three copy the token map, four loads in flight
    // per lane, so the whole set-up is about one memory round trip.
    if (wave == 0) {
        build_expert_table(offsets, E, A, kSBT, col_tiles, s_lo, s_cnt, s_first);
    } else if (gather) {
        constexpr int kStride = 256 - kWave;
        for (int i0 = tid - kWave; i0 < A; i0 += 4 * kStride) {
            int v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = i0 + q * kStride < A ? gather[i0 + q * kStride] : 0;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (i0 + q * kStride < A) s_map[i0 + q * kStride] = v[q];
        }
    }
    __syncthreads();
    auto u = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
    // Work items: tile t's K ranges cut into kc contiguous chunks; item
    // w = kc t + chunk, taken round robin.  With few tiles (small batches)
    // whole tiles leave CUs idle for much of the kernel: kc is then 4 when
    // that finishes at least 10 % sooner in units of whole tiles,
    // ceil(4 tiles / grid) / 4 against ceil(tiles / grid), else 1.  (Two
    // chunks measured slower than both one and four on MI355X -- by 10 %
    // at T = 8, where the count predicted a 7 % gain -- and the chunks'
    // partial sums and extra pass cost a few percent, hence the margin.)
    // The same choice in every workgroup, recorded for stream_reduce_kernel.
    const int NG = gridDim.x;
    const int tiles = u(s_first[E]);
    int kc = 1;
    if (kc_max >= 4 && n_kr >= 4 &&
        10 * (int64_t)((tiles * 4 + NG - 1) / NG) < 36 * (int64_t)((tiles + NG - 1) / NG))
        kc = 4;
    if (kc_max > 1 && blockIdx.x == 0 && tid == 0) *(int *)part = kc;
    float *const slices = part + kSPartHdr;
    const int total = tiles * kc;
    const int my_items = (total > (int)blockIdx.x) ? (total - (int)blockIdx.x + NG - 1) / NG : 0;
    if (my_items == 0) return;  // uniform over the workgroup

    struct Item {
        TileInfo ti;
        int kr0, kr1, chunk;  // K ranges [kr0, kr1) of the tile
    };
    auto item_info = [&](int k) {
        const int w = (int)blockIdx.x + k * NG;
        const int t = w / kc;
        Item it;
        it.chunk = w - t * kc;
        it.kr0 = it.chunk * n_kr / kc;
        it.kr1 = (it.chunk + 1) * n_kr / kc;
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
                // which alternate between two accumulators)
                if ((RG & 1) == par) {
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
        // K chunk of a tile (kc > 1) leaves its raw fp32 sums in its slice
        // of `part` for stream_reduce_kernel (GEMM1: u at column n, v at
        // column N + n of a 2N-wide row).
        const int m = 16 * jfrag + lr;
        if (m < cti.mrem) {
            const int64_t row = cti.row0 + m;
#pragma unroll
            for (int h = 0; h < (SWIGLU ? 2 : 4); ++h) {
                const int n = cti.n0 + 16 * (par + 2 * h) + 4 * lq;
                if (n < N) {
                    if (kc > 1) {
                        constexpr int W = SWIGLU ? 2 : 1;
                        float *sl = slices + ((int64_t)cit.chunk * A + row) * (W * N);
                        *(f32x4 *)(sl + n) = acc[h];
                        if constexpr (SWIGLU) *(f32x4 *)(sl + N + n) = acc[h + 2];
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
}

// The K chunks' partial sums added in chunk order (so the sum is the same
// on every run), then the epilogue: GEMM2 out[r][n] = sum_c o_c[r][n];
// GEMM1 out[r][n] = silu(sum_c u_c[r][n]) * sum_c v_c[r][n].  Nothing to do
// when the GEMM kernel chose one chunk.
template <bool SWIGLU, typename TO>
__global__ __launch_bounds__(256) void stream_reduce_kernel(const float *__restrict__ part,
                                                            int64_t A, int N,
                                                            TO *__restrict__ out) {
    const int kc = *(const int *)part;
    if (kc <= 1) return;
    const float *slices = part + kSPartHdr;
    constexpr int W = SWIGLU ? 2 : 1;
    const int64_t n4 = A * N / 4;               // N is a multiple of 512
    const int64_t slice = A * (int64_t)(W * N);  // floats per chunk
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * 256) {
        const int64_t r = (4 * i) / N, n = (4 * i) % N;
        const float *p = slices + r * (W * N) + n;
        f32x4 uu = *(const f32x4 *)p, vv = {};
        if constexpr (SWIGLU) vv = *(const f32x4 *)(p + N);
        for (int c = 1; c < kc; ++c) {
            uu += *(const f32x4 *)(p + c * slice);
            if constexpr (SWIGLU) vv += *(const f32x4 *)(p + c * slice + N);
        }
        float o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = SWIGLU ? silu(uu[q]) * vv[q] : uu[q];
        store4<TO>(out + 4 * i, o[0], o[1], o[2], o[3]);
    }
}

namespace {

// Most K chunks a launch may cut its tiles into: only at the smallest
// batches (fewer than four rows per expert on average), where the tile count
// can leave CUs idle.  The kernel picks the count it uses.
int stream_chunk_limit(int64_t A, int E) { return (A > 0 && A < 4 * (int64_t)E) ? 4 : 1; }

template <bool SWIGLU, typename TO>
hipError_t launch_stream(const void *act, int64_t act_ld, const int32_t *gather, const void *Wa,
                         const void *Wb, const int32_t *offsets, int E, int N, int K, int64_t A,
                         void *out, int kc_max, float *part, hipStream_t s) {
    hipError_t err = set_lds_limit<stream_gemm_kernel<SWIGLU, TO>>(kSLds);
    if (err != hipSuccess) return err;
    // one workgroup per CU, never more than there can be items:
    // sum_e ceil(c_e / BT) <= ceil(A / BT) + E - 1 tiles, kc_max items each
    const int64_t cols = SWIGLU ? kSRowsT / 2 : kSRowsT;
    const int64_t item_bound = (N + cols - 1) / cols * ((A + kSBT - 1) / kSBT + E - 1) * kc_max;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(device_cus(), item_bound));
    hipLaunchKernelGGL((stream_gemm_kernel<SWIGLU, TO>), dim3(grid), dim3(256), kSLds, s,
                       (const bf16_t *)act, act_ld, gather, (const bf16_t *)Wa,
                       (const bf16_t *)Wb, offsets, E, N, K, (int)A, (TO *)out, kc_max, part);
    if ((err = hipGetLastError()) != hipSuccess || kc_max == 1) return err;
    const int64_t n4 = A * N / 4;  // N is a multiple of 512
    const int rgrid = (int)std::max<int64_t>(1, std::min<int64_t>(1024, (n4 + 255) / 256));
    hipLaunchKernelGGL((stream_reduce_kernel<SWIGLU, TO>), dim3(rgrid), dim3(256), 0, s,
                       (const float *)part, A, N, (TO *)out);
    return hipGetLastError();
}

}  // namespace

size_t stream_partial_bytes(int64_t A, int d, int d_ff, int E) {
    // header + the larger of GEMM1's (u and v: 2 d_ff per row) and GEMM2's
    // (d per row) chunk slices; the two launches run one after the other
    const int kc = stream_chunk_limit(A, E);
    if (kc == 1) return 0;
    return sizeof(float) * ((size_t)kSPartHdr + (size_t)kc * A * std::max(2 * d_ff, d));
}

bool stream_supported(int64_t A, int d, int d_ff, int E) {
    // whole 1 KiB row pieces, and the token map fits its LDS area
    return d % kSKRange == 0 && d_ff % kSKRange == 0 && d >= kSKRange && d_ff >= kSKRange &&
           A <= kSMapMax && E <= 64;
}

hipError_t launch_stream_ffn(const void *act, const int32_t *gather, const int32_t *offsets,
                             const void *W1, const void *W3, const void *W2, int out_f32,
                             int64_t A, int d, int d_ff, int E, void *hbuf, void *out,
                             float *partial, size_t partial_bytes, hipEvent_t mid,
                             hipStream_t s) {
    // K chunks only when the scratch for their partial sums is there
    int kc = stream_chunk_limit(A, E);
    if (kc > 1 && (!partial || partial_bytes < stream_partial_bytes(A, d, d_ff, E))) kc = 1;
    hipError_t err = launch_stream<true, bf16_t>(act, d, gather, W1, W3, offsets, E, d_ff, d, A,
                                                 hbuf, kc, partial, s);
    if (err == hipSuccess && mid) err = hipEventRecord(mid, s);
    if (err != hipSuccess) return err;
    if (out_f32)
        return launch_stream<false, float>(hbuf, d_ff, nullptr, W2, nullptr, offsets, E, d, d_ff,
                                           A, out, kc, partial, s);
    return launch_stream<false, bf16_t>(hbuf, d_ff, nullptr, W2, nullptr, offsets, E, d, d_ff, A,
                                        out, kc, partial, s);
}

}  // namespace moe
