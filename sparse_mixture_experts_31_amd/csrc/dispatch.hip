// dispatch.hip — group the T*k (token, slot) assignments by expert.
//
// Tokens go to the experts they chose, experts can receive none, and an
// expert with a zero gate is skipped entirely (tokentrails lineage, step
// "Two experts per token"; flashpapers summary, "How It Works").  Grouping the
// assignments per expert turns the experts into one grouped GEMM over
// contiguous row blocks.
//
// dispatch_index_kernel (one workgroup of 1024 threads):
//   1. per-expert histogram with LDS integer atomics (order-free, exact);
//   2. exclusive scan of the E counts -> offsets;
//   3. stable ranks, 1024 assignments per round: inside a wave the lanes that
//      share an expert are found with ballots (one per expert), a lane's rank
//      is the popcount of the matching lower lanes, and per-wave totals are
//      prefix-summed across the 16 waves and carried into the next round.
//      The indices are staged in LDS 8192 at a time (eight loads in flight
//      per thread), so a window costs one memory round trip instead of one
//      per round.  Rows inside an expert's block thus follow ascending
//      assignment index (t*k + j): a unique, deterministic order.
// Above 4096 assignments two launches that spread over the chip take over:
// the single workgroup walks the assignments 1024 at a time, about 1.5 us a
// round on MI355X (94 us for 32768), while the two launches take 9-11 us of
// kernel time from 4096 to 32768 assignments.
// The two launches:
// dispatch_chunk_rank_kernel: one wave per chunk of W consecutive
//   assignments; lane e keeps expert e's running count inside the chunk, and
//   64 assignments at a time one ballot per expert gives a lane its rank
//   among the chunk's earlier assignments of the same expert.  The rank goes
//   to row_of (a provisional value), the chunk's E counts to `cnt`.
// dispatch_place_kernel: every workgroup sums the chunk counts (the totals
//   give counts and offsets, which workgroup 0 writes; the chunks before its
//   own give its first row per expert), then each wave turns its chunk's
//   ranks into rows.  Chunks are in assignment order, so the rows are the
//   same stable grouping as above.
// gather_rows_kernel: one wave per token reads the token's row once with
//   16-byte loads and writes it to each of its k rows of x_perm.
#include <algorithm>

#include "common.h"

namespace moe {

constexpr int kDispatchThreads = 1024;
constexpr int kDispatchWaves = kDispatchThreads / kWave;
constexpr int kDispatchWindow = 8192;  // indices staged in LDS at a time
constexpr int64_t kDispatchChunkedFrom = 4096;  // larger batches: the two-launch form

// Workgroup barrier for LDS traffic only.  __syncthreads() also waits for
// every global store of the wave to complete, which here would stall each
// round on the previous round's row_of / token_of stores; nothing in this
// kernel reads those back.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS operations are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kDispatchThreads) void dispatch_index_kernel(
    const int32_t *__restrict__ idx, int A, int E, int k, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ row_of, int32_t *__restrict__ token_of) {
    __shared__ int s_cnt[64];
    __shared__ int s_base[64];
    __shared__ int s_wave[kDispatchWaves][64];
    __shared__ int s_idx[kDispatchWindow];  // the assignments' experts, a window at a time
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    if (tid < 64) s_cnt[tid] = 0;
    lds_barrier();
    // A window of the indices (kPer loads in flight per thread) into s_idx.
    constexpr int kPer = kDispatchWindow / kDispatchThreads;
    auto stage = [&](int w0) {
        int v[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int a = w0 + q * kDispatchThreads + tid;
            v[q] = (a < A) ? idx[a] : -1;
        }
#pragma unroll
        for (int q = 0; q < kPer; ++q) s_idx[q * kDispatchThreads + tid] = v[q];
    };
    // histogram, window by window (the first window stays staged)
    for (int w0 = 0; w0 < A; w0 += kDispatchWindow) {
        stage(w0);
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int e = s_idx[q * kDispatchThreads + tid];  // this thread's own entry
            if ((unsigned)e < (unsigned)E) atomicAdd(&s_cnt[e], 1);
        }
    }
    lds_barrier();
    if (tid == 0) {
        int run = 0;
        for (int e = 0; e < E; ++e) {
            s_base[e] = run;
            offsets[e] = run;
            counts[e] = s_cnt[e];
            run += s_cnt[e];
        }
        offsets[E] = run;
    }
    lds_barrier();

    const uint64_t lower_lanes = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int r0 = 0; r0 < A; r0 += kDispatchThreads) {
        // a new window (the histogram left the last one staged); every
        // thread reads only the entries it stored itself
        if (r0 % kDispatchWindow == 0 && (r0 > 0 || A > kDispatchWindow)) stage(r0);
        const int a = r0 + tid;
        const int e = s_idx[r0 % kDispatchWindow + tid];
        const bool valid = (unsigned)e < (unsigned)E;
        // one ballot per expert (independent of each other, so they
        // pipeline): a lane's rank among the lanes of its expert, and lane
        // ex of the wave keeps expert ex's count
        int rank = 0, cnt = 0;
        for (int ex = 0; ex < E; ++ex) {
            const uint64_t m = __ballot(e == ex);
            if (e == ex) rank = __popcll(m & lower_lanes);
            if (lane == ex) cnt = __popcll(m);
        }
        s_wave[wave][lane] = cnt;
        lds_barrier();
        // per expert, the waves' counts to first rows: thread 16 e + w holds
        // wave w's count, and the 16 of an expert share a wave (a segmented
        // shuffle scan instead of a loop over the waves)
        static_assert(kDispatchWaves == 16, "one 16-lane segment per expert");
        if (tid < kDispatchWaves * E) {
            const int ex = tid / kDispatchWaves, w = tid % kDispatchWaves;
            const int c = s_wave[w][ex];
            int incl = c;
#pragma unroll
            for (int dd = 1; dd < kDispatchWaves; dd <<= 1) {
                const int v = __shfl_up(incl, dd, kDispatchWaves);
                if (w >= dd) incl += v;
            }
            const int base = s_base[ex];
            s_wave[w][ex] = base + incl - c;
            if (w == kDispatchWaves - 1) s_base[ex] = base + incl;
        }
        lds_barrier();
        if (valid) {
            const int row = s_wave[wave][e] + rank;
            row_of[a] = row;
            token_of[row] = a / k;
        } else if (a < A) {
            row_of[a] = -1;
        }
        lds_barrier();
    }
}

constexpr int kChunkWaves = 4;   // chunks (one wave each) per workgroup
constexpr int kChunkBatch = 4;   // index loads in flight per lane

__global__ __launch_bounds__(kChunkWaves * kWave) void dispatch_chunk_rank_kernel(
    const int32_t *__restrict__ idx, int A, int E, int W, int nch, int32_t *__restrict__ row_of,
    int32_t *__restrict__ cnt) {
    const int lane = threadIdx.x & (kWave - 1);
    const int ch = blockIdx.x * kChunkWaves + (int)threadIdx.x / kWave;
    if (ch >= nch) return;  // uniform over the wave
    const int64_t a0 = (int64_t)ch * W, a1 = min((int64_t)A, a0 + W);
    const uint64_t lower_lanes = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int run = 0;  // lane e: assignments of expert e so far in this chunk
    for (int64_t b = a0; b < a1; b += kChunkBatch * kWave) {
        int ev[kChunkBatch];
#pragma unroll
        for (int q = 0; q < kChunkBatch; ++q) {
            const int64_t a = b + q * kWave + lane;
            ev[q] = (a < a1) ? idx[a] : -1;
        }
#pragma unroll
        for (int q = 0; q < kChunkBatch; ++q) {
            const int64_t a = b + q * kWave + lane;
            const int e = ev[q];
            const bool valid = (unsigned)e < (unsigned)E;
            const int before = __shfl(run, valid ? e : 0);
            int rank = 0;
            for (int ex = 0; ex < E; ++ex) {
                const uint64_t m = __ballot(e == ex);
                if (e == ex) rank = __popcll(m & lower_lanes);
                if (lane == ex) run += __popcll(m);
            }
            if (a < a1) row_of[a] = valid ? before + rank : -1;
        }
    }
    if (lane < E) cnt[(int64_t)ch * E + lane] = run;
}

__global__ __launch_bounds__(kChunkWaves * kWave) void dispatch_place_kernel(
    const int32_t *__restrict__ idx, int A, int E, int k, int W, int nch,
    const int32_t *__restrict__ cnt, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ row_of, int32_t *__restrict__ token_of) {
    __shared__ int s_tot[kChunkWaves * kWave], s_pre[kChunkWaves * kWave];
    __shared__ int s_first[64];  // first row of expert e for this workgroup's first chunk
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int ch0 = blockIdx.x * kChunkWaves;
    // Sums over the chunk counts: lane l takes expert l % E of the chunks
    // j, j + J, ... with j = wave * G + l / E (G lane groups per wave).
    const int G = kWave / E, J = kChunkWaves * G;
    int tot = 0, pre = 0;
    if (lane < G * E) {
        const int e = lane % E;
        for (int ch = wave * G + lane / E; ch < nch; ch += J) {
            const int c = cnt[(int64_t)ch * E + e];
            tot += c;
            if (ch < ch0) pre += c;
        }
    }
    s_tot[tid] = tot;
    s_pre[tid] = pre;
    __syncthreads();
    if (wave == 0) {
        int t = 0, p = 0;
        if (lane < E)
            for (int w = 0; w < kChunkWaves; ++w)
                for (int g = 0; g < G; ++g) {
                    t += s_tot[w * kWave + g * E + lane];
                    p += s_pre[w * kWave + g * E + lane];
                }
        int incl = t;
#pragma unroll
        for (int dd = 1; dd < kWave; dd <<= 1) {
            const int v = __shfl_up(incl, dd);
            if (lane >= dd) incl += v;
        }
        if (lane < E) {
            s_first[lane] = incl - t + p;
            if (blockIdx.x == 0) {
                counts[lane] = t;
                offsets[lane] = incl - t;
            }
        }
        if (blockIdx.x == 0 && lane == E - 1) offsets[E] = incl;
    }
    __syncthreads();
    const int ch = ch0 + wave;
    if (ch >= nch) return;  // uniform over the wave
    // this chunk's first row per expert: the workgroup's, plus the earlier
    // chunks of the workgroup
    int first = 0;
    if (lane < E) {
        first = s_first[lane];
        for (int w = 0; w < wave; ++w) first += cnt[(int64_t)(ch0 + w) * E + lane];
    }
    const int64_t a0 = (int64_t)ch * W, a1 = min((int64_t)A, a0 + W);
    for (int64_t b = a0; b < a1; b += kChunkBatch * kWave) {
        int ev[kChunkBatch], rv[kChunkBatch];
#pragma unroll
        for (int q = 0; q < kChunkBatch; ++q) {
            const int64_t a = b + q * kWave + lane;
            ev[q] = (a < a1) ? idx[a] : -1;
            rv[q] = (a < a1) ? row_of[a] : -1;
        }
#pragma unroll
        for (int q = 0; q < kChunkBatch; ++q) {
            const int64_t a = b + q * kWave + lane;
            const bool valid = (unsigned)ev[q] < (unsigned)E;
            const int f = __shfl(first, valid ? ev[q] : 0);
            if (valid) {
                const int row = f + rv[q];
                row_of[a] = row;
                token_of[row] = (int32_t)(a / k);
            }
        }
    }
}

// Assignments per chunk of the two-launch dispatch (a multiple of the wave,
// at most 512 chunks), or 0 where the single workgroup is used.
int dispatch_chunk_size(int64_t A) {
    if (A <= kDispatchChunkedFrom) return 0;
    const int64_t per = (A + 511) / 512;
    return (int)std::max<int64_t>(256, (per + kWave - 1) / kWave * kWave);
}

constexpr int kGatherWaves = 4;

__global__ __launch_bounds__(kGatherWaves * kWave) void gather_rows_kernel(
    const uint4 *__restrict__ x, int64_t T, int row_chunks, int k,
    const int32_t *__restrict__ row_of, uint4 *__restrict__ x_perm) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * kGatherWaves + threadIdx.x / kWave;
    if (t >= T) return;
    int rows[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) rows[j] = (j < k) ? row_of[t * k + j] : -1;
    const uint4 *src = x + t * row_chunks;
    for (int c = lane; c < row_chunks; c += kWave) {
        const uint4 v = src[c];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (rows[j] >= 0) x_perm[(int64_t)rows[j] * row_chunks + c] = v;
    }
}

}  // namespace moe

size_t moe_dispatch_scratch_bytes(int64_t A, int E) {
    const int W = moe::dispatch_chunk_size(A);
    if (W == 0) return 0;
    return sizeof(int32_t) * (size_t)((A + W - 1) / W) * (size_t)E;
}

hipError_t moe_launch_dispatch_index(const int32_t *idx, int64_t A, int E, int k,
                                     int32_t *counts, int32_t *offsets, int32_t *row_of,
                                     int32_t *token_of, int32_t *scratch, hipStream_t s) {
    const int W = moe::dispatch_chunk_size(A);
    if (W == 0 || !scratch) {
        hipLaunchKernelGGL(moe::dispatch_index_kernel, dim3(1), dim3(moe::kDispatchThreads), 0,
                           s, idx, (int)A, E, k, counts, offsets, row_of, token_of);
        return hipGetLastError();
    }
    const int nch = (int)((A + W - 1) / W);
    const dim3 grid((unsigned)((nch + moe::kChunkWaves - 1) / moe::kChunkWaves));
    const dim3 block(moe::kChunkWaves * moe::kWave);
    hipLaunchKernelGGL(moe::dispatch_chunk_rank_kernel, grid, block, 0, s, idx, (int)A, E, W, nch,
                       row_of, scratch);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(moe::dispatch_place_kernel, grid, block, 0, s, idx, (int)A, E, k, W, nch,
                       (const int32_t *)scratch, counts, offsets, row_of, token_of);
    return hipGetLastError();
}

hipError_t moe_launch_gather_rows(const void *x, int dt, int64_t T, int d, int k,
                                  const int32_t *row_of, void *x_perm, hipStream_t s) {
    const int es = (dt == 0) ? 4 : 2;
    const int row_chunks = d * es / 16;
    const dim3 grid((unsigned)((T + moe::kGatherWaves - 1) / moe::kGatherWaves));
    hipLaunchKernelGGL(moe::gather_rows_kernel, grid, dim3(moe::kGatherWaves * moe::kWave), 0, s,
                       (const uint4 *)x, T, row_chunks, k, row_of, (uint4 *)x_perm);
    return hipGetLastError();
}
