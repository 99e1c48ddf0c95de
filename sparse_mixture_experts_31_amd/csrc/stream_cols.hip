// stream_cols.hip — the decode layer's expert GEMMs for the smallest
// batches (one to eight tokens, so at most eight rows per expert).
//
// Same experts and the same weight stream as stream_gemm.hip (the SwiGLU
// MLP W2 (silu(W1 x) * W3 x): fdeinterviews breakdown, "The paper in one
// minute"; tokentrails lineage, Code listing), with the work cut the other
// way.  A few tokens keep only a few experts busy (two for one token under
// top-2) with a few rows each, and the tile kernel's 128-row tiles of them
// cannot give every CU an even share: it cuts their K into pieces whose fp32
// partial sums need a pass of their own after each GEMM.  Here workgroup b owns a
// run of output columns of every active expert and streams those weight rows
// over the whole K, so every CU streams the same bytes and nothing is left to
// add up afterwards:
//  * GEMM1: a stage is 8 columns, W1 rows c .. c + 8 and the same W3 rows
//    (16 rows of 1 KiB, as in the tile kernel), so u and v of a column come
//    out of one MFMA fragment and h = silu(u) v is formed at once;
//  * GEMM2: a stage is 16 W2 rows; the workgroup ends up holding every
//    active expert's outputs on its columns, so it forms y[t] = residual[t]
//    + sum_j g_j o_j[t] there itself (slot order, one fused multiply-add per
//    slot, as combine_kernel does).  The layer is three launches: router,
//    GEMM1, GEMM2.
// The columns are dealt in whole stages (Mixtral on 256 CUs: 7 GEMM1 stages
// and 1 GEMM2 stage per active expert on every CU).  The ring is the tile
// kernel's: five 16 KiB slots, every weight row piece one non-temporal
// global_load_lds, every wave issuing the same number of loads per stage (4
// weight rows, and one or two token rows or as many dwords into LDS nothing
// reads) so each wait is one constant.  A slot is refilled only once every wave is past
// it, so the time a stage's compute takes after its data lands is bytes
// not in flight: all four waves compute every stage, a quarter of its K
// each (4 v_mfma_f32_16x16x32_bf16; four of the sixteen token columns are
// real), and their sums meet in LDS once per expert.  (One wave per stage
// ran GEMM2 at 5.8 TB/s against 6.5 here.)  Every address a stage needs
// comes from per-lane tables read with readlane: a chain of LDS reads per
// stage (expert, its first row, the token of that row) cost 5-10 %.
#include "gemm_common.h"

namespace moe {

namespace {

constexpr int kCStage = 16 * 1024;

// Sizes for TOK token rows per expert (or per chunk of an expert's rows) at
// most: TOK = 4 for one to four tokens, 8 for five to eight (a token picks an
// expert once), 16 for GEMM2 alone at nine to 32 tokens, where an expert with
// more rows is taken in chunks of 16.  Each wave loads TOK / 4 of a chunk's
// token rows with the first stage of its K range and as many dwords into
// `junk` with the others, so every stage issues LOADS loads per wave.  The
// ring has P stages and TB token buffers; a token buffer is reloaded TB K
// ranges (at least TB stages) after it was first read, with the load of a
// stage P - 1 ahead of the consumer, so its stages are done when TB >= P.
// LDS decides the rest: GEMM2 at TOK = 8 takes at most four column stages
// per workgroup, at TOK = 16 one, with a four-stage ring.
template <bool SWIGLU, int TOK>
struct ColsCfg {
    static constexpr int kP = TOK == 16 ? 4 : 5;
    static constexpr int kTB = kP;
    static constexpr int kAMax = TOK == 16 ? 64 : 32;  // assignments T k at most
    static constexpr int kTokLoads = TOK / 4;
    static constexpr int kLoads = 4 + kTokLoads;
    static constexpr int kCPS = SWIGLU ? 8 : 16;  // output columns per stage
    static constexpr int kMaxS = (SWIGLU || TOK == 4) ? 8 : TOK == 8 ? 4 : 1;
    static constexpr int kOCols = SWIGLU ? 0 : kMaxS * 16;  // GEMM2 outputs kept per assignment
    static constexpr int kTokBuf = TOK * 1024;
    static constexpr int kRed = kMaxS * 4 * kWave * 16;  // the waves' partial sums of a stage set
    static constexpr int kLds = kP * kCStage + kTB * kTokBuf + 1024 + kAMax * kOCols * 4 + kRed;
    static_assert(TOK == 4 || TOK == 8 || (TOK == 16 && !SWIGLU), "token rows per chunk");
    static_assert(kTB >= kP, "token buffer reuse");
    static_assert(kAMax <= 64, "one lane per assignment");
    static_assert(kLds <= 160 * 1024 - 2 * 1024, "LDS capacity (2 KiB of static tables)");
};

}  // namespace

// GEMM1 (SWIGLU): act = x [T][act_ld], Wa = W1, Wb = W3 [E][N][K] (N = d_ff,
// K = d), h [T k][N] receives silu(u) v in grouped row order; workgroup 0
// also writes the grouping (counts, offsets, row_of, token_of).  GEMM2: act
// = h [T k][act_ld], Wa = W2 [E][N][K] (N = d, K = d_ff), y [T][N] receives
// the combined output.  topk_idx [T k] holds the experts of every (token,
// slot); out-of-range entries are skipped.  N is a multiple of 512 (16 for
// the stages), K a multiple of 512, T k <= ColsCfg::kAMax, E <= 64, and the
// grid leaves each workgroup between 1 and ColsCfg::kMaxS stages of columns.
template <bool SWIGLU, int TOK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void stream_cols_kernel(
    const bf16_t *__restrict__ act, int64_t act_ld, const int32_t *__restrict__ topk_idx, int k,
    int T, const bf16_t *__restrict__ Wa, const bf16_t *__restrict__ Wb, int E, int N, int K,
    bf16_t *__restrict__ h, const float *__restrict__ gw, const bf16_t *__restrict__ residual,
    bf16_t *__restrict__ y, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ row_of, int32_t *__restrict__ token_of) {
    using C = ColsCfg<SWIGLU, TOK>;
    constexpr int P = C::kP, TB = C::kTB, CPS = C::kCPS, MAXS = C::kMaxS, TL = C::kTokLoads;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    char *const ring = smem;
    char *const tbuf = smem + P * kCStage;
    char *const junk = tbuf + TB * C::kTokBuf;
    float *const s_o = (float *)(junk + 1024);  // GEMM2: [assignment][column] outputs
    char *const red = (char *)(s_o + C::kAMax * C::kOCols);  // [stage][wave] partial sums
    // per expert: count, first row; per entry (a chunk of at most TOK of an
    // expert's rows): expert, first row, rows; per assignment: row; per row:
    // assignment
    __shared__ int s_cnt[64], s_off[64], s_ent[64], s_eoff[64], s_ecnt[64];
    __shared__ int s_row[64], s_asg[64], s_nent;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int A = T * k;
    auto u = [](int v) { return __builtin_amdgcn_readfirstlane(v); };

    // Stable grouping of the assignments by expert (the dispatch kernel's
    // order: experts ascending, then assignment index), by wave 0, one lane
    // per assignment and one lane per expert: a ballot per expert gives each
    // assignment its rank and each expert its count, a shuffle scan the
    // experts' first rows.
    if (wave == 0) {
        const int e = lane < A ? topk_idx[lane] : -1;
        const bool valid = (unsigned)e < (unsigned)E;
        const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        int rank = 0, cnt = 0;
        for (int ex = 0; ex < E; ++ex) {
            const uint64_t m = __ballot(valid && e == ex);
            if (valid && e == ex) rank = __popcll(m & lower);
            if (lane == ex) cnt = __popcll(m);
        }
        int incl = cnt;
#pragma unroll
        for (int dd = 1; dd < kWave; dd <<= 1) {
            const int v = __shfl_up(incl, dd);
            if (lane >= dd) incl += v;
        }
        const int off = incl - cnt;
        if (lane < E) {
            s_cnt[lane] = cnt;
            s_off[lane] = off;
        }
        // the entries, experts ascending: ceil(cnt / TOK) chunks per expert
        // (at most 64: each holds a row)
        const int nch = lane < E ? (cnt + TOK - 1) / TOK : 0;
        int cincl = nch;
#pragma unroll
        for (int dd = 1; dd < kWave; dd <<= 1) {
            const int v = __shfl_up(cincl, dd);
            if (lane >= dd) cincl += v;
        }
        for (int c = 0; c < nch; ++c) {
            const int q = cincl - nch + c;
            s_ent[q] = lane;
            s_eoff[q] = off + c * TOK;
            s_ecnt[q] = min(TOK, cnt - c * TOK);
        }
        if (lane == kWave - 1) s_nent = cincl;
        const int eoff = __shfl(off, valid ? e : 0);  // every lane takes part
        const int row = valid ? eoff + rank : -1;
        if (lane < A) s_row[lane] = row;
        if (valid) s_asg[row] = lane;
        if (SWIGLU && blockIdx.x == 0) {
            if (lane < E) {
                counts[lane] = cnt;
                offsets[lane] = off;
            }
            if (lane == E - 1) offsets[E] = incl;
            if (lane < A) {
                row_of[lane] = row;
                if (valid) token_of[row] = lane / k;
            }
        }
    }
    __syncthreads();

    // This workgroup's columns: stages [u0, u1) of the N / CPS.
    const int NU = N / CPS, NG = gridDim.x;
    const int u0 = (int)((int64_t)blockIdx.x * NU / NG);
    const int S = (int)((int64_t)(blockIdx.x + 1) * NU / NG) - u0;
    const int c0 = u0 * CPS;
    const int n_kc = K / 512;
    const int n_act = u(s_nent);  // entries

    // Per-entry values, lane i for entry i (built once, read with
    // readlane, so a stage's addresses never wait on LDS): the byte offset
    // of its weight matrix, of the token rows TL wave + j this wave loads for
    // it (rows past its count repeat its last), its first grouped row and
    // its count.
    int64_t t_w = 0, t_tok[TL];
    int t_off = 0, t_cnt = 0;
#pragma unroll
    for (int j = 0; j < TL; ++j) t_tok[j] = 0;
    if (lane < n_act) {
        const int e = s_ent[lane];
        t_off = s_eoff[lane];
        t_cnt = s_ecnt[lane];
        t_w = (int64_t)e * N * K * 2;
#pragma unroll
        for (int j = 0; j < TL; ++j) {
            const int g = t_off + min(TL * wave + j, t_cnt - 1);
            const int row = SWIGLU ? s_asg[g] / k : g;
            t_tok[j] = (int64_t)row * act_ld * 2;
        }
    }
    auto lane64 = [](int64_t v, int i) -> int64_t {
        const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, i);
        const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), i);
        return (int64_t)(((uint64_t)hi << 32) | lo);
    };
    const int64_t kb = (int64_t)K * 2;  // bytes per weight row

    // ---- producer: P - 1 stages ahead; stage pq goes to slot pq % P.
    // (pi, pkc, ps): entry, K range, column stage of the next load;
    // its token rows go to buffer (pi n_kc + pkc) % TB.  Past the last
    // stage the loads are dwords into `junk`, so the counts stay.
    int pi = 0, pkc = 0, ps = 0, pq = 0, pt = 0;
    const char *const dummy = (const char *)act + lane * 4;
    const int lofs = lane << 4;
    auto issue = [&]() __attribute__((always_inline)) {
        char *slot = ring + (pq % P) * kCStage;
        if (pi < n_act) {
            const int64_t wo = lane64(t_w, pi) + (int64_t)(c0 + CPS * ps) * kb + pkc * 1024;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = 4 * wave + q;  // row within the stage
                const char *src;
                if constexpr (SWIGLU)
                    src = (const char *)(r < 8 ? Wa : Wb) + wo + (r & 7) * kb;
                else
                    src = (const char *)Wa + wo + r * kb;
                dma16_nt(src + (lofs ^ (r << 4)), slot + r * 1024);
            }
            if (ps == 0) {
#pragma unroll
                for (int j = 0; j < TL; ++j) {
                    const int jr = TL * wave + j;  // token row in the buffer
                    const char *src = (const char *)act + lane64(t_tok[j], pi) + pkc * 1024;
                    dma16(src + (lofs ^ (jr << 4)), tbuf + (pt % TB) * C::kTokBuf + jr * 1024);
                }
            } else {
#pragma unroll
                for (int j = 0; j < TL; ++j) dma4(dummy, junk);
            }
        } else {
#pragma unroll
            for (int q = 0; q < C::kLoads; ++q) dma4(dummy, junk);
        }
        ++pq;
        if (++ps == S) {
            ps = 0;
            ++pt;
            if (++pkc == n_kc) {
                pkc = 0;
                ++pi;
            }
        }
    };

    if (n_act > 0 && S > 0) {
#pragma unroll
        for (int q = 0; q < P - 1; ++q) issue();

        // ---- consumer: every wave computes a quarter of every stage's K
        // (k-steps 4 wave .. + 4 of the sixteen), into its own accumulators
        const int lr = lane & 15, lq = lane >> 4;
        f32x4 acc[MAXS];
#pragma unroll
        for (int s = 0; s < MAXS; ++s) acc[s] = f32x4{};
        int cq = 0;  // stages consumed
        for (int i = 0; i < n_act; ++i) {
            for (int kc = 0; kc < n_kc; ++kc) {
                const char *tb = tbuf + ((i * n_kc + kc) % TB) * C::kTokBuf;
#pragma unroll
                for (int s = 0; s < MAXS; ++s) {
                    if (s < S) {
                        // stage cq landed (this wave's loads, then everyone's),
                        // and every wave is done with the slot loaded next
                        wait_vmcnt_lgkm0<(P - 2) * C::kLoads>();
                        stage_barrier();
                        issue();
                        constexpr int NT = 4;
                        const char *ws = ring + (cq % P) * kCStage;
                        i32x4 w[NT], xv[NT];
#pragma unroll
                        for (int t = 0; t < NT; ++t) {
                            const int c = 4 * (NT * wave + t) + lq;
                            w[t] = *(const i32x4 *)(ws + swz1k(lr, c));
                            xv[t] = *(const i32x4 *)(tb + swz1k(lr & (TOK - 1), c));
                        }
                        f32x4 ab[2] = {acc[s], f32x4{}};
#pragma unroll
                        for (int t = 0; t < NT; ++t) ab[t & 1] = mma16(w[t], xv[t], ab[t & 1]);
                        acc[s] = ab[0] + ab[1];
                        ++cq;
                    }
                }
            }

            // Expert i done: the four waves' sums of each stage meet in LDS
            // (added in wave order), then wave w finishes stages w and w + 4.
            // Lane l holds stage rows 4 (l / 16) .. + 4 for token l % 16
            // (tokens below the expert's count are real); GEMM1: rows 0-7
            // are u, rows 8-15 the same columns' v, 32 lanes apart.
#pragma unroll
            for (int s = 0; s < MAXS; ++s) {
                if (s < S) *(f32x4 *)(red + ((s * 4 + wave) * kWave + lane) * 16) = acc[s];
                acc[s] = f32x4{};
            }
            // LDS writes done, then a barrier without a memory fence (a
            // fence would wait for the ring's loads in flight as well)
            wait_vmcnt_lgkm0<63>();
            stage_barrier();
            const int cnt = __builtin_amdgcn_readlane(t_cnt, i);
            const int off = __builtin_amdgcn_readlane(t_off, i);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int s = wave + 4 * hh;
                if (s < S && s < MAXS) {
                    f32x4 x = *(const f32x4 *)(red + ((s * 4 + 0) * kWave + lane) * 16);
#pragma unroll
                    for (int ww = 1; ww < 4; ++ww)
                        x += *(const f32x4 *)(red + ((s * 4 + ww) * kWave + lane) * 16);
                    const int n = lr;
                    if constexpr (SWIGLU) {
                        f32x4 v;
#pragma unroll
                        for (int q = 0; q < 4; ++q) v[q] = __shfl_xor(x[q], 32);
                        if (lane < 32 && n < cnt) {
                            float r[4];
#pragma unroll
                            for (int q = 0; q < 4; ++q) r[q] = silu(x[q]) * v[q];
                            store4<bf16_t>(h + (int64_t)(off + n) * N + c0 + CPS * s + 4 * lq,
                                           r[0], r[1], r[2], r[3]);
                        }
                    } else if (n < cnt) {
                        const int a = s_asg[off + n];
                        *(f32x4 *)(s_o + a * C::kOCols + CPS * s + 4 * lq) = x;
                    }
                }
            }
            // `red` is written again only after the next expert's stages,
            // whose barriers order these reads before those writes
        }
    }

    // GEMM2: y on this workgroup's columns for every token, from the
    // outputs in LDS, with combine_kernel's arithmetic.
    if constexpr (!SWIGLU) {
        __syncthreads();
        const int c8 = S * CPS / 8;  // 8-column pieces
        for (int q = tid; q < T * c8; q += 256) {
            const int t = q / c8, cl = (q - t * c8) * 8;
            float acc8[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) acc8[c] = 0.f;
            for (int j = 0; j < k; ++j) {
                const int a = t * k + j;
                if (s_row[a] < 0) continue;
                const float g = gw[a];
                const float *o = s_o + a * C::kOCols + cl;
#pragma unroll
                for (int c = 0; c < 8; ++c) acc8[c] = fmaf(g, o[c], acc8[c]);
            }
            const int64_t at = (int64_t)t * N + c0 + cl;
            if (residual) {
                const uint4 rv = *(const uint4 *)(residual + at);
                const uint32_t w4[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc8[2 * i] += bf16_bits_to_f32(w4[i] & 0xffffu);
                    acc8[2 * i + 1] += bf16_bits_to_f32(w4[i] >> 16);
                }
            }
            *(uint4 *)(y + at) =
                make_uint4(pack_bf16x2(acc8[0], acc8[1]), pack_bf16x2(acc8[2], acc8[3]),
                           pack_bf16x2(acc8[4], acc8[5]), pack_bf16x2(acc8[6], acc8[7]));
        }
    }
    wait_vmcnt_lgkm0<0>();  // the trailing loads land before the wave ends
}

namespace {

// Workgroups of each GEMM: one per CU, never more than its stages of columns.
int cols_grid(int stages) { return std::max(1, std::min(device_cus(), stages)); }

// Token rows per expert the kernels are built for at T tokens (0: none).
int cols_tok(int64_t T) { return T < 1 ? 0 : T <= 4 ? 4 : T <= 8 ? 8 : 0; }

template <int TOK>
hipError_t launch_cols(const void *x, const void *W1, const void *W3, const void *W2, int64_t T,
                       int d, int d_ff, int E, void *hbuf, const StreamFuse &f,
                       hipEvent_t gemm1_done, hipStream_t s) {
    using C1 = ColsCfg<true, TOK>;
    using C2 = ColsCfg<false, TOK>;
    hipError_t err = set_lds_limit<stream_cols_kernel<true, TOK>>(C1::kLds);
    if (err == hipSuccess) err = set_lds_limit<stream_cols_kernel<false, TOK>>(C2::kLds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((stream_cols_kernel<true, TOK>), dim3(cols_grid(d_ff / C1::kCPS)), dim3(256),
                       C1::kLds, s, (const bf16_t *)x, (int64_t)d, f.topk_idx, f.k, (int)T,
                       (const bf16_t *)W1, (const bf16_t *)W3, E, d_ff, d, (bf16_t *)hbuf,
                       nullptr, nullptr, nullptr, f.counts, f.offsets, f.row_of, f.token_of);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (gemm1_done && (err = hipEventRecord(gemm1_done, s)) != hipSuccess) return err;
    hipLaunchKernelGGL((stream_cols_kernel<false, TOK>), dim3(cols_grid(d / C2::kCPS)), dim3(256),
                       C2::kLds, s, (const bf16_t *)hbuf, (int64_t)d_ff, f.topk_idx, f.k, (int)T,
                       (const bf16_t *)W2, nullptr, E, d, d_ff, nullptr, f.gw, f.residual, f.y,
                       nullptr, nullptr, nullptr, nullptr);
    return hipGetLastError();
}

template <int TOK>
bool cols_fit(int d, int d_ff) {
    using C1 = ColsCfg<true, TOK>;
    using C2 = ColsCfg<false, TOK>;
    const int s1 = d_ff / C1::kCPS, s2 = d / C2::kCPS;
    const int g1 = cols_grid(s1), g2 = cols_grid(s2);
    return (s1 + g1 - 1) / g1 <= C1::kMaxS && (s2 + g2 - 1) / g2 <= C2::kMaxS;
}

}  // namespace

bool stream_cols_supported(int64_t T, int k, int d, int d_ff, int E) {
    const int tok = cols_tok(T);
    if (tok == 0 || T * k > 32 || E < 1 || E > 64) return false;
    if (d < 512 || d_ff < 512 || d % 512 != 0 || d_ff % 512 != 0) return false;
    return tok == 4 ? cols_fit<4>(d, d_ff) : cols_fit<8>(d, d_ff);
}

bool stream_cols_w2_supported(int64_t T, int k, int d, int d_ff, int E) {
    using C2 = ColsCfg<false, 16>;
    if (T < 9 || T > 32 || T * k > C2::kAMax || E < 1 || E > 64) return false;
    if (d < 512 || d_ff < 512 || d % 512 != 0 || d_ff % 512 != 0) return false;
    const int s2 = d / C2::kCPS, g2 = cols_grid(s2);
    return (s2 + g2 - 1) / g2 <= C2::kMaxS;
}

hipError_t launch_stream_cols_w2(const void *hbuf, const void *W2, int64_t T, int d, int d_ff,
                                 int E, const StreamFuse &f, hipStream_t s) {
    using C2 = ColsCfg<false, 16>;
    hipError_t err = set_lds_limit<stream_cols_kernel<false, 16>>(C2::kLds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((stream_cols_kernel<false, 16>), dim3(cols_grid(d / C2::kCPS)), dim3(256),
                       C2::kLds, s, (const bf16_t *)hbuf, (int64_t)d_ff, f.topk_idx, f.k, (int)T,
                       (const bf16_t *)W2, nullptr, E, d, d_ff, nullptr, f.gw, f.residual, f.y,
                       nullptr, nullptr, nullptr, nullptr);
    return hipGetLastError();
}

hipError_t launch_stream_cols(const void *x, const void *W1, const void *W3, const void *W2,
                              int64_t T, int d, int d_ff, int E, void *hbuf,
                              const StreamFuse &f, hipEvent_t gemm1_done, hipStream_t s) {
    if (cols_tok(T) == 4)
        return launch_cols<4>(x, W1, W3, W2, T, d, d_ff, E, hbuf, f, gemm1_done, s);
    return launch_cols<8>(x, W1, W3, W2, T, d, d_ff, E, hbuf, f, gemm1_done, s);
}

}  // namespace moe
