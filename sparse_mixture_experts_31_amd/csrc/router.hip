// router.hip — router scores fused with top-k and the softmax over the kept
// scores.
//
// The router is a linear map from a token's vector to one score per expert
// (ennepo lecture, router passage; tokentrails lineage, step "The router").
// TopK keeps the k best scores and the softmax runs over them alone
// (flashpapers summary, "How It Works").
//
// WPT wavefronts own TPW tokens and treat the experts EG at a time.  Each
// lane walks its strided share of the wave's slice of d, 8 elements per
// step, and accumulates x_i * Wg_e,i in fp64: a bf16 or fp32
// element times an fp32 weight is exact in fp64, so only the fp64 additions
// round and the final fp32 score is (almost always) the correctly rounded
// value of the exact dot product.  That keeps the discrete top-k choice
// stable against reduction order.  A recursive-halving butterfly reduces the
// TPW*EG partial sums across the wave with TPW*EG fp64 shuffles instead of
// TPW*EG*6.  The fp32 scores land in LDS; lane t < TPW
// then picks the top k of token t (strict '>' over ascending expert index, so
// equal fp32 scores go to the lower index) and the gates
// g_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).  From 1024 tokens on,
// router_topk_lds_kernel does the same per token with Wg held in LDS.
#include "gemm_common.h"

namespace moe {

template <typename Tin>
__device__ __forceinline__ void load8(const Tin *p, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<float>(const float *p, float (&v)[8]) {
    float4 a = *(const float4 *)p;
    float4 b = *(const float4 *)(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t *p, float (&v)[8]) {
    uint4 a = *(const uint4 *)p;
    uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// Sum NV per-lane values across the 64 lanes.  After the call lane L holds
// the full sum of value index (L / (64 / NV)) in v[0].  BY_VALUE reads both
// values of a pair before choosing between them; the other form chooses
// between their addresses, which in the LDS kernel put its accumulators in
// scratch memory (the same additions either way; the four-wave kernel is
// 0.3 us faster with the address form at decode sizes).
template <int NV, bool BY_VALUE = false>
__device__ __forceinline__ void wave_reduce_halving(double (&v)[NV], int lane) {
    int off = 32;
#pragma unroll
    for (int cnt = NV; cnt > 1; cnt >>= 1, off >>= 1) {
        const int half = cnt / 2;
        const bool hi = (lane & off) != 0;
#pragma unroll
        for (int j = 0; j < half; ++j) {
            if constexpr (BY_VALUE) {
                const double lo_v = v[j], hi_v = v[j + half];
                v[j] = (hi ? hi_v : lo_v) + __shfl_xor(hi ? lo_v : hi_v, off);
            } else {
                double send = hi ? v[j] : v[j + half];
                double keep = hi ? v[j + half] : v[j];
                v[j] = keep + __shfl_xor(send, off);
            }
        }
    }
#pragma unroll
    for (; off >= 1; off >>= 1) v[0] += __shfl_xor(v[0], off);
}

constexpr int kRouterWaves = 4;

// The top k of E fp32 scores L (strict '>' over ascending expert index, so
// equal scores go to the lower index): sel[j], sl[j] for j < k.
__device__ __forceinline__ void select_topk(const float *L, int E, int k, int (&sel)[8],
                                            float (&sl)[8]) {
    uint64_t used = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        sel[j] = 0;
        sl[j] = 0.f;
        if (j < k) {
            int best = -1;
            float bv = 0.f;
            for (int e = 0; e < E; ++e) {
                if ((used >> e) & 1ull) continue;
                const float v = L[e];
                if (best < 0 || v > bv) {
                    best = e;
                    bv = v;
                }
            }
            used |= 1ull << best;
            sel[j] = best;
            sl[j] = bv;
        }
    }
}

// Token t's choices and gates g_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).
__device__ __forceinline__ void write_choice(int64_t t, int k, const int (&sel)[8],
                                             const float (&sl)[8], int32_t *__restrict__ out_idx,
                                             float *__restrict__ out_w) {
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (j < k) z += expf(sl[j] - sl[0]);
    const int64_t o = t * k;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j < k) {
            out_idx[o + j] = sel[j];
            out_w[o + j] = expf(sl[j] - sl[0]) / z;
        }
    }
}

// WPT waves share each group of TPW tokens, every wave covering a contiguous
// 1/WPT of d; their fp64 partial sums meet in LDS and are added in wave order.
// With STATS the workgroup also leaves, for the load-balancing statistics,
// the sum over its tokens (in token order) of each expert's full softmax
// probability (fp64, part_p[block][E]) and how many of its tokens' choices
// went to each expert (part_c[block][E]).
template <typename Tin, int TPW, int EG, int WPT, bool STATS = false, int WAVES = kRouterWaves>
__global__ __launch_bounds__(WAVES * kWave) void router_topk_kernel(
    const Tin *__restrict__ x, const float *__restrict__ Wg, int64_t T, int d, int E, int k,
    int32_t *__restrict__ out_idx, float *__restrict__ out_w, float *__restrict__ out_logits,
    double *__restrict__ part_p = nullptr, int32_t *__restrict__ part_c = nullptr,
    int32_t *__restrict__ zero = nullptr, int zero_n = 0) {
    // zero[0, zero_n): counters the launch after this one starts from
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < zero_n; i += WAVES * kWave) zero[i] = 0;
    constexpr int kGroups = WAVES / WPT;  // token groups per workgroup
    __shared__ float s_logit[kGroups][TPW][64];
    __shared__ double s_part[kGroups][WPT][TPW * EG];
    __shared__ double s_prob[STATS ? kGroups * TPW : 1][64];
    __shared__ int s_sel[STATS ? kGroups * TPW : 1][8];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int grp = wave / WPT, part = wave % WPT;
    const int64_t tok0 = ((int64_t)blockIdx.x * kGroups + grp) * TPW;
    const int dpart = d / WPT;
    const int dlo = part * dpart, dhi = dlo + dpart;
    constexpr int lanes_per_value = 64 / (TPW * EG);

    for (int e0 = 0; e0 < E; e0 += EG) {
        double acc[TPW * EG];
#pragma unroll
        for (int i = 0; i < TPW * EG; ++i) acc[i] = 0.0;
#pragma unroll 1
        for (int i = dlo + lane * 8; i < dhi; i += kWave * 8) {
            float xv[TPW][8];
            // rows past T and experts past E are clamped to valid ones (no
            // branches, so the conversions stay next to their use); their
            // sums are never stored
#pragma unroll
            for (int t = 0; t < TPW; ++t)
                load8<Tin>(x + min(tok0 + t, T - 1) * (int64_t)d + i, xv[t]);
            // all EG experts' weights first, then the products with the
            // experts innermost: EG independent accumulation chains in flight
            // (each accumulator still takes its 8 products in order)
            float wv[EG][8];
#pragma unroll
            for (int j = 0; j < EG; ++j)
                load8<float>(Wg + (int64_t)min(e0 + j, E - 1) * d + i, wv[j]);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
#pragma unroll
                for (int t = 0; t < TPW; ++t)
#pragma unroll
                    for (int j = 0; j < EG; ++j)
                        acc[t * EG + j] = fma((double)xv[t][c], (double)wv[j][c], acc[t * EG + j]);
                // one element's conversions at a time (else they are all
                // hoisted and the registers run out)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wave_reduce_halving<TPW * EG>(acc, lane);
        if ((lane % lanes_per_value) == 0) s_part[grp][part][lane / lanes_per_value] = acc[0];
        __syncthreads();
        if (part == 0 && lane < TPW * EG) {
            double v = s_part[grp][0][lane];
#pragma unroll
            for (int p2 = 1; p2 < WPT; ++p2) v += s_part[grp][p2][lane];
            const int t = lane / EG, j = lane % EG;
            if (e0 + j < E) s_logit[grp][t][e0 + j] = (float)v;
        }
        __syncthreads();
    }

    if (part == 0) {
        // scores out (optional), coalesced over the group's TPW x E block
        if (out_logits) {
            for (int q = lane; q < TPW * E; q += kWave) {
                const int t = q / E, e = q % E;
                if (tok0 + t < T) out_logits[(tok0 + t) * E + e] = s_logit[grp][t][e];
            }
        }
        if (lane < TPW) {
            const int t = lane;
            const bool valid = tok0 + t < T;
            const float *L = s_logit[grp][t];
            int sel[8];
            float sl[8];
            select_topk(L, E, k, sel, sl);
            if (valid) write_choice(tok0 + t, k, sel, sl, out_idx, out_w);
            if constexpr (STATS) {
                // full softmax over all E scores (l_max = sl[0]), in fp64
                const int slot = grp * TPW + t;
                double zz = 0.0;
                for (int e = 0; e < E; ++e) zz += exp((double)L[e] - (double)sl[0]);
                for (int e = 0; e < E; ++e)
                    s_prob[slot][e] = valid ? exp((double)L[e] - (double)sl[0]) / zz : 0.0;
#pragma unroll
                for (int j = 0; j < 8; ++j) s_sel[slot][j] = (valid && j < k) ? sel[j] : -1;
            }
        }
    }
    if constexpr (STATS) {
        __syncthreads();
        const int e = threadIdx.x;
        if (e < E) {
            double p = 0.0;
            int c = 0;
            for (int slot = 0; slot < kGroups * TPW; ++slot) {
                p += s_prob[slot][e];
#pragma unroll
                for (int j = 0; j < 8; ++j) c += (s_sel[slot][j] == e);
            }
            part_p[(int64_t)blockIdx.x * E + e] = p;
            part_c[(int64_t)blockIdx.x * E + e] = c;
        }
    }
}

constexpr int kRouterLdsWaves = 8;
constexpr int kRouterLdsBytes = 128 * 1024;  // most Wg bytes held in LDS

// Many tokens: every wave of router_topk_kernel's one-wave-per-token form
// reads all of Wg (E d fp32) per token, which at thousands of tokens makes
// the router an L2 stream of T times Wg.  Here a workgroup copies Wg into
// LDS once and its eight waves walk groups of TPW consecutive tokens (wave w
// of workgroup b: group 8 b + w, then a grid further).  For each token a
// lane covers the same elements of d in the same order with the same fp64
// steps and the same wave reduction as the one-wave-per-token form of
// router_topk_kernel (WPT = 1, which the load statistics use from 1024
// tokens on), so those two give the same scores bit for bit.  Below 1024
// tokens both entry points use the four-wave form (WPT = 4), whose fp64
// partial sums meet in a different order: a score may then differ from the
// one-wave form's in its last fp32 bit, rarely.  A group's tokens share
// each Wg value read from LDS and its conversion to fp64, and the next
// 512-element piece of their rows is loaded while the current one is used.
template <typename Tin, int TPW>
__global__ __launch_bounds__(kRouterLdsWaves * kWave) void router_topk_lds_kernel(
    const Tin *__restrict__ x, const float *__restrict__ Wg, int64_t T, int d, int E, int k,
    int32_t *__restrict__ out_idx, float *__restrict__ out_w, float *__restrict__ out_logits,
    int32_t *__restrict__ zero, int zero_n) {
    extern __shared__ __attribute__((aligned(16))) float s_wg[];  // [E][d]
    // zero[0, zero_n): counters the launch after this one starts from
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < zero_n; i += kRouterLdsWaves * kWave) zero[i] = 0;
    __shared__ float s_logit[kRouterLdsWaves][TPW][64];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    // Wg into LDS, sixteen 16-byte loads in flight per thread
    const int n4 = E * d / 4;  // d is a multiple of 8
    constexpr int kThreads = kRouterLdsWaves * kWave, kBatch = 16;
    for (int i0 = threadIdx.x; i0 < n4; i0 += kBatch * kThreads) {
        float4 v[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q)  // clamped, so the loads need no branch
            v[q] = ((const float4 *)Wg)[min(i0 + q * kThreads, n4 - 1)];
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
            if (i0 + q * kThreads < n4) ((float4 *)s_wg)[i0 + q * kThreads] = v[q];
    }
    __syncthreads();

    constexpr int kStep = kWave * 8;  // elements of d per lane step
    const int npiece = d / kStep;     // d is a multiple of 512
    for (int64_t t0 = ((int64_t)blockIdx.x * kRouterLdsWaves + wave) * TPW; t0 < T;
         t0 += (int64_t)gridDim.x * kRouterLdsWaves * TPW) {
        const Tin *xr[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t)  // rows past T repeat the last row; never stored
            xr[t] = x + min(t0 + t, T - 1) * (int64_t)d + lane * 8;
        for (int e0 = 0; e0 < E; e0 += 8) {
            double acc[TPW][8];
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[t][j] = 0.0;
            float xv[TPW][8], xn[TPW][8];
#pragma unroll
            for (int t = 0; t < TPW; ++t) load8<Tin>(xr[t], xv[t]);
#pragma unroll 1
            for (int p = 0; p < npiece; ++p) {
                const int pn = min(p + 1, npiece - 1);  // the next piece (the last reloads itself)
#pragma unroll
                for (int t = 0; t < TPW; ++t) load8<Tin>(xr[t] + pn * kStep, xn[t]);
                // experts innermost: 8 TPW independent chains (experts past E
                // read a valid row; their sums are never stored)
                float wv[8][8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    load8<float>(s_wg + min(e0 + j, E - 1) * d + lane * 8 + p * kStep, wv[j]);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
#pragma unroll
                    for (int t = 0; t < TPW; ++t)
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            acc[t][j] = fma((double)xv[t][c], (double)wv[j][c], acc[t][j]);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int t = 0; t < TPW; ++t)
#pragma unroll
                    for (int c = 0; c < 8; ++c) xv[t][c] = xn[t][c];
            }
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                wave_reduce_halving<8, true>(acc[t], lane);
                if ((lane & 7) == 0 && e0 + lane / 8 < E)
                    s_logit[wave][t][e0 + lane / 8] = (float)acc[t][0];
            }
        }
        if (out_logits)
            for (int q = lane; q < TPW * E; q += kWave) {
                const int t = q / E, e = q % E;
                if (t0 + t < T) out_logits[(t0 + t) * E + e] = s_logit[wave][t][e];
            }
        if (lane < TPW && t0 + lane < T) {
            int sel[8];
            float sl[8];
            select_topk(s_logit[wave][lane], E, k, sel, sl);
            write_choice(t0 + lane, k, sel, sl, out_idx, out_w);
        }
    }
}

// The router's per-block statistics summed in a fixed order (16 contiguous
// chunks of blocks per expert, then the chunks in order), so the result is
// the same bit for bit on every run:
//   f[e] = count_e / (T k), P[e] = (sum of the token probabilities) / T,
//   laux = E * sum_e f[e] P[e]   (tokentrails lineage, step "Load balancing").
__global__ __launch_bounds__(1024) void balance_reduce_kernel(
    const double *__restrict__ part_p, const int32_t *__restrict__ part_c, int nblocks, int64_t T,
    int E, int k, float *__restrict__ f_out, float *__restrict__ P_out,
    float *__restrict__ laux_out) {
    constexpr int kChunks = 16;
    __shared__ double s_p[kChunks][64];
    __shared__ long long s_c[kChunks][64];
    __shared__ double s_fp[64];
    const int e = threadIdx.x % 64, ch = threadIdx.x / 64;
    if (e < E) {
        const int b0 = (int)((int64_t)nblocks * ch / kChunks);
        const int b1 = (int)((int64_t)nblocks * (ch + 1) / kChunks);
        double p = 0.0;
        long long c = 0;
        for (int b = b0; b < b1; ++b) {
            p += part_p[(int64_t)b * E + e];
            c += part_c[(int64_t)b * E + e];
        }
        s_p[ch][e] = p;
        s_c[ch][e] = c;
    }
    __syncthreads();
    if (threadIdx.x < E) {
        double p = 0.0;
        long long c = 0;
        for (int q = 0; q < kChunks; ++q) {
            p += s_p[q][e];
            c += s_c[q][e];
        }
        const double fe = (double)c / ((double)T * k), pe = p / (double)T;
        f_out[e] = (float)fe;
        P_out[e] = (float)pe;
        s_fp[e] = fe * pe;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = 0.0;
        for (int q = 0; q < E; ++q) s += s_fp[q];
        *laux_out = (float)((double)E * s);
    }
}

}  // namespace moe

namespace {

// Few tokens: four waves split each token's row, so a small batch still
// spreads over many waves (at T = 32 on MI355X: 7.2 us inside the layer,
// against 8.9 us with sixteen waves per token and 16.7 us with one).  Many
// tokens: one wave per token, four tokens per workgroup, or the LDS kernel.
bool router_wide_rows(int64_t T) { return T < 1024; }

template <typename Tin, int TPW>
hipError_t launch_router_lds_t(const Tin *x, const float *Wg, int64_t T, int d, int E, int k,
                               int32_t *idx, float *gw, float *logits, int32_t *zero, int zero_n,
                               hipStream_t s) {
    using namespace moe;
    const int bytes = E * d * (int)sizeof(float);  // <= kRouterLdsBytes
    hipError_t err = set_lds_limit<router_topk_lds_kernel<Tin, TPW>>(kRouterLdsBytes);
    if (err != hipSuccess) return err;
    const int64_t per_block = (int64_t)kRouterLdsWaves * TPW;
    const int64_t blocks = std::min<int64_t>(device_cus(), (T + per_block - 1) / per_block);
    hipLaunchKernelGGL((router_topk_lds_kernel<Tin, TPW>), dim3((unsigned)blocks),
                       dim3(kRouterLdsWaves * kWave), bytes, s, x, Wg, T, d, E, k, idx, gw,
                       logits, zero, zero_n);
    return hipGetLastError();
}

// Tokens per wave: two once that still gives every CU a workgroup.  (On
// MI355X two tokens per wave take the T = 4096 router from 32.3 to 30.8 us
// and the T = 16384 one from 99 to 87 us; four were eight times slower.)
template <typename Tin>
hipError_t launch_router_lds(const Tin *x, const float *Wg, int64_t T, int d, int E, int k,
                             int32_t *idx, float *gw, float *logits, int32_t *zero, int zero_n,
                             hipStream_t s) {
    const int64_t full = (int64_t)moe::kRouterLdsWaves * moe::device_cus();  // waves in one pass
    if (T >= 2 * full)
        return launch_router_lds_t<Tin, 2>(x, Wg, T, d, E, k, idx, gw, logits, zero, zero_n, s);
    return launch_router_lds_t<Tin, 1>(x, Wg, T, d, E, k, idx, gw, logits, zero, zero_n, s);
}

template <bool STATS>
hipError_t launch_router_impl(const void *x, int dt, const float *Wg, int64_t T, int d, int E,
                              int k, int32_t *idx, float *gw, float *logits, double *part_p,
                              int32_t *part_c, hipStream_t s, int32_t *zero = nullptr,
                              int zero_n = 0) {
    using namespace moe;
    const dim3 block(kRouterWaves * kWave);
    const dim3 grid((unsigned)moe_router_blocks(T));
    if (!STATS && !router_wide_rows(T) && d % 512 == 0 && (int64_t)E * d * 4 <= kRouterLdsBytes) {
        // many tokens, Wg small enough for LDS
        if (dt == 0)
            return launch_router_lds((const float *)x, Wg, T, d, E, k, idx, gw, logits, zero,
                                     zero_n, s);
        return launch_router_lds((const bf16_t *)x, Wg, T, d, E, k, idx, gw, logits, zero, zero_n,
                                 s);
    }
    if (router_wide_rows(T)) {
        if (dt == 0)
            hipLaunchKernelGGL((router_topk_kernel<float, 1, 8, 4, STATS>), grid, block, 0, s,
                               (const float *)x, Wg, T, d, E, k, idx, gw, logits, part_p, part_c,
                               zero, zero_n);
        else
            hipLaunchKernelGGL((router_topk_kernel<bf16_t, 1, 8, 4, STATS>), grid, block, 0, s,
                               (const bf16_t *)x, Wg, T, d, E, k, idx, gw, logits, part_p,
                               part_c, zero, zero_n);
    } else {
        if (dt == 0)
            hipLaunchKernelGGL((router_topk_kernel<float, 1, 8, 1, STATS>), grid, block, 0, s,
                               (const float *)x, Wg, T, d, E, k, idx, gw, logits, part_p, part_c,
                               zero, zero_n);
        else
            hipLaunchKernelGGL((router_topk_kernel<bf16_t, 1, 8, 1, STATS>), grid, block, 0, s,
                               (const bf16_t *)x, Wg, T, d, E, k, idx, gw, logits, part_p,
                               part_c, zero, zero_n);
    }
    return hipGetLastError();
}

}  // namespace

int64_t moe_router_blocks(int64_t T) {
    return router_wide_rows(T) ? T : (T + moe::kRouterWaves - 1) / moe::kRouterWaves;
}

hipError_t moe_launch_router(const void *x, int dt, const float *Wg, int64_t T, int d, int E,
                             int k, int32_t *idx, float *gw, float *logits, hipStream_t s,
                             int32_t *zero, int zero_n) {
    return launch_router_impl<false>(x, dt, Wg, T, d, E, k, idx, gw, logits, nullptr, nullptr,
                                     s, zero, zero_n);
}

hipError_t moe_launch_route_balance(const void *x, int dt, const float *Wg, int64_t T, int d,
                                    int E, int k, int32_t *idx, float *gw, double *part_p,
                                    int32_t *part_c, float *f, float *P, float *laux,
                                    hipStream_t s) {
    hipError_t err = launch_router_impl<true>(x, dt, Wg, T, d, E, k, idx, gw, nullptr, part_p,
                                              part_c, s);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(moe::balance_reduce_kernel, dim3(1), dim3(1024), 0, s, part_p, part_c,
                       (int)moe_router_blocks(T), T, E, k, f, P, laux);
    return hipGetLastError();
}
