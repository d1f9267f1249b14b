// MoE routing and token permutation (gfx950).
//
// The decoder's mixture-of-experts FFN (DiffusionGemma technical-report
// summary, Experiment: a small number of active experts among many): router
// softmax over the experts, top-k with gates renormalised over the k chosen,
// then the (token, slot) entries grouped by expert for the grouped GEMMs.
//
// Top-k: one wave per token, k rounds of a DPP wave maximum (the ranking:
// logit descending, ties to the lower expert id).  Router logits may arrive as
// several split-K partial sums; they are added here in a fixed order.
//
// Permutation: per-expert counts with LDS integer atomics, one exclusive scan
// (of the counts rounded up to the row padding), then each entry takes the next
// free row of its expert.  The order of rows
// inside an expert is not fixed, but every expert-GEMM output row depends only
// on its own input row, so the results are bit-identical across runs.
#include "kernels.h"

namespace dg {

constexpr int kMaxExperts = 256;

// One step of a DPP maximum: lane i takes max(x_i, x of the lane CTRL selects);
// lanes without a source keep x_i (old = -inf).
template <int CTRL, int ROW_MASK>
DG_DEV float dpp_max_step(float x) {
    const int y = __builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(x), CTRL,
                                              ROW_MASK, 0xf, false);
    return fmaxf(x, __int_as_float(y));
}

// Maximum over the 64 lanes, uniform: prefix maxima within each 16-lane row (row
// shifts by 1, 2, 4, 8), then the rows' last lanes broadcast into the next rows
// (row_bcast:15, row_bcast:31); lane 63 ends with the wave's maximum.
DG_DEV float wave_max_dpp(float x) {
    x = dpp_max_step<0x111, 0xf>(x);   // row_shr:1
    x = dpp_max_step<0x112, 0xf>(x);   // row_shr:2
    x = dpp_max_step<0x114, 0xf>(x);   // row_shr:4
    x = dpp_max_step<0x118, 0xf>(x);   // row_shr:8
    x = dpp_max_step<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
    x = dpp_max_step<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// Top-k of token t by one wave (no block-level synchronisation), written to the
// token's k slots idx[0..k) and gates[0..k).  Lane l holds the summed logits of
// experts l, 64 + l, ...; k rounds each take the wave maximum and the lowest
// expert id holding it (ballot), which is the ranking (logit descending, ties to
// the lower id).
DG_DEV void topk_token(const float* __restrict__ logits, int nsplit, int M, int E, int k, int t,
                       int32_t* __restrict__ idx, float* __restrict__ gates) {
    const int lane = threadIdx.x & 63;
    constexpr int NQ = kMaxExperts / 64;
    float v[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int e = 64 * q + lane;
        float part[kMaxRouterSplit];
#pragma unroll
        for (int sp = 0; sp < kMaxRouterSplit; ++sp)   // all loads in flight together
            part[sp] = (sp < nsplit && e < E) ? logits[((int64_t)sp * M + t) * E + e] : 0.f;
        float sum = 0.f;
#pragma unroll
        for (int sp = 0; sp < kMaxRouterSplit; ++sp) sum += part[sp];   // fixed order
        v[q] = e < E ? sum : -INFINITY;
    }
    float sel[kMaxTopK];
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
        if (r >= k) break;
        float lm = v[0];
#pragma unroll
        for (int q = 1; q < NQ; ++q) lm = fmaxf(lm, v[q]);
        const float m = wave_max_dpp(lm);
        int win = -1;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const uint64_t b = __ballot(v[q] == m);
            if (win < 0 && b) win = 64 * q + __ffsll((long long)b) - 1;
        }
        // Only NaN logits leave no valid winner (fmaxf skips NaN, so m is then
        // NaN or the -inf of a lane past E): take expert 0 so that every id
        // stays in [0, E); the NaN gate reaches the logits statistics.
        if (win < 0 || win >= E) win = 0;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            if (win == 64 * q + lane) v[q] = -INFINITY;
        sel[r] = m;
        if (lane == 0) idx[r] = win;
    }
    if (lane < k) {
        const float mx = sel[0];
        float s = 0.f, mine = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
            if (j >= k) break;
            const float ex = expf(sel[j] - mx);
            s += ex;
            if (j == lane) mine = ex;
        }
        gates[lane] = mine / s;
    }
}

__global__ __launch_bounds__(256) void k_router_topk(const float* __restrict__ logits, int nsplit,
                                                     int M, int E, int k,
                                                     int32_t* __restrict__ idx,
                                                     float* __restrict__ gates) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= M) return;
    topk_token(logits, nsplit, M, E, k, t, idx + (int64_t)t * k, gates + (int64_t)t * k);
}

// Every expert's rows start at a multiple of pad (16 for the MFMA expert GEMMs,
// whose activation tiles are 16 rows of one expert; 1 otherwise); the rows past
// an expert's entries up to the next multiple are padding, perm_token = -1.
DG_DEV int round_up(int v, int pad) { return (v + pad - 1) / pad * pad; }

// In-place exclusive prefix sum of v[0..n), n <= 256, by wave 0 (four values
// per lane, then a shuffle scan across the lanes); v[n] = total.  The caller
// synchronises the block before and after.
DG_DEV void wave0_exclusive_scan(int32_t* v, int n) {
    if (threadIdx.x >= 64) return;
    const int l = threadIdx.x;
    int a[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * l + i;
        a[i] = e < n ? v[e] : 0;
        s += a[i];
    }
    int inc = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(inc, o, 64);
        if (l >= o) inc += u;
    }
    int run = inc - s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * l + i;
        if (e < n) v[e] = run;
        run += a[i];
    }
    if (l == 63) v[n] = inc;
}

// Work items of `rows`-row chunks of every expert, experts in order: (expert,
// first row of the chunk within the expert, the expert's first row, the end of its
// padded rows); their number to *count.  woff is LDS scratch of E + 1 entries.
DG_DEV void route_items(const int32_t* off, int E, int rows, int32_t* woff,
                        int4* __restrict__ items, int32_t* __restrict__ count) {
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        woff[e] = (off[e + 1] - off[e] + rows - 1) / rows;
    __syncthreads();
    wave0_exclusive_scan(woff, E);
    __syncthreads();
    if (threadIdx.x == 0) *count = woff[E];
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        for (int i = woff[e]; i < woff[e + 1]; ++i)
            items[i] = make_int4(e, (i - woff[e]) * rows, off[e], off[e + 1]);
    __syncthreads();   // woff is reused
}

// From per-expert entry counts cnt[0..E): padded row offsets (to global
// `offsets` and LDS off), the work items of the two expert GEMMs
// (kMoeItemRows- and kMoeRows-row chunks) and -1 in perm_token for the padding
// rows.  woff is LDS scratch of E + 1 entries.
DG_DEV void route_offsets(const int32_t* cnt, int E, int pad, int32_t* off, int32_t* woff,
                          int32_t* __restrict__ offsets, int32_t* __restrict__ perm_token,
                          int4* __restrict__ items, int4* __restrict__ items2,
                          int32_t* __restrict__ count) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) off[e] = round_up(cnt[e], pad);
    __syncthreads();
    wave0_exclusive_scan(off, E);
    __syncthreads();
    route_items(off, E, kMoeItemRows, woff, items, count);
    route_items(off, E, kMoeRows, woff, items2, count + 3);
    for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = off[e];
    if (threadIdx.x == 0) {
        count[1] = 0;   // unit counters of the two expert GEMMs that read these items
        count[2] = 0;
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        for (int j = off[e] + cnt[e]; j < off[e + 1]; ++j) perm_token[j] = -1;
}

// The permutation of n <= kPermSmall entries by one block of kPermThreads threads:
// counts, offsets, work items, and every entry's row (the next free row of its
// expert).
constexpr int kPermSmall = 8192;
constexpr int kPermThreads = 1024;

__global__ __launch_bounds__(kPermThreads) void k_moe_permute(
    const int32_t* __restrict__ idx, int n, int E, int k, int pad, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm_token, int32_t* __restrict__ inv, int4* __restrict__ work,
    int4* __restrict__ work2, int32_t* __restrict__ work_count) {
    __shared__ int32_t cnt[kMaxExperts];
    __shared__ int32_t off[kMaxExperts + 1];
    __shared__ int32_t woff[kMaxExperts + 1];
    constexpr int kPer = kPermSmall / kPermThreads;   // entries per thread
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    // each entry's expert and its place among the expert's entries (the counter's
    // old value), kept in registers for the scatter below
    int ex[kPer], lp[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int f = threadIdx.x + kPermThreads * i;
        ex[i] = f < n ? idx[f] : -1;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) lp[i] = ex[i] >= 0 ? atomicAdd(&cnt[ex[i]], 1) : 0;
    __syncthreads();
    route_offsets(cnt, E, pad, off, woff, offsets, perm_token, work, work2, work_count);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int f = threadIdx.x + kPermThreads * i;
        if (ex[i] < 0) continue;
        const int pos = off[ex[i]] + lp[i];
        perm_token[pos] = f / k;
        inv[f] = pos;
    }
}

// Larger batches (prefill chunks): per-chunk counts, one scan, per-chunk assignment.
__global__ __launch_bounds__(256) void k_moe_count(const int32_t* __restrict__ idx, int n,
                                                   int E, int32_t* __restrict__ counts) {
    __shared__ int32_t cnt[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
    __syncthreads();
    const int base = blockIdx.x * kPermChunk;
    for (int i = threadIdx.x; i < kPermChunk; i += 256) {
        const int f = base + i;
        if (f < n) atomicAdd(&cnt[idx[f]], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) counts[(int64_t)blockIdx.x * E + e] = cnt[e];
}

__global__ __launch_bounds__(256) void k_moe_scan(const int32_t* __restrict__ counts,
                                                  int n_chunks, int E, int pad,
                                                  int32_t* __restrict__ base,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ perm_token,
                                                  int4* __restrict__ work,
                                                  int4* __restrict__ work2,
                                                  int32_t* __restrict__ work_count) {
    __shared__ int32_t tot[kMaxExperts];
    __shared__ int32_t off[kMaxExperts + 1];
    __shared__ int32_t woff[kMaxExperts + 1];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int run = 0;
        for (int c = 0; c < n_chunks; ++c) {
            base[(int64_t)c * E + e] = run;
            run += counts[(int64_t)c * E + e];
        }
        tot[e] = run;
    }
    __syncthreads();
    route_offsets(tot, E, pad, off, woff, offsets, perm_token, work, work2, work_count);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        for (int c = 0; c < n_chunks; ++c) base[(int64_t)c * E + e] += off[e];
}

__global__ __launch_bounds__(256) void k_moe_scatter(const int32_t* __restrict__ idx, int n,
                                                     int E, int k,
                                                     const int32_t* __restrict__ base,
                                                     int32_t* __restrict__ perm_token,
                                                     int32_t* __restrict__ inv) {
    __shared__ int32_t fill[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += 256) fill[e] = 0;
    __syncthreads();
    const int c0 = blockIdx.x * kPermChunk;
    for (int i = threadIdx.x; i < kPermChunk; i += 256) {
        const int f = c0 + i;
        if (f >= n) continue;
        const int e = idx[f];
        const int pos = base[(int64_t)blockIdx.x * E + e] + atomicAdd(&fill[e], 1);
        perm_token[pos] = f / k;
        inv[f] = pos;
    }
}

hipError_t launch_router_permute(const float* logits, int nsplit, int M, int E, int k,
                                 int32_t* idx, float* gates, int32_t* counts, int32_t* base,
                                 int32_t* offsets, int32_t* perm_token, int32_t* inv,
                                 const MoeWork& work, int pad, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if (E > kMaxExperts || (E & 3) || k > 16 || nsplit > kMaxRouterSplit || pad < 1 ||
        kMoeItemRows % pad)
        return hipErrorInvalidValue;
    const int n = M * k;
    if (work.max_items < (n + kMoeItemRows - 1) / kMoeItemRows + E ||
        work.max_items2 < (n + kMoeRows - 1) / kMoeRows + E)
        return hipErrorInvalidValue;
    k_router_topk<<<(M + 3) / 4, 256, 0, s>>>(logits, nsplit, M, E, k, idx, gates);
    if (n <= kPermSmall) {
        k_moe_permute<<<1, kPermThreads, 0, s>>>(idx, n, E, k, pad, offsets, perm_token, inv,
                                                 work.items, work.items2, work.count);
    } else {
        const int n_chunks = (n + kPermChunk - 1) / kPermChunk;
        k_moe_count<<<n_chunks, 256, 0, s>>>(idx, n, E, counts);
        k_moe_scan<<<1, 256, 0, s>>>(counts, n_chunks, E, pad, base, offsets, perm_token,
                                     work.items, work.items2, work.count);
        k_moe_scatter<<<n_chunks, 256, 0, s>>>(idx, n, E, k, base, perm_token, inv);
    }
    return hipGetLastError();
}

}  // namespace dg
