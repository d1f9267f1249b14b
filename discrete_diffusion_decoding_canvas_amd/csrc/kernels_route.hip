// MoE routing and token permutation (gfx950).
//
// The decoder's mixture-of-experts FFN (DiffusionGemma technical-report
// summary, Experiment: a small number of active experts among many): router
// softmax over the experts, top-k with gates renormalised over the k chosen,
// then the (token, slot) entries grouped by expert for the grouped GEMMs.
//
// Top-k: one wave per token.  The logits go to LDS and every lane ranks its
// own logits against all of them (rank = number of larger logits plus equal
// ones with a lower expert id), so the k winners land at their rank in one
// pass with no serial reduction chain.  Router logits may arrive as several
// split-K partial sums; they are added here in a fixed order.
//
// Permutation: per-expert counts with LDS integer atomics, one exclusive scan
// (of the counts rounded up to the row padding), then each entry takes the next
// free row of its expert.  The order of rows
// inside an expert is not fixed, but every expert-GEMM output row depends only
// on its own input row, so the results are bit-identical across runs.
#include "kernels.h"

namespace dg {

constexpr int kMaxExperts = 256;

// Top-k of token t by wave w of the block (no block-level synchronisation:
// only wave-level LDS use).
DG_DEV void topk_token(const float* __restrict__ logits, int nsplit, int M, int E, int k, int t,
                       int32_t* __restrict__ idx, float* __restrict__ gates,
                       float (*lg)[kMaxExperts], float (*sv)[16]) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int e = lane; e < E; e += 64) {
        float part[kMaxRouterSplit];
#pragma unroll
        for (int sp = 0; sp < kMaxRouterSplit; ++sp)   // all loads in flight together
            part[sp] = sp < nsplit ? logits[((int64_t)sp * M + t) * E + e] : 0.f;
        float v = 0.f;
#pragma unroll
        for (int sp = 0; sp < kMaxRouterSplit; ++sp) v += part[sp];   // fixed order
        lg[w][e] = v;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    for (int e = lane; e < E; e += 64) {
        const float v = lg[w][e];
        int rank = 0;
        const float4* row = reinterpret_cast<const float4*>(lg[w]);
        for (int j4 = 0; j4 < (E >> 2); ++j4) {   // E is a multiple of 4 (checked by the launcher)
            const float4 u = row[j4];
            const int j = 4 * j4;
            rank += (u.x > v) || (u.x == v && j < e);
            rank += (u.y > v) || (u.y == v && j + 1 < e);
            rank += (u.z > v) || (u.z == v && j + 2 < e);
            rank += (u.w > v) || (u.w == v && j + 3 < e);
        }
        if (rank < k) {
            idx[(int64_t)t * k + rank] = e;
            sv[w][rank] = v;
        }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (lane < k) {
        const float mx = sv[w][0];
        float s = 0.f;
        for (int j = 0; j < k; ++j) s += expf(sv[w][j] - mx);
        gates[(int64_t)t * k + lane] = expf(sv[w][lane] - mx) / s;
    }
}

__global__ __launch_bounds__(256) void k_router_topk(const float* __restrict__ logits, int nsplit,
                                                     int M, int E, int k,
                                                     int32_t* __restrict__ idx,
                                                     float* __restrict__ gates) {
    __shared__ __attribute__((aligned(16))) float lg[4][kMaxExperts];
    __shared__ float sv[4][16];
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= M) return;
    topk_token(logits, nsplit, M, E, k, t, idx, gates, lg, sv);
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

// From per-expert entry counts cnt[0..E): padded row offsets (to global
// `offsets` and LDS off), the expert-GEMM work items ((expert, first row) for
// every kMoeRows-row chunk, experts in order) and -1 in perm_token for the
// padding rows.  woff is LDS scratch of E + 1 entries.
DG_DEV void route_offsets(const int32_t* cnt, int E, int pad, int32_t* off, int32_t* woff,
                          int32_t* __restrict__ offsets, int32_t* __restrict__ perm_token,
                          int2* __restrict__ items, int32_t* __restrict__ count) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) off[e] = round_up(cnt[e], pad);
    __syncthreads();
    wave0_exclusive_scan(off, E);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        woff[e] = (off[e + 1] - off[e] + kMoeRows - 1) / kMoeRows;
    __syncthreads();
    wave0_exclusive_scan(woff, E);
    __syncthreads();
    for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = off[e];
    if (threadIdx.x == 0) *count = woff[E];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        for (int i = woff[e]; i < woff[e + 1]; ++i) items[i] = make_int2(e, (i - woff[e]) * kMoeRows);
        for (int j = off[e] + cnt[e]; j < off[e + 1]; ++j) perm_token[j] = -1;
    }
}

// The permutation of n <= kPermSmall entries by one block: counts, offsets,
// work items, and every entry's row (the next free row of its expert).
constexpr int kPermSmall = 8192;

DG_DEV void permute_block(const int32_t* __restrict__ idx, int n, int E, int k, int pad,
                          int32_t* __restrict__ offsets, int32_t* __restrict__ perm_token,
                          int32_t* __restrict__ inv, int2* __restrict__ work,
                          int32_t* __restrict__ work_count) {
    __shared__ int32_t cnt[kMaxExperts];
    __shared__ int32_t off[kMaxExperts + 1];
    __shared__ int32_t woff[kMaxExperts + 1];
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    for (int f = threadIdx.x; f < n; f += blockDim.x) atomicAdd(&cnt[idx[f]], 1);
    __syncthreads();
    route_offsets(cnt, E, pad, off, woff, offsets, perm_token, work, work_count);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    for (int f = threadIdx.x; f < n; f += blockDim.x) {
        const int e = idx[f];
        const int pos = off[e] + atomicAdd(&cnt[e], 1);
        perm_token[pos] = f / k;
        inv[f] = pos;
    }
}

// Top-k and permutation in one launch (M * k <= kPermSmall): each block ranks
// its tokens; the last block to finish (a ticket counter, reset by that block
// for the next launch) permutes all entries.
__global__ __launch_bounds__(256) void k_router_route(const float* __restrict__ logits, int nsplit,
                                                      int M, int E, int k, int pad,
                                                      int32_t* __restrict__ idx,
                                                      float* __restrict__ gates,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ perm_token,
                                                      int32_t* __restrict__ inv,
                                                      int2* __restrict__ work,
                                                      int32_t* __restrict__ work_count,
                                                      uint32_t* __restrict__ ticket) {
    __shared__ __attribute__((aligned(16))) float lg[4][kMaxExperts];
    __shared__ float sv[4][16];
    __shared__ bool last;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t < M) topk_token(logits, nsplit, M, E, k, t, idx, gates, lg, sv);
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();                                   // this block's idx before the ticket
        last = atomicAdd(ticket, 1u) == gridDim.x - 1;
    }
    __syncthreads();
    if (!last) return;
    __threadfence();                                       // every block's idx visible here
    permute_block(idx, M * k, E, k, pad, offsets, perm_token, inv, work, work_count);
    if (threadIdx.x == 0) *ticket = 0u;
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
                                                  int2* __restrict__ work,
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
    route_offsets(tot, E, pad, off, woff, offsets, perm_token, work, work_count);
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
        kMoeRows % pad)
        return hipErrorInvalidValue;
    const int n = M * k;
    if (work.max_items < (n + kMoeRows - 1) / kMoeRows + E) return hipErrorInvalidValue;
    if (n <= kPermSmall) {
        k_router_route<<<(M + 3) / 4, 256, 0, s>>>(logits, nsplit, M, E, k, pad, idx, gates,
                                                   offsets, perm_token, inv, work.items,
                                                   work.count, work.ticket);
    } else {
        k_router_topk<<<(M + 3) / 4, 256, 0, s>>>(logits, nsplit, M, E, k, idx, gates);
        const int n_chunks = (n + kPermChunk - 1) / kPermChunk;
        k_moe_count<<<n_chunks, 256, 0, s>>>(idx, n, E, counts);
        k_moe_scan<<<1, 256, 0, s>>>(counts, n_chunks, E, pad, base, offsets, perm_token,
                                     work.items, work.count);
        k_moe_scatter<<<n_chunks, 256, 0, s>>>(idx, n, E, k, base, perm_token, inv);
    }
    return hipGetLastError();
}

}  // namespace dg
