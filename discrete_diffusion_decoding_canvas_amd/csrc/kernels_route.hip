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

__global__ __launch_bounds__(256) void k_router_topk(const float* __restrict__ logits, int nsplit,
                                                     int M, int E, int k,
                                                     int32_t* __restrict__ idx,
                                                     float* __restrict__ gates) {
    __shared__ __attribute__((aligned(16))) float lg[4][kMaxExperts];
    __shared__ float sv[4][16];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + w;
    if (t >= M) return;   // no block-level synchronisation below: only wave-level LDS use
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

// One workgroup for up to kPermSmall entries: counts, scan, row assignment.
constexpr int kPermSmall = 8192;

// Work items of the expert GEMMs: (expert, first row) for every kMoeRows-row
// chunk of every expert that received entries, experts in order.  off holds the
// (padded) row offsets; woff[e] is the first item of expert e.
DG_DEV void emit_work(const int32_t* off, int E, int32_t* woff, int2* items, int32_t* count) {
    if (threadIdx.x == 0) {
        int run = 0;
        for (int e = 0; e < E; ++e) {
            woff[e] = run;
            run += (off[e + 1] - off[e] + kMoeRows - 1) / kMoeRows;
        }
        woff[E] = run;
        *count = run;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        for (int i = woff[e]; i < woff[e + 1]; ++i) items[i] = make_int2(e, (i - woff[e]) * kMoeRows);
}

// Every expert's rows start at a multiple of pad (16 for the MFMA expert GEMMs,
// whose activation tiles are 16 rows of one expert; 1 otherwise); the rows past
// an expert's entries up to the next multiple are padding, perm_token = -1.
DG_DEV int round_up(int v, int pad) { return (v + pad - 1) / pad * pad; }

__global__ __launch_bounds__(1024) void k_moe_permute_small(const int32_t* __restrict__ idx, int n,
                                                            int E, int k, int pad,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ perm_token,
                                                            int32_t* __restrict__ inv,
                                                            int2* __restrict__ work,
                                                            int32_t* __restrict__ work_count) {
    __shared__ int32_t cnt[kMaxExperts];
    __shared__ int32_t off[kMaxExperts + 1];
    __shared__ int32_t woff[kMaxExperts + 1];
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    for (int f = threadIdx.x; f < n; f += blockDim.x) atomicAdd(&cnt[idx[f]], 1);
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int e = 0; e < E; ++e) {
            off[e] = run;
            run += round_up(cnt[e], pad);
        }
        off[E] = run;
    }
    __syncthreads();
    emit_work(off, E, woff, work, work_count);
    __syncthreads();
    for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = off[e];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        for (int j = off[e] + cnt[e]; j < off[e + 1]; ++j) perm_token[j] = -1;
        cnt[e] = 0;
    }
    __syncthreads();
    for (int f = threadIdx.x; f < n; f += blockDim.x) {
        const int e = idx[f];
        const int pos = off[e] + atomicAdd(&cnt[e], 1);
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
    if (threadIdx.x == 0) {
        int run = 0;
        for (int e = 0; e < E; ++e) {
            off[e] = run;
            run += round_up(tot[e], pad);
        }
        off[E] = run;
    }
    __syncthreads();
    emit_work(off, E, woff, work, work_count);
    __syncthreads();
    for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = off[e];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        for (int j = off[e] + tot[e]; j < off[e + 1]; ++j) perm_token[j] = -1;
        for (int c = 0; c < n_chunks; ++c) base[(int64_t)c * E + e] += off[e];
    }
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
    k_router_topk<<<(M + 3) / 4, 256, 0, s>>>(logits, nsplit, M, E, k, idx, gates);
    if (n <= kPermSmall) {
        k_moe_permute_small<<<1, 1024, 0, s>>>(idx, n, E, k, pad, offsets, perm_token, inv,
                                                work.items, work.count);
    } else {
        const int n_chunks = (n + kPermChunk - 1) / kPermChunk;
        k_moe_count<<<n_chunks, 256, 0, s>>>(idx, n, E, counts);
        k_moe_scan<<<1, 256, 0, s>>>(counts, n_chunks, E, pad, base, offsets, perm_token,
                                     work.items, work.count);
        k_moe_scatter<<<n_chunks, 256, 0, s>>>(idx, n, E, k, base, perm_token, inv);
    }
    return hipGetLastError();
}

}  // namespace dg
