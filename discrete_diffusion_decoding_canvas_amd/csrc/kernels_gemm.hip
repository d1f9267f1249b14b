// Dense and expert (grouped) GEMMs for gfx950.
//
// Decoder projections (DiffusionGemma technical-report summary, Method:
// decoder with shared weights; Experiment: mixture-of-experts transformer):
// QKV / output / router projections of the canvas, and the per-expert SwiGLU
// FFN over the tokens routed to each expert.
//
// At 256 canvas tokens these GEMMs stream weights that are read once per pass,
// so the design goal is HBM streaming, not MFMA occupancy:
//   * weights are pre-packed at load time into the exact MFMA B-operand lane
//     order, so every weight load is one coalesced 16-byte load per lane
//     (1 KiB per wave, contiguous) straight into registers;
//   * the waves of a workgroup split the reduction (K) dimension, so a
//     workgroup covers a narrow 64-column slab with many bytes in flight, and
//     the partial tiles are summed once through LDS in a fixed order;
//   * each wave keeps kPrefetch k-steps of operands in flight in registers
//     (a rolling buffer), which hides HBM latency without LDS staging;
//   * tokens sit on the 16-row MFMA side (v_mfma_f32_16x16x32_bf16, or
//     v_mfma_f32_16x16x32_fp8_fp8 for e4m3 experts), 32-row chunks per pass;
//   * the SwiGLU of the first expert GEMM runs in the epilogue (gate and up
//     columns are interleaved per 16-column group at pack time);
//   * narrow GEMMs (the router, N = E) split K across workgroups as well and
//     leave the partial sums to their consumer, which adds them in order.
#include "kernels.h"

namespace dg {

#ifndef DG_GEMM_WAVES
#define DG_GEMM_WAVES 4      // measured best on the 26B-class pass (vs 8 waves, 2-6 stages)
#endif
#ifndef DG_GEMM_PREFETCH
#define DG_GEMM_PREFETCH 6
#endif

constexpr int kTileM = 32;   // rows per chunk (2 MFMA row tiles)
constexpr int kTileN = 64;   // weight columns per workgroup (4 MFMA column groups)
constexpr int kMT = 2;
constexpr int kNT = 4;
constexpr int kWaves = DG_GEMM_WAVES;
constexpr int kThreads = 64 * kWaves;
constexpr int kPrefetch = DG_GEMM_PREFETCH;

union Frag16 {
    uint4 u;
    bf16x8_t b;
    struct { long lo, hi; } l;
};

DG_DEV uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
DG_DEV long ld8(const void* p) { return *reinterpret_cast<const long*>(p); }

struct Stage {
    Frag16 a[kMT];
    Frag16 b[kNT];
};

// ------------------------------------------------------------------ main loop
// A rows given per lane (row pointers for the two row tiles), B packed
// [group][KB][64 lanes][16 bytes] starting at the workgroup's first column group.
// bf16: one k-step = 32 elements; fp8: one k-step = 64 codes (two MFMAs).
template <bool FP8>
DG_DEV void load_stage(Stage& st, const uint8_t* a0, const uint8_t* a1, const uint8_t* bgrp,
                       size_t gstride, int kb, int lane) {
    const int koff = 8 * (lane >> 4);
    if (FP8) {
        st.a[0].l.lo = ld8(a0 + kb * 64 + koff);
        st.a[0].l.hi = ld8(a0 + kb * 64 + 32 + koff);
        st.a[1].l.lo = ld8(a1 + kb * 64 + koff);
        st.a[1].l.hi = ld8(a1 + kb * 64 + 32 + koff);
    } else {
        st.a[0].u = ld16(a0 + (kb * 32 + koff) * 2);
        st.a[1].u = ld16(a1 + (kb * 32 + koff) * 2);
    }
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
        st.b[nt].u = ld16(bgrp + nt * gstride + ((size_t)kb * 64 + lane) * 16);
}

template <bool FP8>
DG_DEV void mma_stage(const Stage& st, f32x4_t (&acc)[kMT][kNT]) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            if (FP8) {
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
                    st.a[mt].l.lo, st.b[nt].l.lo, acc[mt][nt], 0, 0, 0);
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
                    st.a[mt].l.hi, st.b[nt].l.hi, acc[mt][nt], 0, 0, 0);
            } else {
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(st.a[mt].b, st.b[nt].b,
                                                                      acc[mt][nt], 0, 0, 0);
            }
        }
}

template <bool FP8>
DG_DEV void mainloop(const uint8_t* a0, const uint8_t* a1, const uint8_t* bgrp, int KB,
                     int kb_begin, int kb_end, f32x4_t (&acc)[kMT][kNT]) {
    const int lane = threadIdx.x & 63;
    const size_t gstride = (size_t)KB * 1024;   // bytes per packed column group
    Stage buf[kPrefetch];
#pragma unroll
    for (int s = 0; s < kPrefetch - 1; ++s)
        if (kb_begin + s < kb_end) load_stage<FP8>(buf[s], a0, a1, bgrp, gstride, kb_begin + s, lane);
    for (int kb = kb_begin; kb < kb_end; kb += kPrefetch) {
#pragma unroll
        for (int u = 0; u < kPrefetch; ++u) {
            const int k = kb + u;
            if (k < kb_end) {
                const int kn = k + kPrefetch - 1;
                if (kn < kb_end)
                    load_stage<FP8>(buf[(u + kPrefetch - 1) % kPrefetch], a0, a1, bgrp, gstride,
                                    kn, lane);
                mma_stage<FP8>(buf[u], acc);
            }
        }
    }
}

// Sum the waves' partial tiles, in wave order, into red[0][r][c] (r < 32, c < 64).
DG_DEV void reduce_waves(f32x4_t (&acc)[kMT][kNT], float (*red)[kTileM][kTileN]) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                red[w][16 * mt + 4 * (lane >> 4) + j][16 * nt + (lane & 15)] = acc[mt][nt][j];
    __syncthreads();
    for (int e = threadIdx.x; e < kTileM * kTileN; e += kThreads) {
        const int r = e >> 6, c = e & 63;
        float v = red[0][r][c];
#pragma unroll
        for (int i = 1; i < kWaves; ++i) v += red[i][r][c];
        red[0][r][c] = v;
    }
    __syncthreads();
}

DG_DEV void split_range(int KB, int parts, int idx, int& b, int& e) {
    const int per = KB / parts, rem = KB % parts;
    b = idx * per + (idx < rem ? idx : rem);
    e = b + per + (idx < rem ? 1 : 0);
}

DG_DEV void zero_acc(f32x4_t (&acc)[kMT][kNT]) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// ------------------------------------------------------------------ dense bf16 GEMM
// grid (N / 64, ceil(M / 32), ksplit).  With ksplit > 1 workgroup z sums its
// share of K and stores the partial tile at C + z * M * ldc (store epilogue).
template <int EPI>
__global__ __launch_bounds__(kThreads) void k_gemm_bf16(const bf16_t* __restrict__ A, int lda,
                                                        int M, const bf16_t* __restrict__ Bp,
                                                        int K, int N, float* __restrict__ C,
                                                        int ldc) {
    __shared__ float red[kWaves][kTileM][kTileN];
    const int lane = threadIdx.x & 63;
    const int n0 = blockIdx.x * kTileN;
    const int m0 = blockIdx.y * kTileM;
    const int KB = K >> 5;
    f32x4_t acc[kMT][kNT];
    zero_acc(acc);
    int r0 = m0 + (lane & 15), r1 = m0 + 16 + (lane & 15);
    r0 = r0 < M ? r0 : M - 1;
    r1 = r1 < M ? r1 : M - 1;
    int zb, ze, kb0, kb1;
    split_range(KB, gridDim.z, blockIdx.z, zb, ze);
    split_range(ze - zb, kWaves, threadIdx.x >> 6, kb0, kb1);
    mainloop<false>((const uint8_t*)(A + (size_t)r0 * lda), (const uint8_t*)(A + (size_t)r1 * lda),
                    (const uint8_t*)(Bp + (size_t)(n0 >> 4) * KB * 512), KB, zb + kb0, zb + kb1,
                    acc);
    reduce_waves(acc, red);
    float* Cz = C + (size_t)blockIdx.z * M * ldc;
    for (int e = threadIdx.x; e < kTileM * kTileN; e += kThreads) {
        const int r = e >> 6, c = e & 63;
        const int m = m0 + r, n = n0 + c;
        if (m >= M) continue;
        const float v = red[0][r][c];
        if (EPI == kEpiStoreF32) Cz[(size_t)m * ldc + n] = v;
        else Cz[(size_t)m * ldc + n] += v;
    }
}

// ------------------------------------------------------------------ dense f32 GEMM (VALU)
// 64x64 tile, 256 threads x (4x4) outputs, K steps of 16 through LDS.
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ A, int lda, int M,
                                                  const float* __restrict__ B, int K, int N,
                                                  float* __restrict__ C, int ldc) {
    __shared__ float As[16][65];
    __shared__ float Bs[16][64];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += 16) {
        for (int e = threadIdx.x; e < 64 * 16; e += 256) {
            const int r = e >> 4, kk = e & 15;
            const int m = m0 + r, k = k0 + kk;
            As[kk][r] = (m < M && k < K) ? A[(size_t)m * lda + k] : 0.f;
            const int kk2 = e >> 6, c = e & 63;
            const int n = n0 + c, k2 = k0 + kk2;
            Bs[kk2][c] = (n < N && k2 < K) ? B[(size_t)k2 * N + n] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
            if (m < M && n < N) {
                if (EPI == kEpiStoreF32) C[(size_t)m * ldc + n] = acc[i][j];
                else C[(size_t)m * ldc + n] += acc[i][j];
            }
        }
}

// ------------------------------------------------------------------ expert GEMM 1 (MFMA)
// grid (2F / 64 column slabs, work items): one workgroup per (slab, expert
// 32-row chunk), so heavily loaded experts spread over many workgroups.
// Weight slab columns are [g_j | u_j | g_j+1 | u_j+1] (16 each).
template <bool FP8>
__global__ __launch_bounds__(kThreads) void k_moe1_mfma(const void* __restrict__ X, int d, int F,
                                                        const int32_t* __restrict__ perm_token,
                                                        const int32_t* __restrict__ offsets,
                                                        const int2* __restrict__ work,
                                                        const int32_t* __restrict__ work_count,
                                                        const void* __restrict__ W1,
                                                        const float* __restrict__ s1,
                                                        void* __restrict__ H) {
    __shared__ float red[kWaves][kTileM][kTileN];
    if ((int)blockIdx.y >= *work_count) return;
    const int2 item = work[blockIdx.y];
    const int e = item.x;
    const int off = offsets[e];
    const int n_e = min(offsets[e + 1] - off, item.y + kMoeRows);
    const int lane = threadIdx.x & 63;
    const int n0 = blockIdx.x * kTileN;          // weight column (interleaved)
    const int N1 = 2 * F;
    const int KB = FP8 ? (d >> 6) : (d >> 5);
    int kb0, kb1;
    split_range(KB, kWaves, threadIdx.x >> 6, kb0, kb1);
    const size_t gsize = (size_t)KB * 1024;      // bytes per packed column group
    const uint8_t* bgrp = (const uint8_t*)W1 + (size_t)e * (N1 >> 4) * gsize +
                          (size_t)(n0 >> 4) * gsize;
    const size_t xrow = FP8 ? (size_t)d : (size_t)d * 2;
    for (int mc = item.y; mc < n_e; mc += kTileM) {   // one chunk: n_e clipped above
        f32x4_t acc[kMT][kNT];
        zero_acc(acc);
        int e0 = mc + (lane & 15), e1 = mc + 16 + (lane & 15);
        e0 = off + (e0 < n_e ? e0 : n_e - 1);
        e1 = off + (e1 < n_e ? e1 : n_e - 1);
        const int64_t t0 = perm_token[e0], t1 = perm_token[e1];
        mainloop<FP8>((const uint8_t*)X + t0 * xrow, (const uint8_t*)X + t1 * xrow, bgrp, KB, kb0,
                      kb1, acc);
        reduce_waves(acc, red);
        const int h0 = n0 >> 1;
        for (int q = threadIdx.x; q < kTileM * (kTileN / 2); q += kThreads) {
            const int r = q >> 5, hc = q & 31;
            if (mc + r >= n_e) continue;
            const int cg = ((hc >> 4) << 5) + (hc & 15);
            float g = red[0][r][cg], u = red[0][r][cg + 16];
            if (FP8) {
                g *= s1[(size_t)e * N1 + n0 + cg];
                u *= s1[(size_t)e * N1 + n0 + cg + 16];
            }
            const float hv = g / (1.0f + expf(-g)) * u;
            const size_t o = (size_t)(off + mc + r) * F + h0 + hc;
            if (FP8) ((uint8_t*)H)[o] = (uint8_t)f32_to_e4m3(hv);
            else ((bf16_t*)H)[o] = f32_to_bf16(hv);
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ expert GEMM 2 (MFMA)
// grid (d / 64 column slabs, work items): Y[entry, n] = H[entry, :] Wd_e[:, n].
template <bool FP8>
__global__ __launch_bounds__(kThreads) void k_moe2_mfma(const void* __restrict__ H, int d, int F,
                                                        const int32_t* __restrict__ offsets,
                                                        const int2* __restrict__ work,
                                                        const int32_t* __restrict__ work_count,
                                                        const void* __restrict__ W2,
                                                        const float* __restrict__ s2,
                                                        float* __restrict__ Y) {
    __shared__ float red[kWaves][kTileM][kTileN];
    if ((int)blockIdx.y >= *work_count) return;
    const int2 item = work[blockIdx.y];
    const int e = item.x;
    const int off = offsets[e];
    const int n_e = min(offsets[e + 1] - off, item.y + kMoeRows);
    const int lane = threadIdx.x & 63;
    const int n0 = blockIdx.x * kTileN;
    const int KB = FP8 ? (F >> 6) : (F >> 5);
    int kb0, kb1;
    split_range(KB, kWaves, threadIdx.x >> 6, kb0, kb1);
    const size_t gsize = (size_t)KB * 1024;
    const uint8_t* bgrp = (const uint8_t*)W2 + (size_t)e * (d >> 4) * gsize +
                          (size_t)(n0 >> 4) * gsize;
    const size_t hrow = FP8 ? (size_t)F : (size_t)F * 2;
    for (int mc = item.y; mc < n_e; mc += kTileM) {   // one chunk: n_e clipped above
        f32x4_t acc[kMT][kNT];
        zero_acc(acc);
        int e0 = mc + (lane & 15), e1 = mc + 16 + (lane & 15);
        e0 = off + (e0 < n_e ? e0 : n_e - 1);
        e1 = off + (e1 < n_e ? e1 : n_e - 1);
        mainloop<FP8>((const uint8_t*)H + (size_t)e0 * hrow, (const uint8_t*)H + (size_t)e1 * hrow,
                      bgrp, KB, kb0, kb1, acc);
        reduce_waves(acc, red);
        for (int q = threadIdx.x; q < kTileM * kTileN; q += kThreads) {
            const int r = q >> 6, c = q & 63;
            if (mc + r >= n_e) continue;
            float v = red[0][r][c];
            if (FP8) v *= s2[(size_t)e * d + n0 + c];
            Y[(size_t)(off + mc + r) * d + n0 + c] = v;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ expert GEMMs (f32, VALU)
// One thread per (entry, hidden column); the entry's expert found by binary search.
DG_DEV int expert_of(const int32_t* offsets, int E, int entry) {
    int lo = 0, hi = E;   // offsets[lo] <= entry < offsets[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (offsets[mid] <= entry) lo = mid; else hi = mid;
    }
    return lo;
}

__global__ void k_moe1_f32(const float* __restrict__ X, int d, int F,
                           const int32_t* __restrict__ perm_token,
                           const int32_t* __restrict__ offsets, int E, int n_entries,
                           const float* __restrict__ Wg, const float* __restrict__ Wu,
                           float* __restrict__ H) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)n_entries * F) return;
    const int entry = (int)(idx / F), f = (int)(idx % F);
    const int e = expert_of(offsets, E, entry);
    const float* x = X + (int64_t)perm_token[entry] * d;
    const float* wg = Wg + (int64_t)e * d * F + f;
    const float* wu = Wu + (int64_t)e * d * F + f;
    float g = 0.f, u = 0.f;
    for (int k = 0; k < d; ++k) {
        g = fmaf(x[k], wg[(int64_t)k * F], g);
        u = fmaf(x[k], wu[(int64_t)k * F], u);
    }
    H[idx] = g / (1.0f + expf(-g)) * u;
}

__global__ void k_moe2_f32(const float* __restrict__ H, int d, int F,
                           const int32_t* __restrict__ offsets, int E, int n_entries,
                           const float* __restrict__ Wd, float* __restrict__ Y) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)n_entries * d) return;
    const int entry = (int)(idx / d), c = (int)(idx % d);
    const int e = expert_of(offsets, E, entry);
    const float* h = H + (int64_t)entry * F;
    const float* w = Wd + (int64_t)e * F * d + c;
    float y = 0.f;
    for (int f = 0; f < F; ++f) y = fmaf(h[f], w[(int64_t)f * d], y);
    Y[idx] = y;
}

// ================================================================== launchers
hipError_t launch_gemm(int dtype, int epi, const void* A, int lda, int M, const void* B, int K,
                       int N, float* C, int ldc, hipStream_t s, int ksplit) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (dtype == kF32) {
        if (ksplit != 1) return hipErrorInvalidValue;
        dim3 grid((N + 63) / 64, (M + 63) / 64);
        if (epi == kEpiStoreF32)
            k_gemm_f32<kEpiStoreF32><<<grid, 256, 0, s>>>((const float*)A, lda, M,
                                                          (const float*)B, K, N, C, ldc);
        else
            k_gemm_f32<kEpiAddF32><<<grid, 256, 0, s>>>((const float*)A, lda, M,
                                                        (const float*)B, K, N, C, ldc);
    } else {
        if ((K & 31) || (N % kTileN) || ksplit < 1 || (ksplit > 1 && epi != kEpiStoreF32))
            return hipErrorInvalidValue;
        dim3 grid(N / kTileN, (M + kTileM - 1) / kTileM, ksplit);
        if (epi == kEpiStoreF32)
            k_gemm_bf16<kEpiStoreF32><<<grid, kThreads, 0, s>>>((const bf16_t*)A, lda, M,
                                                                (const bf16_t*)B, K, N, C, ldc);
        else
            k_gemm_bf16<kEpiAddF32><<<grid, kThreads, 0, s>>>((const bf16_t*)A, lda, M,
                                                              (const bf16_t*)B, K, N, C, ldc);
    }
    return hipGetLastError();
}

hipError_t launch_moe_gemm1(int dtype, const ExpertWeights& w, const void* X,
                            const int32_t* perm_token, const int32_t* offsets, int E, int d,
                            int F, int max_rows, const MoeWork& work, void* H, hipStream_t s) {
    if (max_rows <= 0) return hipSuccess;
    if (dtype == kF32) {
        int64_t total = (int64_t)max_rows * F;
        k_moe1_f32<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
            (const float*)X, d, F, perm_token, offsets, E, max_rows, (const float*)w.w1,
            (const float*)w.wu, (float*)H);
    } else {
        dim3 grid((2 * F) / kTileN, work.max_items);
        if (dtype == kFP8)
            k_moe1_mfma<true><<<grid, kThreads, 0, s>>>(X, d, F, perm_token, offsets, work.items,
                                                        work.count, w.w1, w.s1, H);
        else
            k_moe1_mfma<false><<<grid, kThreads, 0, s>>>(X, d, F, perm_token, offsets, work.items,
                                                         work.count, w.w1, w.s1, H);
    }
    return hipGetLastError();
}

hipError_t launch_moe_gemm2(int dtype, const ExpertWeights& w, const void* H,
                            const int32_t* offsets, int E, int d, int F, int max_rows,
                            const MoeWork& work, float* Y, hipStream_t s) {
    if (max_rows <= 0) return hipSuccess;
    if (dtype == kF32) {
        int64_t total = (int64_t)max_rows * d;
        k_moe2_f32<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
            (const float*)H, d, F, offsets, E, max_rows, (const float*)w.w2, Y);
    } else {
        dim3 grid(d / kTileN, work.max_items);
        if (dtype == kFP8)
            k_moe2_mfma<true><<<grid, kThreads, 0, s>>>(H, d, F, offsets, work.items, work.count,
                                                        w.w2, w.s2, Y);
        else
            k_moe2_mfma<false><<<grid, kThreads, 0, s>>>(H, d, F, offsets, work.items, work.count,
                                                         w.w2, w.s2, Y);
    }
    return hipGetLastError();
}

}  // namespace dg
