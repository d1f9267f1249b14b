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
//     (1 KiB per wave, contiguous);
//   * dense projections: the waves of a workgroup split the reduction (K)
//     dimension over a 32-row x 64-column tile, each wave keeps kPrefetch
//     k-steps of operands in flight in registers (a rolling buffer), and the
//     partial tiles are summed once through LDS in a fixed order; narrow GEMMs
//     (the router, N = E) split K across workgroups as well and leave the
//     partial sums to their consumer, which adds them in order;
//   * expert GEMMs: a workgroup owns all rows of an expert (up to a whole
//     canvas) for a 64-column slab, the weight fragments go through LDS once
//     and feed every wave, so an expert's weights leave HBM once per pass
//     however many tokens it received;
//   * tokens sit on the 16-row MFMA side (v_mfma_f32_16x16x32_bf16, or
//     v_mfma_f32_16x16x32_fp8_fp8 for e4m3 experts);
//   * the SwiGLU of the first expert GEMM runs in the epilogue (gate and up
//     columns are interleaved per 16-column group at pack time).
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

// ------------------------------------------------------------------ expert GEMMs (MFMA)
// One workgroup per (64-column weight slab, work item); a work item is up to
// kMoeRows = 128 rows of one expert, so an expert's weights leave HBM once per
// 128 of its rows (once per pass for all but the most loaded experts).
//
// The workgroup is split by role:
//   * one producer wave streams the weight slab stage by stage (two packed
//     k-steps of the four 16-column groups, 8 KiB per stage) from HBM straight
//     into an LDS ring of kRing stages with global_load_lds (no registers), and
//     keeps kRing - 2 stages in flight: before each barrier it waits only for the
//     stage the consumers read next (a counted vmcnt wait);
//   * kWideConsumers waves own 32 rows each (two MFMA row tiles), read their
//     activation rows (gathered token rows for GEMM 1, the expert's H rows for
//     GEMM 2) straight into registers kWideLead stages ahead, and run the MFMAs
//     against the weight fragments in LDS.  Waves past the expert's rows only
//     keep the barrier count.
// Small workgroups (5 waves, 48 KiB of LDS) let three share a CU, so a CU keeps
// ~96 KiB of weights in flight.  The producer's barrier is the bare s_barrier (a
// workgroup fence there would wait for every load in flight); the consumers'
// is __syncthreads.
//   GEMM 1: H[entry, :F] = silu(x Wg_e) * (x Wu_e).  The slab's columns are
//           [g_j | u_j | g_j+1 | u_j+1] (16 each), so a lane holds the gate and
//           up values of the same (row, column) and the SwiGLU runs in registers.
//   GEMM 2: Y[entry, :d] = H[entry] Wd_e (fp32).
// fp8: e4m3 operands on both sides, per output column scales applied after the
// accumulation.
constexpr int kWideConsumers = 4;
constexpr int kWideThreads = 64 * (kWideConsumers + 1);
constexpr int kRing = 6;                     // LDS stages (8 KiB each)
constexpr int kWideLead = 3;                 // activation stages loaded ahead per consumer wave
static_assert(kMoeRows == 32 * kWideConsumers, "a work item is one row tile per consumer wave");
static_assert(2 * kNT * (kRing - 2) < 64, "vmcnt holds at most 63 loads");

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= n, other counters free.
constexpr int vmcnt_le(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8); }

// Activation fragments of stage st of the k-step range [kb_lo, kb_hi) (clamped).
template <bool FP8>
DG_DEV void wide_load_a(Frag16 (&a)[2][2], const uint8_t* const (&arow)[2], int st, int kb_lo,
                        int kb_hi, int lane) {
    const int koff = 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int kb = min(kb_lo + 2 * st + ks, kb_hi - 1);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            if (FP8) {
                a[ks][mt].l.lo = ld8(arow[mt] + kb * 64 + koff);
                a[ks][mt].l.hi = ld8(arow[mt] + kb * 64 + 32 + koff);
            } else {
                a[ks][mt].u = ld16(arow[mt] + (kb * 32 + koff) * 2);
            }
        }
    }
}

// Both k-steps of a stage for both row tiles, straight-line.  When K has an odd
// number of packed k-steps the last stage's second k-step is multiplied by a
// zeroed activation fragment (keep1 = false).
template <bool FP8>
DG_DEV void wide_mma(f32x4_t (&acc)[kMT][kNT], const Frag16 (&a)[2][2],
                     const uint4 (*bs)[kNT][64], bool keep1, int lane) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        Frag16 fb[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) fb[nt].u = bs[ks][nt][lane];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            Frag16 am = a[ks][mt];
            if (ks == 1) {
                const uint32_t m = keep1 ? 0xffffffffu : 0u;
                am.u = uint4{am.u.x & m, am.u.y & m, am.u.z & m, am.u.w & m};
            }
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                if (FP8) {
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
                        am.l.lo, fb[nt].l.lo, acc[mt][nt], 0, 0, 0);
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
                        am.l.hi, fb[nt].l.hi, acc[mt][nt], 0, 0, 0);
                } else {
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        am.b, fb[nt].b, acc[mt][nt], 0, 0, 0);
                }
            }
        }
    }
}

DG_DEV void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

using WideRing = uint4[kRing][2][kNT][64];       // [stage][k-step][group][lane]

// Producer wave: the four 16-column groups of a 64-column weight slab, k-steps
// [kb_lo, kb_hi) two per stage, HBM -> LDS ring.  slab points at group 0 of the
// slab plus lane * 16 bytes; gsize is the byte stride between groups.
DG_DEV void wide_produce(const uint8_t* slab, size_t gsize, int kb_lo, int kb_hi, WideRing& bsm) {
    const int NS = (kb_hi - kb_lo + 1) >> 1;
    auto issue = [&](int st) {            // stage st (clamped source) into ring slot st % kRing
        const int sc = min(st, NS - 1);
        const int kb0 = min(kb_lo + 2 * sc, kb_hi - 1), kb1 = min(kb_lo + 2 * sc + 1, kb_hi - 1);
        uint4* dst = &bsm[st % kRing][0][0][0];
#pragma unroll
        for (int g = 0; g < kNT; ++g) {
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(slab + g * gsize + (size_t)kb0 * 1024),
                (__attribute__((address_space(3))) void*)(dst + g * 64), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(slab + g * gsize + (size_t)kb1 * 1024),
                (__attribute__((address_space(3))) void*)(dst + (kNT + g) * 64), 16, 0, 0);
        }
    };
    constexpr int kPerStage = 2 * kNT;    // loads per stage
    for (int st = 0; st < kRing - 1; ++st) issue(st);
    __builtin_amdgcn_s_waitcnt(vmcnt_le(kPerStage * (kRing - 2)));   // stage 0 landed
    bare_barrier();
    for (int st = 0; st < NS; ++st) {
        issue(st + kRing - 1);                                       // into the slot of stage st - 1
        __builtin_amdgcn_s_waitcnt(vmcnt_le(kPerStage * (kRing - 2)));   // stage st + 1 landed
        bare_barrier();
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
}

// A consumer wave without rows keeps the workgroup's barrier count.
DG_DEV void wide_idle(int kb_lo, int kb_hi) {
    const int NS = (kb_hi - kb_lo + 1) >> 1;
    __syncthreads();
    for (int st = 0; st < NS; ++st) __syncthreads();
}

// Consumer wave: acc[2 row tiles][4 column groups] over k-steps [kb_lo, kb_hi).
template <bool FP8>
DG_DEV void wide_consume(f32x4_t (&acc)[kMT][kNT], const uint8_t* const (&arow)[2], int kb_lo,
                         int kb_hi, WideRing& bsm, int lane) {
    const int NS = (kb_hi - kb_lo + 1) >> 1;
    constexpr int kSlots = kWideLead + 1;
    zero_acc(acc);
    Frag16 ra[kSlots][2][2];                      // [slot][k-step][row tile]
#pragma unroll
    for (int j = 0; j < kWideLead; ++j) wide_load_a<FP8>(ra[j], arow, min(j, NS - 1), kb_lo, kb_hi, lane);
    __syncthreads();
    // unrolled over several slot cycles: the compiler drains the loads in flight at
    // the loop head, so the head is kept rare
    constexpr int kUnroll = 3 * kSlots;
    for (int s0 = 0; s0 < NS; s0 += kUnroll) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int st = s0 + u;
            if (st >= NS) break;
            wide_load_a<FP8>(ra[(u + kWideLead) % kSlots], arow, min(st + kWideLead, NS - 1), kb_lo,
                             kb_hi, lane);
            __builtin_amdgcn_sched_barrier(0);      // issue the prefetch before the MFMAs
            wide_mma<FP8>(acc, ra[u % kSlots], bsm[st % kRing], kb_lo + 2 * st + 1 < kb_hi, lane);
            __syncthreads();
        }
    }
}

template <bool FP8, int GEMM>
__global__ __launch_bounds__(kWideThreads) void k_moe_wide(
    const void* __restrict__ A, int K, int N, int F, const int32_t* __restrict__ perm_token,
    const int32_t* __restrict__ offsets, const int2* __restrict__ work,
    const int32_t* __restrict__ work_count, const void* __restrict__ W,
    const float* __restrict__ scales, void* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) WideRing bsm;
    if ((int)blockIdx.y >= *work_count) return;
    const int2 item = work[blockIdx.y];
    const int e = item.x;
    const int off = offsets[e];
    const int n_e = min(offsets[e + 1] - off, item.y + kMoeRows);   // rows end (expert-relative)
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = blockIdx.x * kTileN;
    const int KB = FP8 ? (K >> 6) : (K >> 5);     // packed k-steps

    if (w >= kWideConsumers) {
        const size_t gsize = (size_t)KB * 1024;
        wide_produce((const uint8_t*)W + (size_t)e * (N >> 4) * gsize + (size_t)(n0 >> 4) * gsize +
                         (size_t)lane * 16,
                     gsize, 0, KB, bsm);
        return;
    }
    // ---------------- consumer: rows r = item.y + 32 w + 16 mt + lane % 16 (expert-relative)
    const int wr0 = item.y + 32 * w;
    const bool act0 = wr0 < n_e, act1 = wr0 + 16 < n_e;   // (row tile 1 runs regardless)
    if (!act0) {
        wide_idle(0, KB);
        return;
    }
    const uint8_t* arow[2];
    {
        const size_t row_bytes = FP8 ? (size_t)K : (size_t)K * 2;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            int r = wr0 + 16 * mt + (lane & 15);
            r = r < n_e ? r : n_e - 1;
            const int64_t src_row = GEMM == 1 ? (int64_t)perm_token[off + r] : (int64_t)(off + r);
            arow[mt] = (const uint8_t*)A + src_row * row_bytes;
        }
    }
    f32x4_t acc[kMT][kNT];
    wide_consume<FP8>(acc, arow, 0, KB, bsm, lane);

    // ---------------- epilogue: lane holds column lane % 16 of each group, rows 4 (lane / 16) + i
    const int l16 = lane & 15, g4 = 4 * (lane >> 4);
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
        if (mt == 1 && !act1) break;
        if (GEMM == 1) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int cg = n0 + 32 * p + l16, cu = cg + 16;   // interleaved weight columns
                const float sg = FP8 ? scales[(size_t)e * N + cg] : 1.f;
                const float su = FP8 ? scales[(size_t)e * N + cu] : 1.f;
                const int hcol = (n0 >> 1) + 16 * p + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = wr0 + 16 * mt + g4 + i;
                    if (r >= n_e) continue;
                    const float g = acc[mt][2 * p][i] * sg, uu = acc[mt][2 * p + 1][i] * su;
                    const float hv = g / (1.0f + expf(-g)) * uu;
                    const size_t o = (size_t)(off + r) * F + hcol;
                    if (FP8) ((uint8_t*)out)[o] = (uint8_t)f32_to_e4m3(hv);
                    else ((bf16_t*)out)[o] = f32_to_bf16(hv);
                }
            }
        } else {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                const int c = n0 + 16 * nt + l16;
                const float sc = FP8 ? scales[(size_t)e * N + c] : 1.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = wr0 + 16 * mt + g4 + i;
                    if (r >= n_e) continue;
                    ((float*)out)[(size_t)(off + r) * N + c] = acc[mt][nt][i] * sc;
                }
            }
        }
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
        if ((2 * F) % kTileN || d % (dtype == kFP8 ? 64 : 32)) return hipErrorInvalidValue;
        dim3 grid((2 * F) / kTileN, work.max_items);
        if (dtype == kFP8)
            k_moe_wide<true, 1><<<grid, kWideThreads, 0, s>>>(X, d, 2 * F, F, perm_token, offsets,
                                                              work.items, work.count, w.w1, w.s1, H);
        else
            k_moe_wide<false, 1><<<grid, kWideThreads, 0, s>>>(X, d, 2 * F, F, perm_token, offsets,
                                                               work.items, work.count, w.w1, w.s1, H);
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
        if (d % kTileN || F % (dtype == kFP8 ? 64 : 32)) return hipErrorInvalidValue;
        dim3 grid(d / kTileN, work.max_items);
        if (dtype == kFP8)
            k_moe_wide<true, 2><<<grid, kWideThreads, 0, s>>>(H, F, d, F, nullptr, offsets,
                                                              work.items, work.count, w.w2, w.s2, Y);
        else
            k_moe_wide<false, 2><<<grid, kWideThreads, 0, s>>>(H, F, d, F, nullptr, offsets,
                                                               work.items, work.count, w.w2, w.s2, Y);
    }
    return hipGetLastError();
}

}  // namespace dg
