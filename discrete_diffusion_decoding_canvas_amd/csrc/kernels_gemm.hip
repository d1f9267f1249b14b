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
//   * expert GEMMs: a workgroup owns up to 256 rows of an expert (the second
//     GEMM: all of them; the first: 128, so that an expert with many rows is
//     spread over more CUs) for a 128-column slab, and the weight fragments go
//     through LDS once and feed every wave;
//   * tokens sit on the 16-row MFMA side (v_mfma_f32_16x16x32_bf16, or
//     v_mfma_f32_16x16x32_fp8_fp8 for e4m3 experts);
//   * the SwiGLU of the first expert GEMM runs in the epilogue (gate and up
//     columns are interleaved per 16-column group at pack time).
#include <algorithm>
#include <climits>

#include "head_epilogue.h"

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

// ------------------------------------------------------------------ dense bf16 GEMM, A in fragment order
// A given in MFMA A-fragment order (see frag_offset: [row/16][k-step][lane][16 B]),
// so every activation load is a contiguous 1 KiB per wave.  Tile DMT row tiles of
// 16 x 64 columns; the kDenseWaves waves split K, keep kDensePrefetch k-steps of operands
// in flight in registers and add their partial tiles in LDS in wave order.
// grid (N / 64, ceil(M / (16 DMT)), ksplit); ksplit > 1 stores partial sums at
// C + z * M * ldc (store epilogue only).
#ifndef DG_DENSE_WAVES
#define DG_DENSE_WAVES 8
#endif
#ifndef DG_DENSE_MT
#define DG_DENSE_MT 4
#endif
#ifndef DG_DENSE_PREFETCH
#define DG_DENSE_PREFETCH 4
#endif
constexpr int kDenseMT = DG_DENSE_MT;
constexpr int kDensePrefetch = DG_DENSE_PREFETCH;
constexpr int kDenseWaves = DG_DENSE_WAVES;
constexpr int kDenseThreads = 64 * kDenseWaves;

struct DenseStage {
    Frag16 a[kDenseMT];
    Frag16 b[kNT];
};

template <int EPI>
__global__ __launch_bounds__(kDenseThreads) void k_dense_frag(const uint8_t* __restrict__ Af, int M,
                                                         const bf16_t* __restrict__ Bp, int K,
                                                         int N, float* __restrict__ C, int ldc,
                                                         RopeArgs ra) {
    // row pitch kTileN + 1: the transposed V stores of the QKV epilogue read columns
    __shared__ float red[kDenseWaves][16 * kDenseMT][kTileN + 1];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = blockIdx.x * kTileN;
    const int m0 = blockIdx.y * 16 * kDenseMT;
    const int KB = K >> 5;
    const int tiles = (M + 15) >> 4;
    const uint8_t* ap[kDenseMT];
#pragma unroll
    for (int mt = 0; mt < kDenseMT; ++mt) {
        const int t = min((m0 >> 4) + mt, tiles - 1);   // tiles past M repeat the last one
        ap[mt] = Af + ((size_t)t * KB * 64 + lane) * 16;
    }
    const size_t gstride = (size_t)KB * 1024;
    const uint8_t* bg = (const uint8_t*)(Bp + (size_t)(n0 >> 4) * KB * 512) + (size_t)lane * 16;
    int zb, ze, kb0, kb1;
    split_range(KB, gridDim.z, blockIdx.z, zb, ze);
    split_range(ze - zb, kDenseWaves, w, kb0, kb1);
    kb0 += zb;
    kb1 += zb;
    f32x4_t acc[kDenseMT][kNT];
#pragma unroll
    for (int mt = 0; mt < kDenseMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto load = [&](DenseStage& st, int kb) {
#pragma unroll
        for (int mt = 0; mt < kDenseMT; ++mt) st.a[mt].u = ld16(ap[mt] + (size_t)kb * 1024);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) st.b[nt].u = ld16(bg + nt * gstride + (size_t)kb * 1024);
    };
    DenseStage buf[kDensePrefetch];
#pragma unroll
    for (int i = 0; i < kDensePrefetch - 1; ++i)
        if (kb0 + i < kb1) load(buf[i], kb0 + i);
    for (int kb = kb0; kb < kb1; kb += kDensePrefetch) {
#pragma unroll
        for (int u = 0; u < kDensePrefetch; ++u) {
            const int k = kb + u;
            if (k < kb1) {
                const int kn = k + kDensePrefetch - 1;
                if (kn < kb1) load(buf[(u + kDensePrefetch - 1) % kDensePrefetch], kn);
                const DenseStage& st = buf[u];
#pragma unroll
                for (int mt = 0; mt < kDenseMT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < kNT; ++nt)
                        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(st.a[mt].b, st.b[nt].b,
                                                                              acc[mt][nt], 0, 0, 0);
            }
        }
    }
    // partial tiles of the four waves, added in wave order
#pragma unroll
    for (int mt = 0; mt < kDenseMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                red[w][16 * mt + 4 * (lane >> 4) + j][16 * nt + (lane & 15)] = acc[mt][nt][j];
    __syncthreads();
    if constexpr (EPI == kEpiRope) {
        // The tile is 64 columns of one 128-dim head, pair-tiled: column c < 32 is dim
        // 32 tp + c, column c + 32 its rotary partner 64 + 32 tp + c (rotate-half RoPE,
        // y1 = x1 cos - x2 sin, y2 = x2 cos + x1 sin at the row's position).
        constexpr int D = 128, half = 64;
        const int head = n0 / D, tp = (n0 % D) / 64;
        auto rsum = [&](int r, int c) {
            float v = red[0][r][c];
#pragma unroll
            for (int i = 1; i < kDenseWaves; ++i) v += red[i][r][c];
            return v;
        };
        if (head < ra.Hq + ra.Hkv) {
            bf16_t* base = head < ra.Hq ? (bf16_t*)ra.q + (size_t)head * M * D
                                        : (bf16_t*)ra.kc + (size_t)(head - ra.Hq) * ra.kv_rows * D;
            for (int e = threadIdx.x; e < 16 * kDenseMT * 32; e += kDenseThreads) {
                const int r = e >> 5, c = e & 31;          // consecutive lanes: consecutive dims
                const int m = m0 + r;
                if (m >= M) continue;
                const int64_t pos = ra.pos0 + (ra.period > 0 ? m % ra.period : m);
                const int j = 32 * tp + c;
                const float x1 = rsum(r, c), x2 = rsum(r, c + 32);
                const float cs = ra.cos_t[pos * half + j], sn = ra.sin_t[pos * half + j];
                bf16_t* dst = base + (size_t)(head < ra.Hq ? m : ra.pos0 + m) * D;
                dst[j] = f32_to_bf16(x1 * cs - x2 * sn);
                dst[j + half] = f32_to_bf16(x2 * cs + x1 * sn);
            }
        } else {
            const int hv = head - ra.Hq - ra.Hkv;
            for (int e = threadIdx.x; e < 16 * kDenseMT * kTileN; e += kDenseThreads) {
                const int r = e & (16 * kDenseMT - 1), c = e / (16 * kDenseMT);   // lanes along positions
                const int m = m0 + r;
                if (m >= M) continue;
                const int dim = c < 32 ? 32 * tp + c : half + 32 * tp + (c - 32);
                ((bf16_t*)ra.vc)[vt_index(hv, dim, ra.pos0 + m, D, ra.kv_rows)] = f32_to_bf16(rsum(r, c));
            }
        }
        return;
    }
    float* Cz = C + (size_t)blockIdx.z * M * ldc;
    for (int e = threadIdx.x; e < 16 * kDenseMT * kTileN; e += kDenseThreads) {
        const int r = e >> 6, c = e & 63;
        const int m = m0 + r, n = n0 + c;
        if (m >= M) continue;
        float v = red[0][r][c];
#pragma unroll
        for (int i = 1; i < kDenseWaves; ++i) v += red[i][r][c];
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
// A unit is (kWideN-column weight slab, work item); a work item is up to
// kMoeItemRows (GEMM 1) or kMoeRows = 256 (GEMM 2, a whole canvas) rows of one
// expert, so an expert's weights leave HBM once per item.  Wide slabs keep the
// activation traffic, which every slab re-reads, at K * 2 bytes per row per
// kWideN output columns.  The kernels are persistent (about one workgroup per
// CU taking units in turn).
//
// kWideWaves waves, each with two roles:
//   * weight streaming: a stage is two packed k-steps of the slab's kWideNT
//     16-column groups (2 kWideNT KiB, one 1 KiB copy per (k-step, group));
//     wave w issues kCopies of them, from HBM straight into an LDS ring of
//     kRing stages with buffer loads to LDS (no registers), kRing - 1 stages
//     ahead.  Before the barrier that ends stage st each wave waits, with a
//     counted vmcnt, only for its own copies of stage st + 1; after the
//     barrier the whole stage is in LDS;
//   * MFMA: wave w owns rows 16 kWideMT w .. + 16 kWideMT - 1 of the item
//     (kWideMT MFMA row tiles), reads its activation fragments (contiguous
//     1 KiB per load, see frag_offset) into registers kWideLead stages ahead,
//     and multiplies them with the stage's fragments in LDS.  Waves past the
//     expert's rows only stream weights.
// Sixteen waves of <= 128 VGPRs fill a CU; the ring takes most of its LDS.
// The barrier is the bare s_barrier: a workgroup fence would wait for every
// load in flight.
//   GEMM 1: H[entry, :F] = silu(x Wg_e) * (x Wu_e).  The slab's columns are
//           [g_j | u_j | g_j+1 | u_j+1 | ...] (16 each), so a lane holds the
//           gate and up values of the same (row, column) and the SwiGLU runs in
//           registers.
//   GEMM 2: Y[entry, :d] = H[entry] Wd_e, stored as binary16 (f32_to_f16_sat;
//           a saturated value sets kBadRange in *bad) for the combine.  Column groups past d (when d is not a multiple of
//           kWideN) read as zero and are not stored.
// fp8: e4m3 operands on both sides, per output column scales applied after the
// accumulation.
// MX: MX FP4 weights (E2M1 codes, an E8M0 scale per 32 along K) against e4m3
// activations on the block-scaled 16x16x128 MFMA: a k-step is 128 of K, the
// weight chunk of a (group, k-step) is still 1 KiB, the activation fragment of a
// 16-row tile 2 KiB (frag_offset_mx), and the scales of a stage come as one 16-byte
// load per lane (mx_scale_bytes).
constexpr int kFmtBF16 = 0, kFmtFP8 = 1, kFmtMX = 2;
#ifndef DG_WIDE_RING
#define DG_WIDE_RING 6
#endif
constexpr int kWideNT = 8;                          // 16-column groups per slab
constexpr int kWideN = 16 * kWideNT;                // slab width
#ifndef DG_WIDE_MT
#define DG_WIDE_MT 1
#endif
constexpr int kWideMT = DG_WIDE_MT;                 // 16-row MFMA tiles per wave
constexpr int kWideWaves = kMoeRows / (16 * kWideMT);
constexpr int kWideThreads = 64 * kWideWaves;
constexpr int kWideWavesPerEU = kWideWaves / 4;     // one workgroup per CU: the VGPR budget
constexpr int kCopies = 2 * kWideNT / kWideWaves;   // 1 KiB weight copies per wave per stage
constexpr int kRing = DG_WIDE_RING;                 // LDS stages (2 kWideNT KiB each)
#ifndef DG_WIDE_LEAD
#define DG_WIDE_LEAD 1
#endif
constexpr int kWideLead = DG_WIDE_LEAD;             // activation stages loaded ahead per wave
constexpr int kWideSlots = kWideLead + 1;
static_assert(kCopies >= 1 && kCopies * kWideWaves == 2 * kWideNT, "copies split evenly over the waves");
static_assert(kCopies <= 2, "a wave's copies are of one column group");
static_assert(kWideWaves <= 16, "at most 16 waves per workgroup");
static_assert(kRing >= 3 && kRing * 2 * kWideNT * 1024 <= 160 * 1024, "ring size");
static_assert(kRing - 1 >= kWideLead, "prologue order");
static_assert(kWideNT % 4 == 0, "fragments are read from LDS four groups at a time");

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= n, other counters free.
constexpr int vmcnt_le(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8); }

// Vector-memory operations a wave issues per stage: the activation loads (one
// 16-byte fragment load per (k-step, row tile), two for MX; MX adds one 16-byte
// scale load) and its weight copies.  The counted waits below take these as lower
// bounds (the compiler may split a load, never merge two): every operation issued
// after the copy waited for only makes the wait stricter.
template <int FMT>
constexpr int wide_a_ops() { return FMT == kFmtMX ? 2 * 2 * kWideMT + 1 : 2 * kWideMT; }
template <int FMT>
constexpr int wide_wait_active() { return (kRing - 2) * (wide_a_ops<FMT>() + kCopies); }
constexpr int kWideWaitIdle = (kRing - 2) * kCopies;
static_assert(wide_wait_active<kFmtMX>() < 64 && wide_wait_active<kFmtBF16>() < 64,
              "vmcnt holds at most 63 operations");

using WideAcc = f32x4_t[kWideMT][kWideNT];
// Activation fragments of one stage: [k-step][row tile] (MX: two 16-byte halves of
// the 32-byte fragment, and the stage's weight scales).
template <int FMT>
struct WideFrag {
    Frag16 a[2][kWideMT];
};
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
template <>
struct WideFrag<kFmtMX> {
    i32x8_t a[2][kWideMT];   // the 32-byte operand, loaded as two 16-byte halves
    uint4 sc;
};

// Activation fragments of stage st of the k-step range [kb_lo, kb_hi) (clamped).
// afrag[mt] points at the row tile's fragment of k-step 0 plus the lane's bytes
// (lane * 16, MX lane * 32); k-steps are astride apart (1 KiB in fragment order, 64 B
// along a natural bf16 row, MX 2 KiB).  MX: sc points at the unit's scales of stage 0
// plus lane * 16 (stages 1 KiB apart).
template <int FMT>
DG_DEV void wide_load_a(WideFrag<FMT>& a, const uint8_t* const (&afrag)[kWideMT], int st,
                        int kb_lo, int kb_hi, uint32_t astride, const uint8_t* sc) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int kb = min(kb_lo + 2 * st + ks, kb_hi - 1);
#pragma unroll
        for (int mt = 0; mt < kWideMT; ++mt) {
            if constexpr (FMT == kFmtMX) {
                const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(afrag[mt] + (size_t)kb * astride);
                const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(afrag[mt] + (size_t)kb * astride + 16);
                a.a[ks][mt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            } else {
                a.a[ks][mt].u = ld16(afrag[mt] + (size_t)kb * astride);
            }
        }
    }
    if constexpr (FMT == kFmtMX) a.sc = ld16(sc + (size_t)st * 1024);
}

// The weight fragments are read from LDS in inline asm: the waves also issue
// LDS copies, and the compiler cannot tell the ring slots apart, so for a plain
// LDS read it would first wait for every copy in flight.  The barrier that ends
// the previous stage orders these reads after the copies they need.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWideReadGroups = 8;   // column groups read per LDS round trip (a whole k-step)
static_assert(kWideReadGroups == 4 || kWideReadGroups == 8, "");

DG_DEV void lds_read8(u32x4_t (&f)[8], uint32_t addr) {
    asm volatile(
        "ds_read_b128 %0, %8\n"
        "ds_read_b128 %1, %8 offset:1024\n"
        "ds_read_b128 %2, %8 offset:2048\n"
        "ds_read_b128 %3, %8 offset:3072\n"
        "ds_read_b128 %4, %8 offset:4096\n"
        "ds_read_b128 %5, %8 offset:5120\n"
        "ds_read_b128 %6, %8 offset:6144\n"
        "ds_read_b128 %7, %8 offset:7168\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5]),
          "=&v"(f[6]), "=&v"(f[7])
        : "v"(addr)
        : "memory");
}

DG_DEV void lds_read4(u32x4_t (&f)[4], uint32_t addr) {
    asm volatile(
        "ds_read_b128 %0, %4\n"
        "ds_read_b128 %1, %4 offset:1024\n"
        "ds_read_b128 %2, %4 offset:2048\n"
        "ds_read_b128 %3, %4 offset:3072\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3])
        : "v"(addr)
        : "memory");
}

DG_DEV void lds_read_groups(u32x4_t (&f)[4], uint32_t addr) { lds_read4(f, addr); }
DG_DEV void lds_read_groups(u32x4_t (&f)[8], uint32_t addr) { lds_read8(f, addr); }

// Both k-steps of a stage, straight-line.  When K has an odd number of packed
// k-steps the last stage's second k-step is multiplied by a zeroed activation
// fragment (keep1 = false).
// MX: the block-scaled MFMA on one 32-byte e4m3 activation fragment and one 16-byte
// E2M1 weight fragment.  The instruction reads only the low half of an E2M1 operand,
// so its upper half is left undefined (no register copies); the scale of the lane's K
// block is byte 0 of each scale operand (activations: 127, i.e. 1).
DG_DEV f32x4_t mfma_mx(const i32x8_t& a, const i32x4_t& b, uint32_t bscale, f32x4_t c) {
    const i32x8_t bv = __builtin_shufflevector(b, b, 0, 1, 2, 3, -1, -1, -1, -1);
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bv, c, 0, 4, 0, 127, 0, (int)bscale);
}

template <int FMT>
DG_DEV void wide_mma(WideAcc& acc, const WideFrag<FMT>& a, const uint4 (*bs)[kWideNT][64],
                     bool keep1, int lane) {
    constexpr bool FP8 = FMT == kFmtFP8;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        // MX skips a second k-step past K (a wave-uniform branch); the others multiply
        // it by a zeroed activation fragment
        if (FMT == kFmtMX && ks == 1 && !keep1) break;
        const uint32_t m = (ks == 0 || keep1) ? 0xffffffffu : 0u;
        Frag16 am[kWideMT];
        if constexpr (FMT != kFmtMX) {
#pragma unroll
            for (int mt = 0; mt < kWideMT; ++mt) {
                const uint4 v = a.a[ks][mt].u;
                am[mt].u = uint4{v.x & m, v.y & m, v.z & m, v.w & m};
            }
        }
        // MX reads four weight groups per LDS round trip (its 32-byte activation
        // fragments leave fewer registers for the weight fragments)
        constexpr int RG = FMT == kFmtMX ? 4 : kWideReadGroups;
#pragma unroll
        for (int n4 = 0; n4 < kWideNT; n4 += RG) {
            Frag16 fb[RG];
            {
                u32x4_t f[RG];
                lds_read_groups(f, (uint32_t)(uintptr_t)&bs[ks][n4][lane]);
#pragma unroll
                for (int i = 0; i < RG; ++i) fb[i].u = uint4{f[i].x, f[i].y, f[i].z, f[i].w};
            }
#pragma unroll
            for (int mt = 0; mt < kWideMT; ++mt)
#pragma unroll
                for (int i = 0; i < RG; ++i) {
                    f32x4_t& c = acc[mt][n4 + i];
                    if constexpr (FMT == kFmtMX) {
                        // scale byte (k-step ks, group n4 + i) of the stage's 16 bytes
                        const int gi = n4 + i;
                        const uint32_t w = ((2 * ks + gi / 4) == 0) ? a.sc.x : ((2 * ks + gi / 4) == 1) ? a.sc.y
                                         : ((2 * ks + gi / 4) == 2) ? a.sc.z : a.sc.w;
                        const i32x4_t b = {(int)fb[i].u.x, (int)fb[i].u.y, (int)fb[i].u.z, (int)fb[i].u.w};
                        c = mfma_mx(a.a[ks][mt], b, w >> (8 * (gi & 3)), c);
                    } else if constexpr (FP8) {
                        c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(am[mt].l.lo, fb[i].l.lo, c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(am[mt].l.hi, fb[i].l.hi, c, 0, 0, 0);
                    } else {
                        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am[mt].b, fb[i].b, c, 0, 0, 0);
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

using WideRing = uint4[kRing][2][kWideNT][64];   // [stage][k-step][group][lane]

// The part of the weight stream a wave copies: copies q = w * kCopies + c,
// c < kCopies, with k-step q % 2 of column group q / 2 (so a wave's copies are
// of one group).  The copy is a buffer load to LDS: the group's packed weights
// are the buffer (rsrc), the lane's 16 bytes its constant VGPR offset
// (voff = lane * 16) and the k-step its scalar offset, so no VGPR is rewritten
// per copy (a rewritten address register would make the compiler wait for the
// copy before reusing it).
struct WeightStream {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t voff;
    int g, ks0;            // column group, first k-step parity
    int kb_lo, kb_hi, NS;  // k-step range and its stage count
};

// Copies of stage st (clamped to the last stage) into ring slot `slot`.
DG_DEV void wide_copy_b(const WeightStream& ws, int st, int slot, WideRing& bsm) {
    const int sc = min(st, ws.NS - 1);
#pragma unroll
    for (int c = 0; c < kCopies; ++c) {
        const int ks = ws.ks0 + c;
        const int kb = min(ws.kb_lo + 2 * sc + ks, ws.kb_hi - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ws.rsrc, (__attribute__((address_space(3))) void*)&bsm[slot][ks][ws.g][0], 16, ws.voff,
            kb * 1024, 0, 0);
    }
}

// Buffer resource of one packed 16-column group (nbytes bytes at p): raw, no
// stride; loads past nbytes (all of them for nbytes = 0) return zero.
DG_DEV __amdgpu_buffer_rsrc_t group_rsrc(const void* p, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)nbytes, 0x00020000);
}

// The copies of stages 0..kRing - 2 of a stream into slots 0..kRing - 2.  A
// persistent workgroup issues them for its next unit before the epilogue of the
// current one (every slot is free once the current unit's last barrier passed).
DG_DEV void wide_fill(const WeightStream& ws, WideRing& bsm) {
#pragma unroll
    for (int st = 0; st < kRing - 1; ++st) wide_copy_b(ws, st, st, bsm);
}

// A wave without rows streams its share of the weights and keeps the barrier
// count (that of wide_mainloop: kRing - 1 filled stages, then NS + 2 barriers).
// The loads of a wave return in issue order, so a count that a wave's stores
// (an epilogue between the fill and here) push up only makes a wait stricter.
DG_DEV void wide_stream_only(const WeightStream& ws, WideRing& bsm) {
    __builtin_amdgcn_s_waitcnt(vmcnt_le(kWideWaitIdle));             // own copies of stage 0
    bare_barrier();
    for (int s0 = 0; s0 < ws.NS; s0 += kRing) {
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
            const int st = s0 + u;
            if (st >= ws.NS) break;
            wide_copy_b(ws, st + kRing - 1, (u + kRing - 1) % kRing, bsm);   // into the slot of st - 1
            __builtin_amdgcn_s_waitcnt(vmcnt_le(kWideWaitIdle));     // own copies of st + 1
            bare_barrier();
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
    bare_barrier();   // every wave's copies landed: the ring may be refilled
}

// Operations a wave has issued after its copies of stage st + 1 when stage st
// (st < kRing - 2) ends: the prologue's later copies and activation loads, and
// stages 0..st.  From stage kRing - 2 on it is wide_wait_active.
template <int FMT>
constexpr int wide_wait_early(int st) {
    return (kRing - 3 - st) * kCopies + kWideLead * wide_a_ops<FMT>() +
           (st + 1) * (wide_a_ops<FMT>() + kCopies);
}
constexpr int kWideEarly = kRing - 3 - kWideLead;   // stages whose exact count is below the steady one
static_assert(kWideEarly <= 0 || wide_wait_early<kFmtBF16>(kWideEarly - 1) < wide_wait_active<kFmtBF16>(), "");
static_assert(kWideEarly <= 0 || wide_wait_early<kFmtBF16>(kWideEarly) >= wide_wait_active<kFmtBF16>(), "");
static_assert(kWideEarly <= 0 || wide_wait_early<kFmtMX>(kWideEarly - 1) < wide_wait_active<kFmtMX>(), "");
static_assert(kWideEarly <= 0 || wide_wait_early<kFmtMX>(kWideEarly) >= wide_wait_active<kFmtMX>(), "");

// The exact wait at the end of stage u < N of the first pass (u is a constant
// once the stage loop is unrolled, and the chain folds to one s_waitcnt).
template <int FMT, int N>
DG_DEV void wide_wait_first(int u) {
    if constexpr (N > 0) {
        if (u == N - 1) __builtin_amdgcn_s_waitcnt(vmcnt_le(wide_wait_early<FMT>(N - 1)));
        wide_wait_first<FMT, N - 1>(u);
    }
}

// acc over the stream's k-steps, after wide_fill of the same stream.  The
// prologue issues the activation loads of stages 0..kWideLead - 1; stage st
// then issues the activation loads of stage st + kWideLead and the copies of
// stage st + kRing - 1, runs its MFMAs, waits for this wave's copies of stage
// st + 1 and meets the barrier.  The slot indices are compile-time: the loop is
// unrolled over kRing * kWideSlots stages.
template <int FMT>
DG_DEV void wide_mainloop(WideAcc& acc, const uint8_t* const (&afrag)[kWideMT],
                          const WeightStream& ws, WideRing& bsm, int lane,
                          uint32_t astride = 1024, const uint8_t* sc = nullptr) {
    const int NS = ws.NS;
#pragma unroll
    for (int mt = 0; mt < kWideMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < kWideNT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    asm volatile("" ::: "memory");   // the copies stay ahead of the activation loads
    WideFrag<FMT> ra[kWideSlots];
#pragma unroll
    for (int j = 0; j < kWideLead; ++j)
        wide_load_a<FMT>(ra[j], afrag, min(j, NS - 1), ws.kb_lo, ws.kb_hi, astride, sc);
    asm volatile("" ::: "memory");
    // issued after the copies of stage 0: the other kRing - 2 stages' copies and
    // kWideLead stages of activations
    __builtin_amdgcn_s_waitcnt(vmcnt_le((kRing - 2) * kCopies + kWideLead * wide_a_ops<FMT>()));
    bare_barrier();
    constexpr int kUnroll = kRing * kWideSlots;
    static_assert(kUnroll >= kWideEarly, "");
    for (int s0 = 0; s0 < NS; s0 += kUnroll) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int st = s0 + u;
            if (st >= NS) break;
            wide_load_a<FMT>(ra[(u + kWideLead) % kWideSlots], afrag, min(st + kWideLead, NS - 1),
                             ws.kb_lo, ws.kb_hi, astride, sc);
            wide_copy_b(ws, st + kRing - 1, (u + kRing - 1) % kRing, bsm);
            __builtin_amdgcn_sched_barrier(0);      // issue the loads before the MFMAs
            wide_mma<FMT>(acc, ra[u % kWideSlots], bsm[u % kRing], ws.kb_lo + 2 * st + 1 < ws.kb_hi,
                          lane);
            __builtin_amdgcn_sched_barrier(0);
            if (s0 == 0) wide_wait_first<FMT, kWideEarly>(u);
            __builtin_amdgcn_s_waitcnt(vmcnt_le(wide_wait_active<FMT>()));   // own copies of st + 1
            bare_barrier();
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
    bare_barrier();   // every wave's copies landed and LDS reads done: the ring may be refilled
}

// One unit of an expert GEMM: a work item (up to kMoeItemRows rows of one expert)
// times one kWideN-column slab.  Units are numbered item-major, so the slabs of
// an item (which share its activation rows) are taken up together.
struct MoeUnit {
    int e, off, n_e;   // expert, its first row, its rows end (expert-relative, item-clamped)
    int wr0, n0;       // this wave's first row (expert-relative), the slab's first column
    WeightStream ws;
};

template <int ITEM_ROWS>
DG_DEV MoeUnit moe_unit(int u, int n_slabs, const int4& item, int N, int KB, const void* W, int w,
                        int lane) {
    MoeUnit c;
    c.e = item.x;
    c.off = item.z;                                                // a multiple of 16
    c.n_e = min(item.w - item.z, item.y + ITEM_ROWS);
    c.n0 = (u % n_slabs) * kWideN;
    // rows r = item.y + 16 (kWideMT w + mt) + lane % 16 (expert-relative); n_e is
    // a multiple of 16, so a row tile is wholly inside or outside the expert
    c.wr0 = item.y + 16 * kWideMT * w;
    const size_t gsize = (size_t)KB * 1024;                         // bytes per packed 16-column group
    c.ws.g = w * kCopies / 2;
    c.ws.ks0 = (w * kCopies) & 1;
    const int gcol = (c.n0 >> 4) + c.ws.g;                         // the group's first column / 16
    c.ws.rsrc = group_rsrc((const uint8_t*)W + ((size_t)c.e * (N >> 4) + gcol) * gsize,
                           gcol < (N >> 4) ? (uint32_t)gsize : 0u);
    c.ws.voff = (uint32_t)lane * 16;
    c.ws.kb_lo = 0;
    c.ws.kb_hi = KB;
    c.ws.NS = (KB + 1) >> 1;
    return c;
}

// Epilogue of a unit: lane holds column lane % 16 of each group, rows 4 (lane / 16) + i.
// fp8 applies the per-column scales; MX needs none (the block scales act in the MFMA)
// and writes H in the MX activation order (K = F padded to 128).
template <int FMT, int GEMM>
DG_DEV void moe_epilogue(const WideAcc& acc, const MoeUnit& c, int N, int F,
                         const float* __restrict__ scales, void* __restrict__ out, int lane,
                         int32_t* __restrict__ bad) {
    constexpr bool FP8 = FMT == kFmtFP8;            // per-column scales
    constexpr bool E4 = FMT != kFmtBF16;            // e4m3 H
    const int l16 = lane & 15, g4 = 4 * (lane >> 4);
    bool range = false;
#pragma unroll
    for (int mt = 0; mt < kWideMT; ++mt) {
        if (c.wr0 + 16 * mt >= c.n_e) break;
        if (GEMM == 1) {
#pragma unroll
            for (int p = 0; p < kWideNT / 2; ++p) {
                const int cg = c.n0 + 32 * p + l16, cu = cg + 16;   // interleaved weight columns
                const float sg = FP8 ? scales[(size_t)c.e * N + cg] : 1.f;
                const float su = FP8 ? scales[(size_t)c.e * N + cu] : 1.f;
                const int hcol = (c.n0 >> 1) + 16 * p + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = c.wr0 + 16 * mt + g4 + i;
                    const float g = acc[mt][2 * p][i] * sg, uu = acc[mt][2 * p + 1][i] * su;
                    const float hv = g / (1.0f + expf(-g)) * uu;
                    // GEMM 2's A order
                    const size_t o = FMT == kFmtMX ? frag_offset_mx(c.off + r, hcol, (F + 127) & ~127)
                                                   : frag_offset<E4>(c.off + r, hcol, F);
                    if (E4) ((uint8_t*)out)[o] = (uint8_t)f32_to_e4m3(hv);
                    else *(bf16_t*)((uint8_t*)out + o) = f32_to_bf16(hv);
                }
            }
        } else {
#pragma unroll
            for (int nt = 0; nt < kWideNT; ++nt) {
                const int col = c.n0 + 16 * nt + l16;
                if (col >= N) break;
                const float sc = FP8 ? scales[(size_t)c.e * N + col] : 1.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = c.wr0 + 16 * mt + g4 + i;
                    ((_Float16*)out)[(size_t)(c.off + r) * N + col] =
                        f32_to_f16_sat(acc[mt][nt][i] * sc, range);
                }
            }
        }
    }
    if (range && bad) atomicOr(bad, kBadRange);
}

// Activations: Af in fragment order (frag_offset) by permuted row, or, with perm
// (bf16 GEMM 1), the natural bf16 token rows X [tokens][K]: lane l of a row tile
// reads 16 bytes of token perm[row0 + l % 16] (token 0 for padding rows, whose
// results are never combined) at k-chunk l / 16 of each k-step, the same
// fragment the permutation would have copied.
// Persistent: about one workgroup per CU, each taking units from the counter
// unit_ctr (zeroed by the routing kernel that wrote the work items) until
// work_count * n_slabs are taken.  After a unit's last stage the workgroup
// takes its next unit and issues that unit's first kRing - 1 weight stages (and,
// bf16 GEMM 1, its token indices) before it runs the current unit's epilogue, so
// the weight stream does not stop between units and no workgroup is launched for
// an absent item.  A work item carries its expert's row range, so a unit needs
// one load after the counter.
template <int FMT>
DG_DEV void moe_afrag(const uint8_t* (&afrag)[kWideMT], const MoeUnit& c, const uint8_t* Af,
                      int K, int KB, const int32_t* __restrict__ perm, int lane) {
#pragma unroll
    for (int mt = 0; mt < kWideMT; ++mt) {
        const int r = c.wr0 + 16 * mt < c.n_e ? c.wr0 + 16 * mt : c.wr0;   // past the rows: tile 0
        if (FMT == kFmtBF16 && perm != nullptr) {
            const int tok = max(perm[c.off + r + (lane & 15)], 0);
            afrag[mt] = Af + ((size_t)tok * K + 8 * (lane >> 4)) * 2;
        } else if (FMT == kFmtMX) {
            afrag[mt] = Af + ((size_t)((c.off + r) >> 4) * KB * 64 + lane) * 32;
        } else {
            afrag[mt] = Af + ((size_t)((c.off + r) >> 4) * KB * 64 + lane) * 16;
        }
    }
}

template <int FMT, int GEMM>
__global__ __launch_bounds__(kWideThreads, kWideWavesPerEU) void k_moe_wide(
    const uint8_t* Af, int K, int N, int F, const int4* __restrict__ work,
    const int32_t* __restrict__ work_count, int32_t* __restrict__ unit_ctr,
    const void* __restrict__ W, const float* __restrict__ scales, void* __restrict__ out,
    const int32_t* __restrict__ perm, int32_t* __restrict__ bad,
    const uint8_t* __restrict__ wscales = nullptr) {
    __shared__ __attribute__((aligned(16))) WideRing bsm;
    __shared__ int s_unit[2];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    // packed k-steps (MX: K is padded to a multiple of 128 by the caller)
    const int KB = FMT == kFmtMX ? (K >> 7) : FMT == kFmtFP8 ? (K >> 6) : (K >> 5);
    const int n_slabs = (N + kWideN - 1) / kWideN;
    const int total = *work_count * n_slabs;
    if (threadIdx.x == 0) s_unit[0] = atomicAdd(unit_ctr, 1);
    __syncthreads();
    int u = __builtin_amdgcn_readfirstlane(s_unit[0]);
    if (u >= total) return;
    constexpr int kItem = GEMM == 1 ? kMoeItemRows : kMoeRows;   // rows of one work item
    MoeUnit c = moe_unit<kItem>(u, n_slabs, work[u / n_slabs], N, KB, W, w, lane);
    wide_fill(c.ws, bsm);
    const uint8_t* afrag[kWideMT];
    if (c.wr0 < c.n_e) moe_afrag<FMT>(afrag, c, Af, K, KB, perm, lane);
    for (int it = 1;; ++it) {
        const bool rows = c.wr0 < c.n_e;          // uniform per wave
        WideAcc acc;
        if (rows) {
            // MX: this unit's (expert, slab) block scales, stage 0, this lane
            const uint8_t* sc = nullptr;
            if constexpr (FMT == kFmtMX)
                sc = wscales + (((size_t)c.e * n_slabs + c.n0 / kWideN) * ((KB + 1) >> 1) * 64 + lane) * 16;
            wide_mainloop<FMT>(acc, afrag, c.ws, bsm, lane,
                               FMT == kFmtMX ? 2048u : (FMT == kFmtBF16 && perm != nullptr) ? 64u : 1024u,
                               sc);
        } else {
            wide_stream_only(c.ws, bsm);
        }
        if (threadIdx.x == 0) s_unit[it & 1] = atomicAdd(unit_ctr, 1);
        __syncthreads();
        const int un = __builtin_amdgcn_readfirstlane(s_unit[it & 1]);
        int4 item;
        if (un < total) {
            item = work[un / n_slabs];
            wide_fill(moe_unit<kItem>(un, n_slabs, item, N, KB, W, w, lane).ws, bsm);
        }
        if (rows) moe_epilogue<FMT, GEMM>(acc, c, N, F, scales, out, lane, bad);
        if (un >= total) break;
        u = un;
        c = moe_unit<kItem>(un, n_slabs, item, N, KB, W, w, lane);   // recomputed: less live state
        if (c.wr0 < c.n_e) moe_afrag<FMT>(afrag, c, Af, K, KB, perm, lane);
    }
}

// LM head on the same pipeline: the "weights" are the packed embedding E (one
// 128-id slab per unit, streamed once), the activations the final normed hidden
// rows in fragment order, and the epilogue the streaming vocabulary statistics
// of each (row, 128-id slice) (head_epilogue).  Units (slab, 256-row block) are
// numbered slab-fastest and dealt round-robin to a persistent grid; the next
// unit's first weight stages are issued before the current unit's epilogue.
static_assert(kWideN == kHeadCols, "one unit's slab is one partial slice");

struct HeadUnit {
    int n0, wr0;
    WeightStream ws;
};

DG_DEV HeadUnit head_unit(int u, int n_slabs, const void* Ep, int KB, int w, int lane) {
    HeadUnit c;
    c.n0 = (u % n_slabs) * kWideN;                                 // first vocabulary id of the slab
    c.wr0 = (u / n_slabs) * kMoeRows + 16 * kWideMT * w;           // this wave's first row
    const size_t gsize = (size_t)KB * 1024;
    c.ws.g = w * kCopies / 2;
    c.ws.ks0 = (w * kCopies) & 1;
    const int gcol = (c.n0 >> 4) + c.ws.g;
    c.ws.rsrc = group_rsrc((const uint8_t*)Ep + (size_t)gcol * gsize, (uint32_t)gsize);
    c.ws.voff = (uint32_t)lane * 16;
    c.ws.kb_lo = 0;
    c.ws.kb_hi = KB;
    c.ws.NS = (KB + 1) >> 1;
    return c;
}

template <bool ENT>
__global__ __launch_bounds__(kWideThreads, kWideWavesPerEU) void k_head_wide(
    const uint8_t* Hf, int C, int d, const void* __restrict__ Ep, int V, float inv_tau,
    const uint8_t* __restrict__ mask, uint32_t key0, uint32_t key1, uint32_t c2, HeadPartials p,
    float* __restrict__ logits_out, uint16_t* __restrict__ sc_w) {
    __shared__ __attribute__((aligned(16))) WideRing bsm;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int KB = d >> 5;
    const int n_slabs = V / kWideN;
    const int total = n_slabs * ((C + kMoeRows - 1) / kMoeRows);
    int u = blockIdx.x;
    if (u >= total) return;
    HeadUnit c = head_unit(u, n_slabs, Ep, KB, w, lane);
    wide_fill(c.ws, bsm);
    for (;;) {
        const bool rows = c.wr0 < C;              // uniform per wave
        WideAcc acc;
        if (rows) {
            const uint8_t* afrag[kWideMT];
#pragma unroll
            for (int mt = 0; mt < kWideMT; ++mt) {
                const int r = c.wr0 + 16 * mt < C ? c.wr0 + 16 * mt : c.wr0;
                afrag[mt] = Hf + ((size_t)(r >> 4) * KB * 64 + lane) * 16;
            }
            wide_mainloop<kFmtBF16>(acc, afrag, c.ws, bsm, lane);
        } else {
            wide_stream_only(c.ws, bsm);
        }
        const int un = u + gridDim.x;
        if (un < total) wide_fill(head_unit(un, n_slabs, Ep, KB, w, lane).ws, bsm);
        if (rows) {
            static_assert(kWideMT <= 2, "head epilogue of one or two 16-row groups");
            const EpiArgs ea{C, V, c.n0, c.wr0, lane >> 4, lane & 15, inv_tau, mask, key0, key1, c2, p,
                             logits_out, sc_w};
            head_epilogue<0, ENT>(acc[0], ea);
            if constexpr (kWideMT > 1) head_epilogue<1, ENT>(acc[1], ea);
        }
        if (un >= total) break;
        u = un;
        c = head_unit(u, n_slabs, Ep, KB, w, lane);
    }
}

// Self-conditioning signal, its vocabulary-sized contraction u = P E (P the
// posterior rows p0 = Softmax(L_t / tau) in bf16, E the token embedding; the
// technical-report summary's update equations, the argument of FFW).  Same
// pipeline once more: the "weights" are E packed as the B operand of a
// [K = V] x [N = d] product (one 128-column slab of d per unit, the vocabulary
// as the streamed k-steps), the activations the natural posterior rows read in
// place (lane l of a row tile: 16 bytes of row l % 16 at k-chunk l / 16).
// M is small and K huge, so the work is cut stream-K style: the k-steps of all
// (256-row block, slab) units, unit after unit, are split into gridDim.x equal
// ranges, one per workgroup.  A range of at most KB k-steps touches at most two
// units; the workgroup stores one partial 256 x 128 tile per unit touched (slot
// 2 b + segment) and k_sc_reduce adds the tiles of each unit in range order.
DG_DEV WeightStream sc_stream(const void* Ep, int KB, int n_groups, int slab, int lo, int hi,
                              int w, int lane) {
    WeightStream ws;
    const size_t gsize = (size_t)KB * 1024;                         // bytes per packed 16-column group
    ws.g = w * kCopies / 2;
    ws.ks0 = (w * kCopies) & 1;
    const int gcol = slab * kWideNT + ws.g;
    ws.rsrc = group_rsrc((const uint8_t*)Ep + (size_t)gcol * gsize,
                         gcol < n_groups ? (uint32_t)gsize : 0u);    // groups past d read as zero
    ws.voff = (uint32_t)lane * 16;
    ws.kb_lo = lo;
    ws.kb_hi = hi;
    ws.NS = (hi - lo + 1) >> 1;
    return ws;
}

__global__ __launch_bounds__(kWideThreads, kWideWavesPerEU) void k_sc_expect(
    const uint8_t* __restrict__ P, int M, int V, const void* __restrict__ Ep, int d,
    float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) WideRing bsm;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int KB = V >> 5;
    const int n_slabs = (d + kWideN - 1) / kWideN;
    const int total = ((M + kMoeRows - 1) / kMoeRows) * n_slabs * KB;
    int x0, x1;
    split_range(total, gridDim.x, blockIdx.x, x0, x1);
    if (x0 >= x1) return;
    int unit = x0 / KB;
    WeightStream ws = sc_stream(Ep, KB, d >> 4, unit % n_slabs, x0 - unit * KB,
                                min(KB, x1 - unit * KB), w, lane);
    wide_fill(ws, bsm);
    for (int seg = 0; seg < 2; ++seg) {
        const int wr0 = (unit / n_slabs) * kMoeRows + 16 * kWideMT * w;   // this wave's first row
        const bool rows = wr0 < M;                                  // uniform per wave
        WideAcc acc;
        if (rows) {
            const uint8_t* afrag[kWideMT];
#pragma unroll
            for (int mt = 0; mt < kWideMT; ++mt) {
                const int r = min(wr0 + 16 * mt + (lane & 15), M - 1);
                afrag[mt] = P + ((size_t)r * V + 8 * (lane >> 4)) * 2;
            }
            wide_mainloop<kFmtBF16>(acc, afrag, ws, bsm, lane, 64u);
        } else {
            wide_stream_only(ws, bsm);
        }
        const int nx = (unit + 1) * KB;                             // the range goes on in unit + 1
        const bool more = seg == 0 && nx < x1;
        if (more) {
            ws = sc_stream(Ep, KB, d >> 4, (unit + 1) % n_slabs, 0, min(KB, x1 - nx), w, lane);
            wide_fill(ws, bsm);
        }
        if (rows) {
#pragma unroll
            for (int mt = 0; mt < kWideMT; ++mt) {
                float* dst = part + ((size_t)(2 * blockIdx.x + seg) * kMoeRows + 16 * (kWideMT * w + mt) +
                                     4 * (lane >> 4)) * kWideN + (lane & 15);
#pragma unroll
                for (int nt = 0; nt < kWideNT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[i * kWideN + 16 * nt] = acc[mt][nt][i];
            }
        }
        if (!more) break;
        ++unit;
    }
}

// u[r, c] = sum of the partial tiles of unit (r / 256, c / 128) over the ranges
// that touch it, in range order; also u in bf16 MFMA fragment order for the
// feed-forward block's first GEMM.  One thread per four columns.
__global__ __launch_bounds__(256) void k_sc_reduce(const float* __restrict__ part, int M, int d,
                                                   int V, int grid, float* __restrict__ u,
                                                   uint8_t* __restrict__ uf) {
    const int d4 = d >> 2;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * d4) return;
    const int r = (int)(i / d4), c = (int)(i % d4) * 4;
    const int KB = V >> 5;
    const int n_slabs = (d + kWideN - 1) / kWideN;
    const int total = ((M + kMoeRows - 1) / kMoeRows) * n_slabs * KB;
    const int per = total / grid, rem = total % grid;
    const int edge = rem * (per + 1);
    auto range_of = [&](int x) { return x < edge ? x / (per + 1) : rem + (x - edge) / per; };
    const int unit = (r / kMoeRows) * n_slabs + c / kWideN;
    const int b0 = range_of(unit * KB), b1 = range_of(unit * KB + KB - 1);
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int b = b0; b <= b1; ++b) {
        const int start = b * per + min(b, rem);
        const int seg = start / KB == unit ? 0 : 1;
        const float4 v = *reinterpret_cast<const float4*>(
            part + ((size_t)(2 * b + seg) * kMoeRows + r % kMoeRows) * kWideN + c % kWideN);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    *reinterpret_cast<float4*>(u + (size_t)r * d + c) = acc;
    ushort4 h;
    h.x = f32_to_bf16(acc.x);
    h.y = f32_to_bf16(acc.y);
    h.z = f32_to_bf16(acc.z);
    h.w = f32_to_bf16(acc.w);
    *reinterpret_cast<ushort4*>(uf + frag_offset<false>(r, c, d)) = h;   // c % 8 in {0, 4}
}

// fp8 GEMM 1's activation fragments: the e4m3 token rows of every 16-row tile
// of the permuted entries in MFMA A-operand order (frag_offset), zero for
// padding rows.  Done once here, the expert GEMM's activation loads become
// contiguous 1 KiB reads instead of 16-row gathers repeated for every weight
// slab.  (bf16 GEMM 1 reads the token rows in place instead.)
// MX: the fragments of the block-scaled 16x16x128 MFMA instead (frag_offset_mx): a
// lane's 32 bytes are columns 16 g .. + 15 and 64 + 16 g .. + 15 of a 128-column k-step.
template <bool MX>
__global__ __launch_bounds__(256) void k_moe_gather_frag8(const uint8_t* __restrict__ X, int K,
                                                          const int32_t* __restrict__ perm_token,
                                                          const int32_t* __restrict__ offsets,
                                                          int E, uint8_t* __restrict__ Xf) {
    const int KB = MX ? (K >> 7) : (K >> 6);
    const int kb = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int tile = blockIdx.y;
    if (kb >= KB || 16 * tile >= offsets[E]) return;
    const int lane = threadIdx.x & 63, g = lane >> 4;
    const int tok = perm_token[16 * tile + (lane & 15)];
    if constexpr (MX) {
        uint4 lo = make_uint4(0u, 0u, 0u, 0u), hi = lo;
        if (tok >= 0) {
            const uint8_t* row = X + (size_t)tok * K + kb * 128 + 16 * g;
            lo = *reinterpret_cast<const uint4*>(row);
            hi = *reinterpret_cast<const uint4*>(row + 64);
        }
        uint4* dst = reinterpret_cast<uint4*>(Xf + (((size_t)tile * KB + kb) * 64 + lane) * 32);
        dst[0] = lo;
        dst[1] = hi;
    } else {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (tok >= 0) {
            const uint8_t* row = X + (size_t)tok * K;
            const uint2 lo = *reinterpret_cast<const uint2*>(row + kb * 64 + 8 * g);
            const uint2 hi = *reinterpret_cast<const uint2*>(row + kb * 64 + 32 + 8 * g);
            v = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
        *reinterpret_cast<uint4*>(Xf + (((size_t)tile * KB + kb) * 64 + lane) * 16) = v;
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
hipError_t launch_gemm_frag(int epi, const void* Af, int M, const void* B, int K, int N, float* C,
                            int ldc, hipStream_t s, int ksplit, const RopeArgs* rope) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if ((K & 31) || (N % kTileN) || ksplit < 1 || (ksplit > 1 && epi != kEpiStoreF32))
        return hipErrorInvalidValue;
    dim3 grid(N / kTileN, (M + 16 * kDenseMT - 1) / (16 * kDenseMT), ksplit);
    const RopeArgs ra = rope ? *rope : RopeArgs{};
    if (epi == kEpiRope) {
        if (!rope || ksplit != 1 || N != (ra.Hq + 2 * ra.Hkv) * 128 || !ra.q || !ra.kc || !ra.vc)
            return hipErrorInvalidValue;
        k_dense_frag<kEpiRope><<<grid, kDenseThreads, 0, s>>>((const uint8_t*)Af, M, (const bf16_t*)B,
                                                          K, N, C, ldc, ra);
    } else if (epi == kEpiStoreF32) {
        k_dense_frag<kEpiStoreF32><<<grid, kDenseThreads, 0, s>>>((const uint8_t*)Af, M, (const bf16_t*)B,
                                                              K, N, C, ldc, ra);
    } else {
        k_dense_frag<kEpiAddF32><<<grid, kDenseThreads, 0, s>>>((const uint8_t*)Af, M, (const bf16_t*)B,
                                                            K, N, C, ldc, ra);
    }
    return hipGetLastError();
}

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

// Workgroups of a persistent wide kernel: one per CU of the current device.
static int persistent_wgs() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

static unsigned moe_grid(int max_items, int n_slabs) {
    const int64_t units = (int64_t)max_items * n_slabs;
    return (unsigned)std::min<int64_t>(units, persistent_wgs());
}

hipError_t launch_moe_gemm1(int dtype, const ExpertWeights& w, const void* X,
                            const int32_t* perm_token, const int32_t* offsets, int E, int d,
                            int F, int max_rows, const MoeWork& work, void* Xf, void* H,
                            hipStream_t s) {
    if (max_rows <= 0) return hipSuccess;
    if (dtype == kF32) {
        int64_t total = (int64_t)max_rows * F;
        k_moe1_f32<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
            (const float*)X, d, F, perm_token, offsets, E, max_rows, (const float*)w.w1,
            (const float*)w.wu, (float*)H);
    } else {
        const int kq = dtype == kMX ? 128 : dtype == kFP8 ? 64 : 32;
        if ((2 * F) % kWideN || d % kq || F % (dtype == kMX ? 32 : kq)) return hipErrorInvalidValue;
        const unsigned grid = moe_grid(work.max_items, (2 * F) / kWideN);
        if (dtype == kMX) {
            if (!Xf || !w.x1) return hipErrorInvalidValue;
            k_moe_wide<kFmtMX, 1><<<grid, kWideThreads, 0, s>>>((const uint8_t*)Xf, d, 2 * F, F,
                                                                work.items, work.count, work.count + 1,
                                                                w.w1, nullptr, H, nullptr, nullptr, w.x1);
        } else if (dtype == kFP8) {
            if (!Xf) return hipErrorInvalidValue;
            k_moe_wide<kFmtFP8, 1><<<grid, kWideThreads, 0, s>>>((const uint8_t*)Xf, d, 2 * F, F,
                                                                 work.items, work.count, work.count + 1,
                                                                 w.w1, w.s1, H, nullptr, nullptr);
        } else {
            // token rows read in place through the permutation
            k_moe_wide<kFmtBF16, 1><<<grid, kWideThreads, 0, s>>>((const uint8_t*)X, d, 2 * F, F,
                                                                  work.items, work.count, work.count + 1,
                                                                  w.w1, w.s1, H, perm_token, nullptr);
        }
    }
    return hipGetLastError();
}

hipError_t launch_head_wide(const void* hf, int C, int d, const void* E, int V, float inv_tau,
                            const uint8_t* mask, uint32_t key0, uint32_t key1, uint32_t c2,
                            const HeadPartials& p, float* logits_out, hipStream_t s,
                            uint16_t* sc_w) {
    if (C <= 0) return hipSuccess;
    if ((V % kWideN) || (d & 31)) return hipErrorInvalidValue;
    const int64_t units = (int64_t)(V / kWideN) * ((C + kMoeRows - 1) / kMoeRows);
    const unsigned grid = (unsigned)std::min<int64_t>(units, persistent_wgs());
    if (p.q)
        k_head_wide<true><<<grid, kWideThreads, 0, s>>>((const uint8_t*)hf, C, d, E, V, inv_tau, mask,
                                                        key0, key1, c2, p, logits_out, sc_w);
    else
        k_head_wide<false><<<grid, kWideThreads, 0, s>>>((const uint8_t*)hf, C, d, E, V, inv_tau, mask,
                                                         key0, key1, c2, p, logits_out, sc_w);
    return hipGetLastError();
}

int sc_grid(int M, int d, int V) {
    const int64_t n_units = (int64_t)((M + kMoeRows - 1) / kMoeRows) * ((d + kWideN - 1) / kWideN);
    const int64_t total = n_units * (V >> 5);
    // about one range per CU of at least 16 k-steps, and no fewer ranges than units
    // (a range then spans at most two units)
    const int64_t g = std::max<int64_t>(std::min<int64_t>(persistent_wgs(), total / 16), n_units);
    return (int)g;
}

size_t sc_part_floats(int M, int d, int V) {
    return (size_t)sc_grid(M, d, V) * 2 * kMoeRows * kWideN;
}

hipError_t launch_sc_expect(const uint16_t* P, int M, int V, const void* Ep, int d, float* part,
                            hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if ((V & 31) || (d & 15) || (int64_t)V * 64 > 0xffffffffLL) return hipErrorInvalidValue;
    if ((int64_t)((M + kMoeRows - 1) / kMoeRows) * ((d + kWideN - 1) / kWideN) * (V >> 5) > INT32_MAX)
        return hipErrorInvalidValue;
    k_sc_expect<<<sc_grid(M, d, V), kWideThreads, 0, s>>>((const uint8_t*)P, M, V, Ep, d, part);
    return hipGetLastError();
}

hipError_t launch_sc_reduce(const float* part, int M, int d, int V, float* u, void* uf,
                            hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if ((d & 15) || (V & 31)) return hipErrorInvalidValue;
    const int64_t n = (int64_t)M * (d / 4);
    k_sc_reduce<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(part, M, d, V, sc_grid(M, d, V), u,
                                                           (uint8_t*)uf);
    return hipGetLastError();
}

hipError_t launch_moe_gather8(const void* X, int d, const int32_t* perm_token,
                              const int32_t* offsets, int E, int max_rows, void* Xf, hipStream_t s,
                              bool mx) {
    if (max_rows <= 0) return hipSuccess;
    if (d % (mx ? 128 : 64) || !Xf) return hipErrorInvalidValue;
    const int KB = mx ? d / 128 : d / 64;
    dim3 gg((KB + 3) / 4, (max_rows + kMoePad - 1) / kMoePad);   // tiles past offsets[E] exit
    if (mx)
        k_moe_gather_frag8<true><<<gg, 256, 0, s>>>((const uint8_t*)X, d, perm_token, offsets, E,
                                                    (uint8_t*)Xf);
    else
        k_moe_gather_frag8<false><<<gg, 256, 0, s>>>((const uint8_t*)X, d, perm_token, offsets, E,
                                                     (uint8_t*)Xf);
    return hipGetLastError();
}

hipError_t launch_moe_gemm2(int dtype, const ExpertWeights& w, const void* H,
                            const int32_t* offsets, int E, int d, int F, int max_rows,
                            const MoeWork& work, float* Y, int32_t* bad, hipStream_t s) {
    if (max_rows <= 0) return hipSuccess;
    if (dtype == kF32) {
        int64_t total = (int64_t)max_rows * d;
        k_moe2_f32<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
            (const float*)H, d, F, offsets, E, max_rows, (const float*)w.w2, Y);
    } else {
        if (d % 16 || F % (dtype == kFP8 ? 64 : 32)) return hipErrorInvalidValue;
        const unsigned grid = moe_grid(work.max_items2, (d + kWideN - 1) / kWideN);
        if (dtype == kMX) {
            if (!w.x2) return hipErrorInvalidValue;
            // K of H and W2 padded to a multiple of 128 (zero columns / rows)
            k_moe_wide<kFmtMX, 2><<<grid, kWideThreads, 0, s>>>((const uint8_t*)H, (F + 127) & ~127,
                                                                d, F, work.items2, work.count + 3,
                                                                work.count + 2, w.w2, nullptr, Y,
                                                                nullptr, bad, w.x2);
        } else if (dtype == kFP8) {
            k_moe_wide<kFmtFP8, 2><<<grid, kWideThreads, 0, s>>>((const uint8_t*)H, F, d, F,
                                                                 work.items2, work.count + 3,
                                                                 work.count + 2, w.w2, w.s2, Y,
                                                                 nullptr, bad);
        } else {
            k_moe_wide<kFmtBF16, 2><<<grid, kWideThreads, 0, s>>>((const uint8_t*)H, F, d, F,
                                                                  work.items2, work.count + 3,
                                                                  work.count + 2, w.w2, w.s2, Y,
                                                                  nullptr, bad);
        }
    }
    return hipGetLastError();
}

}  // namespace dg
