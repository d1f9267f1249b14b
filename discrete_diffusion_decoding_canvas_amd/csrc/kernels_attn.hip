// Attention over [KV cache || canvas] for gfx950.
//
// The decoder attends bidirectionally across the canvas and to the context KV
// cache; the causal encoder (prefill / commit) attends causally
// (DiffusionGemma technical-report summary, Method: generation pipeline;
// alphasignal, paragraph on bidirectional attention: every canvas position
// attends to every other).  GQA: query head h reads KV head h / (Hq / Hkv).
//
// bf16 kernel (D = 128).  A workgroup owns 256 query rows of one KV head's
// group (the G query heads of the group packed row after row) and a range of
// keys; the key range is split over workgroups for occupancy and the splits
// are merged by a fixed-order combine.  Two producer waves copy every 32-key
// block of K (16-byte pieces of the key rows) and of V^T (the transposed,
// key-permuted cache) into a 6-block LDS ring with global_load_lds, landing in
// MFMA fragment order and keeping the consumers two blocks ahead; eight
// consumer waves own 32 query rows each and read their operand fragments from
// the ring:
//   S^T = K Q^T  (v_mfma_f32_16x16x32_bf16, A = K rows, B = Q rows) puts the
//   scores of one query in one lane column, so the online-softmax statistics
//   and the rescale of the output stay lane-local;
//   O^T = V^T P^T (v_mfma_f32_16x16x32_f16: A = V^T from the transposed,
//   key-permuted bf16 V cache, converted to binary16 in LDS by the V producer
//   wave, exact; B = P taken straight from the score registers, rounded to
//   binary16: 11 significant bits, against 8 for bf16; the causal encoder, whose
//   K/V persist in the cache, adds the remainder as a second binary16 part).
// Softmax runs in fp32 in the log2 domain: the running max is kept on raw
// scores and each exponent scale*log2(e)*(s - m) is one fma ahead of exp2.
#include <type_traits>

#include "kernels.h"

namespace dg {

constexpr int kAttnD = 128;
#ifndef DG_ATTN_WAVES
#define DG_ATTN_WAVES 8
#endif
#ifndef DG_ATTN_RING
#define DG_ATTN_RING 6
#endif
constexpr int kAttnWaves = DG_ATTN_WAVES;    // consumer waves (32 query rows each)
constexpr int kAttnRows = 32 * kAttnWaves;   // query rows per workgroup
constexpr int kAttnThreads = 64 * (kAttnWaves + 2);   // + a K and a V^T producer wave
constexpr int kAttnRing = DG_ATTN_RING;      // 32-key blocks in the LDS ring (16 KiB each)
static_assert(kAttnRing >= 3, "two blocks ahead of the one being consumed");
#ifndef DG_ATTN_PRE
#define DG_ATTN_PRE 3
#endif
constexpr int kAttnPre = DG_ATTN_PRE;         // blocks copied before the first barrier
static_assert(kAttnPre >= 3 && kAttnPre <= kAttnRing - 1, "blocks 0..2 before the first iteration ends");

union AFrag {
    uint4 u;
    bf16x8_t b;
    f16x8_t f;
    uint16_t h[8];
    uint32_t u32[4];
};

// One 32-key block of the LDS ring, in MFMA fragment order: K fragments
// [key half][32-dim step][lane] (A operand of S^T = K Q^T) and V^T fragments
// [16-dim group][lane] (A operand of O^T = V^T P^T); every fragment set is 1 KiB,
// written by one global_load_lds instruction and read back conflict-free.
struct AttnSlot {
    uint4 k[2][4][64];
    uint4 v[8][64];
};

DG_DEV void attn_bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= n, other counters free.
constexpr int attn_vmcnt_le(int n) {
    return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8);
}

DG_DEV void dma16(const uint16_t* src, uint4* dst) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// The V^T fragments of one ring slot, bf16 as copied from the cache, rewritten
// in place as binary16 (the PV MFMA's operand type) by the V producer wave once
// its copies of the block have landed.  bf16 values in binary16's normal range
// convert exactly (round toward zero only trims values below 2^-14 and clamps
// magnitudes above 65504).  LDS is read and written in inline asm so that the
// compiler does not wait for this wave's later copies in flight.
typedef __fp16 half2_t __attribute__((ext_vector_type(2)));

DG_DEV uint32_t bf16x2_to_f16x2(uint32_t w) {
    const half2_t h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
    return __builtin_bit_cast(uint32_t, h);
}

typedef unsigned int v4u32_t __attribute__((ext_vector_type(4)));

DG_DEV void convert_v_slot(uint4 (*v)[64], int lane) {
    const uint32_t addr = (uint32_t)(uintptr_t)&v[0][lane];
    v4u32_t f[8];
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
#pragma unroll
    for (int i = 0; i < 8; ++i)
        f[i] = v4u32_t{bf16x2_to_f16x2(f[i].x), bf16x2_to_f16x2(f[i].y), bf16x2_to_f16x2(f[i].z),
                       bf16x2_to_f16x2(f[i].w)};
    asm volatile(
        "ds_write_b128 %0, %1\n"
        "ds_write_b128 %0, %2 offset:1024\n"
        "ds_write_b128 %0, %3 offset:2048\n"
        "ds_write_b128 %0, %4 offset:3072\n"
        "ds_write_b128 %0, %5 offset:4096\n"
        "ds_write_b128 %0, %6 offset:5120\n"
        "ds_write_b128 %0, %7 offset:6144\n"
        "ds_write_b128 %0, %8 offset:7168\n"
        "s_waitcnt lgkmcnt(0)"
        :
        : "v"(addr), "v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(f[4]), "v"(f[5]), "v"(f[6]),
          "v"(f[7])
        : "memory");
}

// 2^x with the hardware exponential; results below the smallest normal flush to
// zero (a softmax weight under 2^-126 of the row maximum is dropped).
DG_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kAttnLazy = 8.f;   // log2 units a score may exceed the reference max by

// S^T block of 32 keys x 32 query rows (two query blocks): four independent
// accumulation chains over the four 32-dimension steps.
DG_DEV void attn_scores(f32x4_t (&st)[2][2], const AttnSlot& sl, const AFrag (&qf)[2][4],
                        int lane) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) st[qb][kh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        AFrag kf[2];
        kf[0].u = sl.k[0][s][lane];
        kf[1].u = sl.k[1][s][lane];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
                st[qb][kh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kh].b, qf[qb][s].b,
                                                                     st[qb][kh], 0, 0, 0);
    }
}

template <bool CAUSAL>
__global__ __launch_bounds__(kAttnThreads) void k_attn_bf16(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ Vt,
    int Hq, int Hkv, int M, int S, int64_t k_rows, int64_t v_rows, float scale_log2,
    int64_t q_pos0, int keys_per_split, int n_splits, bf16_t* __restrict__ O,
    uint8_t* __restrict__ Of, float* __restrict__ part_o, float* __restrict__ part_ml,
    int32_t* __restrict__ bad, int ctx, int canvas) {
    __shared__ AttnSlot ring[kAttnRing];
    const int G = Hq / Hkv;
    const int GM = G * M;
    const int kvh = blockIdx.y;
    const int split = blockIdx.z;
    const int row_base = blockIdx.x * kAttnRows;
    // batch of canvases: this workgroup's rows are queries of one canvas (canvas is a
    // multiple of kAttnRows), whose own keys sit boff rows past the shared context
    const int boff = canvas > 0 ? (row_base % M) / canvas * canvas : 0;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, g = lane >> 4;

    int kbeg = split * keys_per_split;
    int kend = kbeg + keys_per_split < S ? kbeg + keys_per_split : S;
    if (CAUSAL) {
        const int r_hi = row_base + kAttnRows - 1 < GM ? row_base + kAttnRows - 1 : GM - 1;
        const int mmax = (row_base / M != r_hi / M) ? M - 1 : r_hi % M;
        const int64_t lim = q_pos0 + mmax + 1;
        if (lim < kend) kend = (int)lim;
    }
    const int n_blocks = kend > kbeg ? (kend - kbeg + 31) / 32 : 0;

    if (w >= kAttnWaves) {
        // ---------------- producers: wave kAttnWaves copies K, the next one V^T, HBM -> LDS
        const bool is_v = w == kAttnWaves + 1;
        const bf16_t* Kh = K + (int64_t)kvh * k_rows * kAttnD;
        const bf16_t* Vh = Vt + (int64_t)kvh * kAttnD * v_rows;
        const int last = n_blocks > 0 ? n_blocks - 1 : 0;
        auto issue = [&](int b) {           // block b (clamped) into ring slot b % kAttnRing
            const int key0 = kbeg + 32 * min(b, last);
            AttnSlot* slot = &ring[b % kAttnRing];
            if (!is_v) {
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    int key = min(key0 + 16 * kh + l16, S - 1);
                    if (key >= ctx) key += boff;
                    const bf16_t* src = Kh + (int64_t)key * kAttnD + 8 * g;
#pragma unroll
                    for (int st = 0; st < 4; ++st) dma16(src + 32 * st, &slot->k[kh][st][0]);
                }
            } else {
                const int vkey0 = key0 >= ctx ? key0 + boff : key0;   // ctx % 32 == 0 when batched
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
                    dma16(Vh + (int64_t)(16 * dt + l16) * v_rows + vkey0 + 8 * g, &slot->v[dt][0]);
            }
        };
        // The consumers read K of block b + 1 and V of block b in iteration b, so before
        // the barrier that opens iteration b the blocks up to b + 1 must have landed and
        // the V of block b must be in binary16.
        // Before the first barrier only kAttnPre blocks are asked for (every CU starts at
        // once, and the first two are the ones waited for); the first iteration asks for
        // the rest of the ring.
        for (int b = 0; b < kAttnPre; ++b) issue(b);
        __builtin_amdgcn_s_waitcnt(attn_vmcnt_le(8 * (kAttnPre - 2)));   // blocks 0, 1 landed
        if (is_v && n_blocks > 0) convert_v_slot(ring[0].v, lane);
        attn_bare_barrier();
        for (int b = 0; b < n_blocks; ++b) {
            if (b == 0) {
                for (int i = kAttnPre; i < kAttnRing; ++i) issue(i);   // unused slots
            } else {
                issue(b + kAttnRing - 1);                               // into the slot of block b - 1
            }
            __builtin_amdgcn_s_waitcnt(attn_vmcnt_le(8 * (kAttnRing - 3)));   // block b + 2 landed
            if (is_v && b + 1 < n_blocks) convert_v_slot(ring[(b + 1) % kAttnRing].v, lane);
            attn_bare_barrier();
        }
        __builtin_amdgcn_s_waitcnt(attn_vmcnt_le(0));
        return;
    }

    // ---------------- consumers: this wave's 32 rows, two query blocks of 16, packed over the heads
    const int wrow = row_base + 32 * w;
    const bool wave_active = wrow < GM;
    AFrag qf[2][4];
    int qm[2], qh[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        int r = wrow + 16 * qb + l16;
        const bool ok = r < GM;
        r = ok ? r : GM - 1;
        qh[qb] = kvh * G + r / M;
        qm[qb] = ok ? r % M : -1;
        const bf16_t* src = Q + ((int64_t)qh[qb] * M + r % M) * kAttnD + 8 * g;
#pragma unroll
        for (int s = 0; s < 4; ++s) qf[qb][s].u = *reinterpret_cast<const uint4*>(src + 32 * s);
    }
    // Running reference maximum per query row, kept in log2 units (score * scale_log2).
    // It is raised only when a score exceeds it by more than kAttnLazy (a factor 2^8):
    // the weights 2^(score - ref) then stay below 2^8, the sums are the same in exact
    // arithmetic, and most blocks need neither a cross-lane maximum nor a rescale.
    float m_ref[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};
    f32x4_t o[2][8];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[qb][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    __syncthreads();

    int qlim[2];                        // causal: last key position each query row sees
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) qlim[qb] = (int)(q_pos0 + qm[qb]);
    int wave_qlim = min(qlim[0], qlim[1]);   // causal: keys up to here need no per-row test
#pragma unroll
    for (int o2 = 1; o2 < 64; o2 <<= 1) wave_qlim = min(wave_qlim, __shfl_xor(wave_qlim, o2, 64));

    // One block of 32 keys: softmax weights of the scores st (block key0), then the PV
    // MFMAs.  MASK: keys past kend (and, causal, past each row's position) are -inf.
    auto softmax_pv = [&](const f32x4_t (&st)[2][2], int key0, const AttnSlot& sl, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        auto score = [&](int qb, int kh, int j) {
            const float v = st[qb][kh][j];
            if (!MASK) return v;
            const int key = key0 + 16 * kh + 4 * g + j;
            bool ok = key < kend;
            if (CAUSAL) ok = ok && key <= qlim[qb];
            return ok ? v : -INFINITY;
        };
        float lm[2];
        bool need = false;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            lm[qb] = -INFINITY;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int j = 0; j < 4; ++j) lm[qb] = fmaxf(lm[qb], score(qb, kh, j));
            need |= fmaf(lm[qb], scale_log2, -m_ref[qb]) > kAttnLazy;
        }
        if (__any(need)) {
            // raise the reference of every row of this wave to its maximum so far
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float mx = lm[qb];
                mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const float m_new = fmaxf(m_ref[qb], mx * scale_log2);
                if (m_new > m_ref[qb]) {
                    const float alpha = m_ref[qb] == -INFINITY ? 0.f : fast_exp2(m_ref[qb] - m_new);
                    l_run[qb] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) o[qb][dt] *= alpha;
                    m_ref[qb] = m_new;
                }
            }
        }
        // P in binary16 (round to nearest even; p < 2^9).  The causal encoder, whose K/V
        // stay in the cache for every later pass, adds the rounding remainder as a second
        // binary16 part (about 22 significant bits) and sums p in fp32; a decoder pass uses
        // one part and sums the binary16 weights the PV product uses, two per fp32 dot
        // product with (1, 1).
        AFrag pf[2], pl[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float nb = m_ref[qb] == -INFINITY ? 0.f : -m_ref[qb];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p = fast_exp2(fmaf(score(qb, i >> 2, i & 3), scale_log2, nb));
                const _Float16 hi = (_Float16)p;
                pf[qb].f[i] = hi;
                if (CAUSAL) {
                    psum += p;
                    pl[qb].f[i] = (_Float16)(p - (float)hi);
                }
            }
            if (!CAUSAL) {
                const half2_t one2 = {(__fp16)1.0f, (__fp16)1.0f};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    psum = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pf[qb].u32[j]), one2, psum, false);
            }
            l_run[qb] += psum;
        }
        // O^T += V^T P^T (the V cache is binary16)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            AFrag vf;
            vf.u = sl.v[dt][lane];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                o[qb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf.f, pf[qb].f, o[qb][dt], 0, 0, 0);
                if (CAUSAL)
                    o[qb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf.f, pl[qb].f, o[qb][dt], 0, 0, 0);
            }
        }
    };

    // Software pipeline per wave: block b's softmax and PV MFMAs run after the score
    // MFMAs of block b + 1 are issued, so the matrix cores and the VALU overlap.  The
    // blocks that need no key mask (all but the last, and for the causal encoder all
    // before this wave's diagonal) come first and run a loop of their own.
    // The unmasked blocks go two at a time, the score registers swapping roles.
    f32x4_t sa[2][2], sb[2][2];
    auto block = [&](int b, const f32x4_t (&st)[2][2], f32x4_t (&sn)[2][2], auto mask_tag) {
        if (wave_active) {
            if (b + 1 < n_blocks) attn_scores(sn, ring[(b + 1) % kAttnRing], qf, lane);
            softmax_pv(st, kbeg + 32 * b, ring[b % kAttnRing], mask_tag);
        }
        __syncthreads();
    };
    int n_full = (kend - kbeg) / 32;
    if (CAUSAL) n_full = min(n_full, max(0, (wave_qlim - kbeg + 1) / 32));
    if (wave_active && n_blocks > 0) attn_scores(sa, ring[0], qf, lane);
    int b = 0;
    for (; b + 1 < n_full; b += 2) {
        block(b, sa, sb, std::false_type{});
        block(b + 1, sb, sa, std::false_type{});
    }
    auto swap_in = [&]() {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) sa[qb][kh] = sb[qb][kh];
    };
    if (b < n_full) {
        block(b++, sa, sb, std::false_type{});
        swap_in();
    }
    for (; b < n_blocks; ++b) {
        block(b, sa, sb, std::true_type{});
        swap_in();
    }
    if (!wave_active) return;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float l = l_run[qb];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        const int q = qm[qb];
        if (q < 0) continue;
        const int h = qh[qb];
        if (n_splits == 1) {
            const float inv = 1.0f / l;
            bf16_t* dst = O + (int64_t)q * Hq * kAttnD + (int64_t)h * kAttnD;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                uint2 pk;
                pk.x = (uint32_t)f32_to_bf16(o[qb][dt][0] * inv) |
                       ((uint32_t)f32_to_bf16(o[qb][dt][1] * inv) << 16);
                pk.y = (uint32_t)f32_to_bf16(o[qb][dt][2] * inv) |
                       ((uint32_t)f32_to_bf16(o[qb][dt][3] * inv) << 16);
                if (O) *reinterpret_cast<uint2*>(dst + 16 * dt + 4 * g) = pk;
                if (Of)
                    *reinterpret_cast<uint2*>(Of + frag_offset<false>(q, h * kAttnD + 16 * dt + 4 * g,
                                                                      Hq * kAttnD)) = pk;
            }
        } else {
            // the split's own softmax average (bounded by max |V|) as binary16,
            // rounded to nearest, finite values saturated at its largest one
            const int64_t pr = ((int64_t)split * Hq + h) * M + q;
            const float inv = l > 0.f ? 1.0f / l : 0.f;
            _Float16* dst = reinterpret_cast<_Float16*>(part_o) + pr * kAttnD;
            bool range = false;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                f16x4_t pk;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pk[i] = f32_to_f16_sat(o[qb][dt][i] * inv, range);
                *reinterpret_cast<f16x4_t*>(dst + 16 * dt + 4 * g) = pk;
            }
            if (range && bad) atomicOr(bad, kBadRange);
            if (g == 0) {
                part_ml[pr * 2 + 0] = m_ref[qb];   // log2 units, as the weights
                part_ml[pr * 2 + 1] = l;
            }
        }
    }
}

// Fixed-order combine of the key splits: with each split's average A_s = O_s / l_s
// (stored as binary16), O = sum_s 2^(m_s - m*) l_s A_s / sum_s 2^(m_s - m*) l_s.
// One wave per (query, head): lane s first holds split s's statistics (n_splits <=
// 64); then lane 16 i + c takes the 8 dimensions 8c.. of splits i, i + 4, i + 8, ..
// (one 16-byte load each, four in flight together) and the four partial sums of a
// chunk are added by two lane exchanges, in the same order for every call.
template <typename T>
__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      int n_splits, int Hq, int M,
                                                      T* __restrict__ O, uint8_t* __restrict__ Of) {
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (wid >= M * Hq) return;
    const int q = wid / Hq, h = wid % Hq;
    float ms = -INFINITY, ls = 0.f;
    if (lane < n_splits) {
        const float2 ml = *reinterpret_cast<const float2*>(
            part_ml + ((((int64_t)lane * Hq + h) * M + q) * 2));
        ms = ml.x;
        ls = ml.y;
    }
    const float mstar = wave_max(ms);
    const float wl = (ms == -INFINITY) ? 0.f : exp2f(ms - mstar) * ls;
    const float den = wave_sum(wl);
    const int gi = lane >> 4, c = lane & 15;
    const _Float16* pa = reinterpret_cast<const _Float16*>(part_o) + 8 * c;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // splits past n_splits re-read the last one with weight 0
    for (int t0 = 0; t0 < n_splits; t0 += 16) {
        f16x8_t v[4];
        float ws[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int sp = t0 + 4 * t + gi;
            ws[t] = __shfl(wl, sp < 64 ? sp : 63, 64);
            const int sl = sp < n_splits ? sp : n_splits - 1;
            v[t] = *reinterpret_cast<const f16x8_t*>(pa + (((int64_t)sl * Hq + h) * M + q) * kAttnD);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += ws[t] * (float)v[t][i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        acc[i] += __shfl_xor(acc[i], 16, 64);
        acc[i] += __shfl_xor(acc[i], 32, 64);
    }
    if (gi != 0) return;
    T r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = from_f32<T>(acc[i] / den);
    if (O) {
        T* dst = O + (int64_t)q * Hq * kAttnD + (int64_t)h * kAttnD + 8 * c;
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[i] = r[i];
    }
    if (Of) {
        T* f = reinterpret_cast<T*>(Of + frag_offset<false>(q, h * kAttnD + 8 * c, Hq * kAttnD));
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = r[i];
    }
}

// f32 attention (VALU): one thread per (head, query), online softmax over keys.
template <int D>
__global__ __launch_bounds__(64) void k_attn_f32(const float* __restrict__ Q,
                                                 const float* __restrict__ K,
                                                 const float* __restrict__ V, int Hq, int Hkv,
                                                 int M, int S, int64_t rows, float scale,
                                                 int causal, int64_t q_pos0,
                                                 float* __restrict__ O, int ctx, int canvas) {
    const int q = blockIdx.x * 64 + threadIdx.x;
    const int h = blockIdx.y;
    if (q >= M) return;
    const int boff = canvas > 0 ? q / canvas * canvas : 0;   // batch: the canvas's own rows
    const int kvh = h / (Hq / Hkv);
    float qv[D], ov[D];
#pragma unroll
    for (int t = 0; t < D; ++t) {
        qv[t] = Q[((int64_t)h * M + q) * D + t] * scale;
        ov[t] = 0.f;
    }
    int kend = S;
    if (causal) {
        const int64_t lim = q_pos0 + q + 1;
        if (lim < kend) kend = (int)lim;
    }
    float m = -INFINITY, l = 0.f;
    const float* Kh = K + (int64_t)kvh * rows * D;
    const float* Vh = V + (int64_t)kvh * rows * D;
    for (int j = 0; j < kend; ++j) {
        const int64_t jr = j >= ctx ? j + boff : j;
        float s = 0.f;
#pragma unroll
        for (int t = 0; t < D; ++t) s = fmaf(qv[t], Kh[jr * D + t], s);
        const float mn = fmaxf(m, s);
        const float a = expf(m - mn), p = expf(s - mn);
        l = l * a + p;
#pragma unroll
        for (int t = 0; t < D; ++t) ov[t] = ov[t] * a + p * Vh[jr * D + t];
        m = mn;
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int t = 0; t < D; ++t) O[(int64_t)q * Hq * D + (int64_t)h * D + t] = ov[t] * inv;
}

// ================================================================== launchers
// Splits of the key range: about 256 workgroups in total, at least 256 keys each.
#ifndef DG_ATTN_TARGET_WGS
#define DG_ATTN_TARGET_WGS 256
#endif
// With T target workgroups of R = kAttnRows query rows, a split call (n >= 2
// splits) has qwgs < T query workgroups and Hq M <= R qwgs, so n Hq M <=
// (T / qwgs + 1) R qwgs = R (T + qwgs) < 2 R T query rows of partials.
static_assert(2 * kAttnRows * DG_ATTN_TARGET_WGS <= kAttnMaxPartRows, "partials bound");
static int attn_splits(int Hq, int Hkv, int M, int S) {
    const int G = Hq / Hkv;
    const int qwgs = Hkv * ((G * M + kAttnRows - 1) / kAttnRows);
    int n = (DG_ATTN_TARGET_WGS + qwgs - 1) / qwgs;
    const int max_by_keys = (S + 255) / 256;
    if (n > max_by_keys) n = max_by_keys;
    if (n > 64) n = 64;
    return n < 1 ? 1 : n;
}

// Split count and keys per split (a multiple of the 32-key block).
static void attn_split_plan(int Hq, int Hkv, int M, int S, int& n, int& kps) {
    n = attn_splits(Hq, Hkv, M, S);
    kps = (S + n - 1) / n;
    kps = (kps + 31) & ~31;
    n = (S + kps - 1) / kps;
}

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t attention_part_bytes(int dtype, int Hq, int Hkv, int M, int S, int D) {
    if (dtype == kF32 || M <= 0 || S <= 0 || Hkv <= 0 || Hq % Hkv) return 0;
    int n, kps;
    attn_split_plan(Hq, Hkv, M, S, n, kps);
    if (n <= 1) return 0;
    const size_t rows = (size_t)n * Hq * M;
    return align256(rows * D * 2) + rows * 8;
}

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    const int ctx = a.canvas > 0 ? (int)a.ctx : a.S;   // no remap: every key below ctx
    if (a.canvas > 0) {
        // every query's keys: the shared context, then its canvas's own rows
        if (a.causal || a.M % a.canvas || a.ctx < 0 || a.S != a.ctx + a.canvas ||
            a.kv_rows < a.ctx + a.M || (dtype != kF32 && (a.canvas % kAttnRows || (a.ctx & 31) ||
                                                        a.v_rows < a.ctx + a.M)))
            return hipErrorInvalidValue;
    }
    if (dtype == kF32) {
        dim3 grid((a.M + 63) / 64, a.Hq);
        if (a.D == 64)
            k_attn_f32<64><<<grid, 64, 0, s>>>((const float*)a.q, (const float*)a.k,
                                               (const float*)a.v, a.Hq, a.Hkv, a.M, a.S,
                                               a.kv_rows, a.scale, a.causal, a.q_pos0,
                                               (float*)a.o, ctx, a.canvas);
        else if (a.D == 128)
            k_attn_f32<128><<<grid, 64, 0, s>>>((const float*)a.q, (const float*)a.k,
                                                (const float*)a.v, a.Hq, a.Hkv, a.M, a.S,
                                                a.kv_rows, a.scale, a.causal, a.q_pos0,
                                                (float*)a.o, ctx, a.canvas);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
    if (a.D != kAttnD || (a.v_rows & 31) || a.v_rows < a.S || a.kv_rows < a.S || (!a.o && !a.of))
        return hipErrorInvalidValue;
    int n, kps;
    attn_split_plan(a.Hq, a.Hkv, a.M, a.S, n, kps);
    const size_t prow = (size_t)n * a.Hq * a.M;
    if (n > 1 && (!a.part || align256(prow * a.D * 2) + prow * 8 > a.part_bytes))
        return hipErrorInvalidValue;
    const int G = a.Hq / a.Hkv;
    dim3 grid((G * a.M + kAttnRows - 1) / kAttnRows, a.Hkv, n);
    const float sl2 = a.scale * 1.4426950408889634f;
    float* po = (float*)a.part;
    float* pml = n > 1 ? (float*)((char*)a.part + align256(prow * a.D * 2)) : nullptr;
    if (a.causal)
        k_attn_bf16<true><<<grid, kAttnThreads, 0, s>>>((const bf16_t*)a.q, (const bf16_t*)a.k,
                                               (const bf16_t*)a.v, a.Hq, a.Hkv, a.M, a.S,
                                               a.kv_rows, a.v_rows, sl2, a.q_pos0, kps, n,
                                               (bf16_t*)a.o, (uint8_t*)a.of, po, pml, a.bad, ctx,
                                               a.canvas);
    else
        k_attn_bf16<false><<<grid, kAttnThreads, 0, s>>>((const bf16_t*)a.q, (const bf16_t*)a.k,
                                                (const bf16_t*)a.v, a.Hq, a.Hkv, a.M, a.S,
                                                a.kv_rows, a.v_rows, sl2, a.q_pos0, kps, n,
                                                (bf16_t*)a.o, (uint8_t*)a.of, po, pml, a.bad, ctx,
                                               a.canvas);
    if (n > 1)
        k_attn_combine<bf16_t><<<(a.M * a.Hq + 3) / 4, 256, 0, s>>>(po, pml, n, a.Hq, a.M,
                                                                    (bf16_t*)a.o, (uint8_t*)a.of);
    return hipGetLastError();
}

}  // namespace dg
