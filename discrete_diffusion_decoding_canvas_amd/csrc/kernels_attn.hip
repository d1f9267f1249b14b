// Attention over [KV cache || canvas] for gfx950.
//
// The decoder attends bidirectionally across the canvas and to the context KV
// cache; the causal encoder (prefill / commit) attends causally
// (DiffusionGemma technical-report summary, Method: generation pipeline;
// alphasignal, paragraph on bidirectional attention: every canvas position
// attends to every other).  GQA: query head h reads KV head h / (Hq / Hkv).
//
// bf16 kernel (D = 128).  A workgroup of 8 waves owns 256 query rows of one KV
// head's group (the G query heads of the group packed row after row) and a
// range of keys; the key range is split over workgroups for occupancy and the
// splits are merged by a fixed-order combine.  Per block of 32 keys the eight
// waves load K and V once into double-buffered LDS (row pitches padded so the
// 16-byte fragment reads are bank-conflict free) and every wave reads its
// MFMA fragments from there:
//   S^T = K Q^T  (v_mfma_f32_16x16x32_bf16, A = K rows, B = Q rows) puts the
//   scores of one query in one lane column, so the online-softmax statistics
//   and the rescale of the output stay lane-local;
//   O^T = V^T P^T (A = V^T from the transposed, key-permuted V cache, B = P
//   taken straight from the score registers), with P split into hi + lo bf16
//   parts so the softmax weights keep ~16 significant bits.
// Softmax runs in fp32 in the log2 domain (exp2), scale applied to fp32 scores.
#include "kernels.h"

namespace dg {

constexpr int kAttnD = 128;
constexpr int kAttnWaves = 8;
constexpr int kAttnRows = 32 * kAttnWaves;   // query rows per workgroup
constexpr int kKPitch = 136;                 // LDS row pitch of a K row (bf16): 272 B
constexpr int kVPitch = 40;                  // LDS row pitch of a V^T row (bf16): 80 B

union AFrag {
    uint4 u;
    bf16x8_t b;
    uint16_t h[8];
};

template <bool CAUSAL>
__global__ __launch_bounds__(512) void k_attn_bf16(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ Vt,
    int Hq, int Hkv, int M, int S, int64_t k_rows, int64_t v_rows, float scale_log2,
    int64_t q_pos0, int keys_per_split, int n_splits, bf16_t* __restrict__ O,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
    __shared__ __attribute__((aligned(16))) bf16_t ks[2][32][kKPitch];
    __shared__ __attribute__((aligned(16))) bf16_t vs[2][kAttnD][kVPitch];
    const int G = Hq / Hkv;
    const int GM = G * M;
    const int kvh = blockIdx.y;
    const int split = blockIdx.z;
    const int row_base = blockIdx.x * kAttnRows;
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
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

    // this wave's 32 rows: two query blocks of 16, packed over the group's heads
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
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};
    f32x4_t o[2][8];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[qb][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // cooperative loads: thread -> one 16-byte piece of the K block and of the V^T block
    const bf16_t* Kh = K + (int64_t)kvh * k_rows * kAttnD;
    const bf16_t* Vh = Vt + (int64_t)kvh * kAttnD * v_rows;
    const int lk_key = tid >> 4, lk_col = (tid & 15) * 8;
    const int lv_dim = tid >> 2, lv_col = (tid & 3) * 8;
    auto gload = [&](int key0, uint4& kr, uint4& vr) {
        int key = key0 + lk_key;
        key = key < S ? key : S - 1;
        kr = *reinterpret_cast<const uint4*>(Kh + (int64_t)key * kAttnD + lk_col);
        vr = *reinterpret_cast<const uint4*>(Vh + (int64_t)lv_dim * v_rows + key0 + lv_col);
    };
    auto lstore = [&](int buf, const uint4& kr, const uint4& vr) {
        *reinterpret_cast<uint4*>(&ks[buf][lk_key][lk_col]) = kr;
        *reinterpret_cast<uint4*>(&vs[buf][lv_dim][lv_col]) = vr;
    };
    uint4 kreg, vreg;
    if (n_blocks > 0) {
        gload(kbeg, kreg, vreg);
        lstore(0, kreg, vreg);
    }
    __syncthreads();

    for (int b = 0; b < n_blocks; ++b) {
        const int key0 = kbeg + 32 * b;
        const int buf = b & 1;
        if (b + 1 < n_blocks) gload(key0 + 32, kreg, vreg);   // next block in flight
        if (wave_active) {
            AFrag kf[2][4], vf[8];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    kf[kh][s].u = *reinterpret_cast<const uint4*>(&ks[buf][16 * kh + l16][32 * s + 8 * g]);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
                vf[dt].u = *reinterpret_cast<const uint4*>(&vs[buf][16 * dt + l16][8 * g]);
            // scores of both query blocks: four independent accumulation chains
            f32x4_t st[2][2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) st[qb][kh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int kh = 0; kh < 2; ++kh)
                        st[qb][kh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            kf[kh][s].b, qf[qb][s].b, st[qb][kh], 0, 0, 0);
            AFrag pf[2], pl[2];
            float alpha[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int64_t qpos = q_pos0 + qm[qb];
                float sc[8];
                float mx = -INFINITY;
#pragma unroll
                for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int key = key0 + 16 * kh + 4 * g + j;
                        bool ok = key < kend;
                        if (CAUSAL) ok = ok && key <= qpos;
                        const float v = ok ? st[qb][kh][j] * scale_log2 : -INFINITY;
                        sc[4 * kh + j] = v;
                        mx = fmaxf(mx, v);
                    }
                mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const float m_new = fmaxf(m_run[qb], mx);
                const float base = (m_new == -INFINITY) ? 0.f : m_new;
                alpha[qb] = exp2f(m_run[qb] - base);
                float psum = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float p = exp2f(sc[i] - base);
                    psum += p;
                    const __bf16 hi = (__bf16)p;                 // round to nearest even
                    pf[qb].b[i] = hi;
                    pl[qb].b[i] = (__bf16)(p - (float)hi);
                }
                l_run[qb] = l_run[qb] * alpha[qb] + psum;
                m_run[qb] = m_new;
            }
            // O^T = alpha O^T + V^T P^T: sixteen independent accumulators, hi parts then
            // lo parts (the accumulation into C rounds to nearest even, so the chain over
            // the key blocks costs no more than fp32 summation)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) o[qb][dt] *= alpha[qb];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
                    o[qb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt].b, pf[qb].b,
                                                                        o[qb][dt], 0, 0, 0);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
                    o[qb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt].b, pl[qb].b,
                                                                        o[qb][dt], 0, 0, 0);
        }
        if (b + 1 < n_blocks) lstore(buf ^ 1, kreg, vreg);
        __syncthreads();
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
                *reinterpret_cast<uint2*>(dst + 16 * dt + 4 * g) = pk;
            }
        } else {
            const int64_t pr = ((int64_t)split * Hq + h) * M + q;
            float* dst = part_o + pr * kAttnD;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
                *reinterpret_cast<f32x4_t*>(dst + 16 * dt + 4 * g) = o[qb][dt];
            if (g == 0) {
                part_ml[pr * 2 + 0] = m_run[qb];
                part_ml[pr * 2 + 1] = l;
            }
        }
    }
}

// Fixed-order combine of the key splits: O = sum_s 2^(m_s - m*) O_s / sum_s 2^(m_s - m*) l_s.
// One wave per (query, head); each lane owns two of the 128 dimensions.
template <typename T>
__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      int n_splits, int Hq, int M,
                                                      T* __restrict__ O) {
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (wid >= M * Hq) return;
    const int q = wid / Hq, h = wid % Hq;
    // lane s holds split s's statistics (n_splits <= 64); every split wrote its partials
    float ms = -INFINITY, ls = 0.f;
    if (lane < n_splits) {
        const float2 ml = *reinterpret_cast<const float2*>(
            part_ml + ((((int64_t)lane * Hq + h) * M + q) * 2));
        ms = ml.x;
        ls = ml.y;
    }
    const float mstar = wave_max(ms);
    const float wgt = (ms == -INFINITY) ? 0.f : exp2f(ms - mstar);
    const float den = wave_sum(wgt * ls);
    float n0 = 0.f, n1 = 0.f;
#pragma unroll 8
    for (int s = 0; s < n_splits; ++s) {
        const float ws = __shfl(wgt, s, 64);
        const int64_t pr = ((int64_t)s * Hq + h) * M + q;
        const float2 v = *reinterpret_cast<const float2*>(part_o + pr * kAttnD + 2 * lane);
        n0 += ws * v.x;
        n1 += ws * v.y;
    }
    T* dst = O + (int64_t)q * Hq * kAttnD + (int64_t)h * kAttnD + 2 * lane;
    dst[0] = from_f32<T>(n0 / den);
    dst[1] = from_f32<T>(n1 / den);
}

// f32 attention (VALU): one thread per (head, query), online softmax over keys.
template <int D>
__global__ __launch_bounds__(64) void k_attn_f32(const float* __restrict__ Q,
                                                 const float* __restrict__ K,
                                                 const float* __restrict__ V, int Hq, int Hkv,
                                                 int M, int S, int64_t rows, float scale,
                                                 int causal, int64_t q_pos0,
                                                 float* __restrict__ O) {
    const int q = blockIdx.x * 64 + threadIdx.x;
    const int h = blockIdx.y;
    if (q >= M) return;
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
        float s = 0.f;
#pragma unroll
        for (int t = 0; t < D; ++t) s = fmaf(qv[t], Kh[(int64_t)j * D + t], s);
        const float mn = fmaxf(m, s);
        const float a = expf(m - mn), p = expf(s - mn);
        l = l * a + p;
#pragma unroll
        for (int t = 0; t < D; ++t) ov[t] = ov[t] * a + p * Vh[(int64_t)j * D + t];
        m = mn;
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int t = 0; t < D; ++t) O[(int64_t)q * Hq * D + (int64_t)h * D + t] = ov[t] * inv;
}

// ================================================================== launchers
// Splits of the key range: about 256 workgroups in total, at least 256 keys each.
static int attn_splits(int Hq, int Hkv, int M, int S) {
    const int G = Hq / Hkv;
    const int qwgs = Hkv * ((G * M + kAttnRows - 1) / kAttnRows);
    int n = (256 + qwgs - 1) / qwgs;
    const int max_by_keys = (S + 255) / 256;
    if (n > max_by_keys) n = max_by_keys;
    if (n > 64) n = 64;
    return n < 1 ? 1 : n;
}

int64_t attention_part_floats(int dtype, int Hq, int Hkv, int M, int S, int D) {
    if (dtype == kF32) return 0;
    const int n = attn_splits(Hq, Hkv, M, S);
    return n > 1 ? (int64_t)n * Hq * M * (D + 2) : 0;
}

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    if (dtype == kF32) {
        dim3 grid((a.M + 63) / 64, a.Hq);
        if (a.D == 64)
            k_attn_f32<64><<<grid, 64, 0, s>>>((const float*)a.q, (const float*)a.k,
                                               (const float*)a.v, a.Hq, a.Hkv, a.M, a.S,
                                               a.kv_rows, a.scale, a.causal, a.q_pos0,
                                               (float*)a.o);
        else if (a.D == 128)
            k_attn_f32<128><<<grid, 64, 0, s>>>((const float*)a.q, (const float*)a.k,
                                                (const float*)a.v, a.Hq, a.Hkv, a.M, a.S,
                                                a.kv_rows, a.scale, a.causal, a.q_pos0,
                                                (float*)a.o);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
    if (a.D != kAttnD || (a.v_rows & 31) || a.v_rows < a.S || a.kv_rows < a.S)
        return hipErrorInvalidValue;
    int n = attn_splits(a.Hq, a.Hkv, a.M, a.S);
    int kps = (a.S + n - 1) / n;
    kps = (kps + 31) & ~31;
    n = (a.S + kps - 1) / kps;
    if (n > 1 && (int64_t)n * a.Hq * a.M * (a.D + 2) > a.part_capacity) return hipErrorInvalidValue;
    const int G = a.Hq / a.Hkv;
    dim3 grid((G * a.M + kAttnRows - 1) / kAttnRows, a.Hkv, n);
    const float sl2 = a.scale * 1.4426950408889634f;
    float* pml = a.part_o + (int64_t)n * a.Hq * a.M * a.D;
    if (a.causal)
        k_attn_bf16<true><<<grid, 512, 0, s>>>((const bf16_t*)a.q, (const bf16_t*)a.k,
                                               (const bf16_t*)a.v, a.Hq, a.Hkv, a.M, a.S,
                                               a.kv_rows, a.v_rows, sl2, a.q_pos0, kps, n,
                                               (bf16_t*)a.o, a.part_o, pml);
    else
        k_attn_bf16<false><<<grid, 512, 0, s>>>((const bf16_t*)a.q, (const bf16_t*)a.k,
                                                (const bf16_t*)a.v, a.Hq, a.Hkv, a.M, a.S,
                                                a.kv_rows, a.v_rows, sl2, a.q_pos0, kps, n,
                                                (bf16_t*)a.o, a.part_o, pml);
    if (n > 1)
        k_attn_combine<bf16_t><<<(a.M * a.Hq + 3) / 4, 256, 0, s>>>(a.part_o, pml, n, a.Hq, a.M,
                                                                    (bf16_t*)a.o);
    return hipGetLastError();
}

}  // namespace dg
