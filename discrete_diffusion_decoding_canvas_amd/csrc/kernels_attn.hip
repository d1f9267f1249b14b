// Attention over [KV cache || canvas] for gfx950.
//
// The decoder attends bidirectionally across the canvas and to the context KV
// cache; the causal encoder (prefill / commit) attends causally
// (DiffusionGemma technical-report summary, Method: generation pipeline;
// alphasignal, paragraph on bidirectional attention: every canvas position
// attends to every other).  GQA: query head h reads KV head h / (Hq / Hkv).
//
// bf16 kernel (D = 128), one wave per 32 queries of one head, four waves per
// workgroup, split over keys for occupancy with a fixed-order combine:
//   S^T = K Q^T  (v_mfma_f32_16x16x32_bf16, A = K rows, B = Q rows) puts the
//   scores of one query in one lane column, so the online-softmax statistics
//   and the rescale of the output stay lane-local;
//   O^T = V^T P^T (A = V^T from the transposed, key-permuted V cache, B = P
//   taken straight from the score registers) needs no shuffle of P.
// Softmax runs in fp32 in the log2 domain (exp2), scale applied to fp32 scores.
#include "kernels.h"

namespace dg {

constexpr int kAttnD = 128;
constexpr int kAttnWaveQ = 32;
constexpr int kAttnBlockQ = 128;

union AFrag {
    uint4 u;
    bf16x8_t b;
    uint16_t h[8];
};

template <bool CAUSAL>
__global__ __launch_bounds__(256) void k_attn_bf16(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ Vt,
    int Hq, int Hkv, int M, int S, int64_t k_rows, int64_t v_rows, float scale_log2,
    int64_t q_pos0, int keys_per_split, int n_splits, bf16_t* __restrict__ O, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
    const int G = Hq / Hkv;
    const int qtiles = (M + kAttnBlockQ - 1) / kAttnBlockQ;
    const int kvh = blockIdx.y;
    const int h = kvh * G + blockIdx.x / qtiles;
    const int qt = blockIdx.x % qtiles;
    const int split = blockIdx.z;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const int qbase = qt * kAttnBlockQ + w * kAttnWaveQ;
    if (qbase >= M) return;   // no block-level synchronisation below

    int kbeg = split * keys_per_split;
    int kend = kbeg + keys_per_split < S ? kbeg + keys_per_split : S;
    if (CAUSAL) {
        const int qlast = qbase + kAttnWaveQ - 1 < M ? qbase + kAttnWaveQ - 1 : M - 1;
        const int64_t lim = q_pos0 + qlast + 1;
        if (lim < kend) kend = (int)lim;
    }

    // Q fragments (B operand of S^T): query row, dims 32s + 8g .. +7
    AFrag qf[2][4];
    int qrow[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        int q = qbase + 16 * qb + l16;
        qrow[qb] = q;
        q = q < M ? q : M - 1;
        const bf16_t* src = Q + ((int64_t)h * M + q) * kAttnD + 8 * g;
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

    const bf16_t* Kh = K + (int64_t)kvh * k_rows * kAttnD;
    const bf16_t* Vh = Vt + (int64_t)kvh * kAttnD * v_rows;
    for (int key0 = kbeg; key0 < kend; key0 += 32) {
        AFrag kf[2][4];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            int kr = key0 + 16 * kh + l16;
            kr = kr < S ? kr : S - 1;
            const bf16_t* src = Kh + (int64_t)kr * kAttnD + 8 * g;
#pragma unroll
            for (int s = 0; s < 4; ++s) kf[kh][s].u = *reinterpret_cast<const uint4*>(src + 32 * s);
        }
        AFrag vf[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
            vf[dt].u = *reinterpret_cast<const uint4*>(Vh + (int64_t)(16 * dt + l16) * v_rows +
                                                       key0 + 8 * g);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            f32x4_t st[2];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                st[kh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    st[kh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kh][s].b, qf[qb][s].b,
                                                                     st[kh], 0, 0, 0);
            }
            float sc[8];
            const int64_t qpos = q_pos0 + qrow[qb];
            float mx = -INFINITY;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int key = key0 + 16 * kh + 4 * g + j;
                    bool ok = key < kend;
                    if (CAUSAL) ok = ok && key <= qpos;
                    float v = ok ? st[kh][j] * scale_log2 : -INFINITY;
                    sc[4 * kh + j] = v;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m_run[qb], mx);
            const float base = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = exp2f(m_run[qb] - base);
            // P = hi + lo in two bf16 parts (~16 significant bits): the softmax
            // weights stay fp32-accurate through the bf16 MFMA.
            float psum = 0.f;
            AFrag pf, pl;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p = exp2f(sc[i] - base);
                psum += p;
                const bf16_t hi = f32_to_bf16(p);
                pf.h[i] = hi;
                pl.h[i] = f32_to_bf16(p - bf16_to_f32(hi));
            }
            l_run[qb] = l_run[qb] * alpha + psum;
            m_run[qb] = m_new;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                o[qb][dt] *= alpha;
                o[qb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt].b, pf.b, o[qb][dt],
                                                                    0, 0, 0);
                o[qb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt].b, pl.b, o[qb][dt],
                                                                    0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float l = l_run[qb];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        const int q = qrow[qb];
        if (q >= M) continue;
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
template <typename T>
__global__ void k_attn_combine(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                               int n_splits, int Hq, int M, int D, T* __restrict__ O) {
    const int q = blockIdx.x, h = blockIdx.y;
    float mstar = -INFINITY;
    for (int s = 0; s < n_splits; ++s)
        mstar = fmaxf(mstar, part_ml[(((int64_t)s * Hq + h) * M + q) * 2]);
    for (int t = threadIdx.x; t < D; t += blockDim.x) {
        float num = 0.f, den = 0.f;
        for (int s = 0; s < n_splits; ++s) {
            const int64_t pr = ((int64_t)s * Hq + h) * M + q;
            const float ms = part_ml[pr * 2];
            if (ms == -INFINITY) continue;
            const float wgt = exp2f(ms - mstar);
            num += wgt * part_o[pr * D + t];
            den += wgt * part_ml[pr * 2 + 1];
        }
        O[(int64_t)q * Hq * D + (int64_t)h * D + t] = from_f32<T>(num / den);
    }
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
static int attn_splits(int Hq, int M, int S) {
    const int qwgs = Hq * ((M + kAttnBlockQ - 1) / kAttnBlockQ);
    int n = (512 + qwgs - 1) / qwgs;
    const int max_by_keys = (S + 255) / 256;      // at least 256 keys per split
    if (n > max_by_keys) n = max_by_keys;
    if (n > 64) n = 64;
    return n < 1 ? 1 : n;
}

int64_t attention_part_floats(int dtype, int Hq, int M, int S, int D) {
    if (dtype == kF32) return 0;
    const int n = attn_splits(Hq, M, S);
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
    int n = attn_splits(a.Hq, a.M, a.S);
    int kps = (a.S + n - 1) / n;
    kps = (kps + 31) & ~31;
    n = (a.S + kps - 1) / kps;
    if (n > 1 && (int64_t)n * a.Hq * a.M * (a.D + 2) > a.part_capacity) return hipErrorInvalidValue;
    const int G = a.Hq / a.Hkv;
    dim3 grid(G * ((a.M + kAttnBlockQ - 1) / kAttnBlockQ), a.Hkv, n);
    const float sl2 = a.scale * 1.4426950408889634f;
    float* pml = a.part_o + (int64_t)n * a.Hq * a.M * a.D;
    if (a.causal)
        k_attn_bf16<true><<<grid, 256, 0, s>>>((const bf16_t*)a.q, (const bf16_t*)a.k,
                                               (const bf16_t*)a.v, a.Hq, a.Hkv, a.M, a.S,
                                               a.kv_rows, a.v_rows, sl2, a.q_pos0, kps, n,
                                               (bf16_t*)a.o, a.part_o, pml);
    else
        k_attn_bf16<false><<<grid, 256, 0, s>>>((const bf16_t*)a.q, (const bf16_t*)a.k,
                                                (const bf16_t*)a.v, a.Hq, a.Hkv, a.M, a.S,
                                                a.kv_rows, a.v_rows, sl2, a.q_pos0, kps, n,
                                                (bf16_t*)a.o, a.part_o, pml);
    if (n > 1)
        k_attn_combine<bf16_t><<<dim3(a.M, a.Hq), 128, 0, s>>>(a.part_o, pml, n, a.Hq, a.M,
                                                               a.D, (bf16_t*)a.o);
    return hipGetLastError();
}

}  // namespace dg
