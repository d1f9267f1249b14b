// Tied LM head with a streaming vocabulary epilogue (gfx950).
//
// Logits L_t = Decoder(x_t, z_t, H) in R^{C x V} and p0 = Softmax(L_t / tau)
// (DiffusionGemma technical-report summary, Method: decoder and update
// equations); the head is tied to the token embedding E in R^{V x d}.
// The C x V logits are never stored: each vocabulary slice is reduced to
// per-row partials (max, lowest argmax, sum of exp(z - max)) and, for
// rows still unlocked, the Gumbel-max redraw (best z + G and its id) with
// Philox4x32-10 uniforms drawn per (vocabulary id, position).  ENT adds the
// weighted sum q = sum exp(z - max) (z - max) of the predictive entropy.
#include "head_epilogue.h"

namespace dg {

// f32 head (VALU): one thread per (row, vocabulary id), workgroup = 256 ids of one row.
template <bool ENT>
__global__ __launch_bounds__(256) void k_lm_head_f32(
    const float* __restrict__ Hn, int C, int d, const float* __restrict__ E, int V,
    float inv_tau, const uint8_t* __restrict__ mask, uint32_t key0, uint32_t key1, uint32_t c2,
    HeadPartials p, float* __restrict__ logits_out) {
    __shared__ Run sh[256];
    const int row = blockIdx.y;
    const int v = blockIdx.x * 256 + threadIdx.x;
    Run r = {-INFINITY, 0x7fffffff, 0.f, -INFINITY, 0x7fffffff, 0.f};
    if (v < V) {
        const float* h = Hn + (size_t)row * d;
        const float* e = E + (size_t)v * d;
        float acc = 0.f;
        for (int k = 0; k < d; ++k) acc = fmaf(h[k], e[k], acc);
        const float z = acc * inv_tau;
        if (logits_out) logits_out[(size_t)row * V + v] = z;
        r.m = z;
        r.a = v;
        r.s = 1.f;
        if (mask[row] == 0) {
            u32x4 rw = philox4x32_10(u32x4{(uint32_t)v, (uint32_t)(row >> 2), c2, kGumbelTag},
                                     key0, key1);
            const uint32_t words[4] = {rw.x, rw.y, rw.z, rw.w};
            r.g = z + gumbel_of(words[row & 3]);
            r.gi = v;
        }
    }
    sh[threadIdx.x] = r;
    __syncthreads();
    for (int wdt = 128; wdt > 0; wdt >>= 1) {
        if (threadIdx.x < wdt) {
            Run x = sh[threadIdx.x];
            const Run y = sh[threadIdx.x + wdt];
            run_merge<ENT>(x, y.m, y.a, y.s, y.g, y.gi, y.q);
            sh[threadIdx.x] = x;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const size_t o = (size_t)row * p.n_slices + blockIdx.x;
        p.m[o] = sh[0].m;
        p.a[o] = sh[0].a;
        p.s[o] = sh[0].s;
        p.g[o] = sh[0].g;
        p.gi[o] = sh[0].gi;
        if constexpr (ENT) p.q[o] = sh[0].q;
    }
}

int lm_head_slices(int dtype, int V) {
    return dtype == kF32 ? (V + 255) / 256 : V / kHeadCols;
}

hipError_t launch_lm_head(int dtype, const void* h, const void* hf, int C, int d, const void* E,
                          int V, float inv_tau, const uint8_t* mask, uint64_t seed, int step,
                          int k_blk, const HeadPartials& p, float* logits_out, hipStream_t s,
                          uint16_t* sc_w) {
    const uint32_t key0 = (uint32_t)seed, key1 = (uint32_t)(seed >> 32);
    const uint32_t c2 = (uint32_t)step | ((uint32_t)k_blk << 16);
    if (dtype != kF32 && hf != nullptr)
        return launch_head_wide(hf, C, d, E, V, inv_tau, mask, key0, key1, c2, p, logits_out, s,
                                sc_w);
    if (dtype != kF32 || sc_w != nullptr) return hipErrorInvalidValue;   // bf16 rows come in fragment order
    dim3 grid((V + 255) / 256, C);
    auto k = p.q ? k_lm_head_f32<true> : k_lm_head_f32<false>;
    k<<<grid, 256, 0, s>>>((const float*)h, C, d, (const float*)E, V, inv_tau, mask, key0, key1,
                           c2, p, logits_out);
    return hipGetLastError();
}

}  // namespace dg
