// Tied LM head with a streaming vocabulary epilogue (gfx950).
//
// Logits L_t = Decoder(x_t, z_t, H) in R^{C x V} and p0 = Softmax(L_t / tau)
// (DiffusionGemma technical-report summary, Method: decoder and update
// equations); the head is tied to the token embedding E in R^{V x d}.
// The C x V logits are never stored: each workgroup reduces its vocabulary
// slice to per-row partials (max, lowest argmax, sum of exp(z - max)) and, for
// rows still unlocked, the Gumbel-max redraw (best z + G and its id) with
// Philox4x32-10 uniforms drawn per (vocabulary id, position).  ENT adds the
// weighted sum q = sum exp(z - max) (z - max) of the predictive entropy.
#include "head_epilogue.h"

namespace dg {

// bf16 head: workgroup of 8 waves owns 256 rows x 256 vocabulary ids; per
// k-step of 32 the rows' and the ids' slices are copied cooperatively into
// double-buffered LDS in MFMA fragment order (the embedding is packed that way
// at load time, so its copy is contiguous), and each wave (64 rows x 128 ids)
// reads its fragments from LDS.
template <bool ENT>
__global__ __launch_bounds__(512) void k_lm_head_bf16(
    const bf16_t* __restrict__ Hn, int C, int d, const bf16_t* __restrict__ Ep, int V,
    float inv_tau, const uint8_t* __restrict__ mask, uint32_t key0, uint32_t key1, uint32_t c2,
    HeadPartials p, float* __restrict__ logits_out) {
    __shared__ __attribute__((aligned(16))) uint4 a_lds[2][16][64];   // 16 row groups x 1 KiB
    __shared__ __attribute__((aligned(16))) uint4 b_lds[2][16][64];   // 16 id groups x 1 KiB
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const int wr = w & 3, wc = w >> 2;
    const int row_base = blockIdx.y * kHeadRows;
    const int v0 = blockIdx.x * kHeadTile + kHeadCols * wc;   // this wave's first id
    const int rbase = row_base + 64 * wr;
    const int KB = d >> 5;
    f32x4_t acc[4][8];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // cooperative copy of one k-step: pieces tid and tid + 512 of A (256 rows) and of
    // B (256 ids); a piece is one fragment lane (16 bytes) of one 16-row / 16-id group
    const int pg0 = tid >> 6, pg1 = pg0 + 8;
    const int chunk = lane >> 4;
    int ar0 = row_base + 16 * pg0 + l16, ar1 = row_base + 16 * pg1 + l16;
    ar0 = ar0 < C ? ar0 : C - 1;
    ar1 = ar1 < C ? ar1 : C - 1;
    const uint4* a0 = reinterpret_cast<const uint4*>(Hn + (size_t)ar0 * d + 8 * chunk);
    const uint4* a1 = reinterpret_cast<const uint4*>(Hn + (size_t)ar1 * d + 8 * chunk);
    const size_t gstride = (size_t)KB * 64;   // uint4 per 16-id group
    const uint4* b0 = reinterpret_cast<const uint4*>(Ep) +
                      (size_t)(blockIdx.x * (kHeadTile / 16) + pg0) * gstride + lane;
    const uint4* b1 = b0 + 8 * gstride;
    uint4 ra0 = a0[0], ra1 = a1[0], rb0 = b0[0], rb1 = b1[0];
    a_lds[0][pg0][lane] = ra0;
    a_lds[0][pg1][lane] = ra1;
    b_lds[0][pg0][lane] = rb0;
    b_lds[0][pg1][lane] = rb1;
    __syncthreads();
    for (int kb = 0; kb < KB; ++kb) {
        const int buf = kb & 1;
        const bool more = kb + 1 < KB;
        if (more) {
            ra0 = a0[4 * (kb + 1)];      // 32 bf16 = 4 uint4 per k-step along a row
            ra1 = a1[4 * (kb + 1)];
            rb0 = b0[64 * (kb + 1)];
            rb1 = b1[64 * (kb + 1)];
        }
        HFrag fa[4], fb[8];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) fa[mt].u = a_lds[buf][4 * wr + mt][lane];
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) fb[nt].u = b_lds[buf][8 * wc + nt][lane];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mt].b, fb[nt].b,
                                                                      acc[mt][nt], 0, 0, 0);
        if (more) {
            a_lds[buf ^ 1][pg0][lane] = ra0;
            a_lds[buf ^ 1][pg1][lane] = ra1;
            b_lds[buf ^ 1][pg0][lane] = rb0;
            b_lds[buf ^ 1][pg1][lane] = rb1;
        }
        __syncthreads();
    }
    if (rbase >= C) return;
    const EpiArgs ea{C, V, v0, rbase, g, l16, inv_tau, mask, key0, key1, c2, p, logits_out};
    head_epilogue<0, ENT>(acc[0], ea);
    head_epilogue<1, ENT>(acc[1], ea);
    head_epilogue<2, ENT>(acc[2], ea);
    head_epilogue<3, ENT>(acc[3], ea);
}

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
                          int k_blk, const HeadPartials& p, float* logits_out, hipStream_t s) {
    const uint32_t key0 = (uint32_t)seed, key1 = (uint32_t)(seed >> 32);
    const uint32_t c2 = (uint32_t)step | ((uint32_t)k_blk << 16);
    if (dtype != kF32 && hf != nullptr)
        return launch_head_wide(hf, C, d, E, V, inv_tau, mask, key0, key1, c2, p, logits_out, s);
    if (dtype == kF32) {
        dim3 grid((V + 255) / 256, C);
        auto k = p.q ? k_lm_head_f32<true> : k_lm_head_f32<false>;
        k<<<grid, 256, 0, s>>>((const float*)h, C, d, (const float*)E, V, inv_tau, mask, key0, key1,
                               c2, p, logits_out);
    } else {
        if ((V % kHeadTile) || (d & 31)) return hipErrorInvalidValue;
        dim3 grid(V / kHeadTile, (C + kHeadRows - 1) / kHeadRows);
        auto k = p.q ? k_lm_head_bf16<true> : k_lm_head_bf16<false>;
        k<<<grid, 512, 0, s>>>((const bf16_t*)h, C, d, (const bf16_t*)E, V, inv_tau, mask, key0,
                               key1, c2, p, logits_out);
    }
    return hipGetLastError();
}

}  // namespace dg
