// Tied LM head with a streaming vocabulary epilogue (gfx950).
//
// Logits L_t = Decoder(x_t, z_t, H) in R^{C x V} and p0 = Softmax(L_t / tau)
// (DiffusionGemma technical-report summary, Method: decoder and update
// equations); the head is tied to the token embedding E in R^{V x d}.
// The C x V logits are never stored: each workgroup reduces its vocabulary
// slice to per-row partials (max, lowest argmax, sum of exp(z - max)) and, for
// rows still unlocked, the Gumbel-max redraw (best z + G and its id) with
// Philox4x32-10 uniforms drawn per (vocabulary id, position).
#include "kernels.h"

namespace dg {

constexpr int kHeadRows = 256;    // rows per workgroup (4 waves x 64)
constexpr int kHeadCols = 128;    // vocabulary ids per workgroup (8 MFMA column groups)

union HFrag {
    uint4 u;
    bf16x8_t b;
};

struct Run {
    float m;
    int32_t a;
    float s;
    float g;
    int32_t gi;
};

DG_DEV void run_merge(Run& x, float ym, int32_t ya, float ys, float yg, int32_t ygi) {
    if (ym > x.m || (ym == x.m && ya < x.a)) {
        x.s = ys + (x.m == -INFINITY ? 0.f : x.s * __expf(x.m - ym));
        x.m = ym;
        x.a = ya;
    } else {
        x.s += (ym == -INFINITY ? 0.f : ys * __expf(ym - x.m));
    }
    if (yg > x.g || (yg == x.g && ygi < x.gi)) { x.g = yg; x.gi = ygi; }
}

DG_DEV float gumbel_of(uint32_t w) { return -logf(-logf(philox_open_uniform(w))); }

__global__ __launch_bounds__(256) void k_lm_head_bf16(
    const bf16_t* __restrict__ Hn, int C, int d, const bf16_t* __restrict__ Ep, int V,
    float inv_tau, const uint8_t* __restrict__ mask, uint32_t key0, uint32_t key1, uint32_t c2,
    HeadPartials p, float* __restrict__ logits_out) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const int v0 = blockIdx.x * kHeadCols;
    const int rbase = blockIdx.y * kHeadRows + 64 * w;
    if (rbase >= C) return;   // no block-level synchronisation in this kernel
    const int KB = d >> 5;
    f32x4_t acc[4][8];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const bf16_t* arow[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        int r = rbase + 16 * mt + l16;
        r = r < C ? r : C - 1;
        arow[mt] = Hn + (size_t)r * d + 8 * g;
    }
    const size_t gstride = (size_t)KB * 512;
    const bf16_t* bgrp = Ep + (size_t)(v0 >> 4) * gstride + (size_t)lane * 8;
    HFrag ca[4], cb[8], na[4], nb[8];
    auto load = [&](int kb, HFrag (&fa)[4], HFrag (&fb)[8]) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) fa[mt].u = *reinterpret_cast<const uint4*>(arow[mt] + kb * 32);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
            fb[nt].u = *reinterpret_cast<const uint4*>(bgrp + nt * gstride + (size_t)kb * 512);
    };
    load(0, ca, cb);
    for (int kb = 0; kb < KB; ++kb) {
        if (kb + 1 < KB) load(kb + 1, na, nb);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca[mt].b, cb[nt].b,
                                                                      acc[mt][nt], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) ca[i] = na[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) cb[i] = nb[i];
    }
    // ---------------- epilogue: per row, fold the lane's 8 columns, then the 16 lanes
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int r4 = rbase + 16 * mt + 4 * g;      // rows r4 .. r4+3 in this lane
        bool unl[4];
        bool any = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            unl[j] = (r4 + j < C) && mask[r4 + j] == 0;
            any |= unl[j];
        }
        Run run[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) run[j] = Run{-INFINITY, 0x7fffffff, 0.f, -INFINITY, 0x7fffffff};
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const int v = v0 + 16 * nt + l16;
            u32x4 rw = {0u, 0u, 0u, 0u};
            if (any) rw = philox4x32_10(u32x4{(uint32_t)v, (uint32_t)(r4 >> 2), c2, kGumbelTag},
                                        key0, key1);
            const uint32_t words[4] = {rw.x, rw.y, rw.z, rw.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float z = acc[mt][nt][j] * inv_tau;
                if (logits_out != nullptr && r4 + j < C) logits_out[(size_t)(r4 + j) * V + v] = z;
                if (z > run[j].m) {
                    run[j].s = (run[j].m == -INFINITY ? 0.f : run[j].s * __expf(run[j].m - z)) + 1.f;
                    run[j].m = z;
                    run[j].a = v;
                } else {
                    run[j].s += __expf(z - run[j].m);
                }
                if (unl[j]) {
                    const float gs = z + gumbel_of(words[j]);
                    if (gs > run[j].g) { run[j].g = gs; run[j].gi = v; }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                const float ym = __shfl_xor(run[j].m, o, 64);
                const int32_t ya = __shfl_xor(run[j].a, o, 64);
                const float ys = __shfl_xor(run[j].s, o, 64);
                const float yg = __shfl_xor(run[j].g, o, 64);
                const int32_t ygi = __shfl_xor(run[j].gi, o, 64);
                run_merge(run[j], ym, ya, ys, yg, ygi);
            }
            if (l16 == 0 && r4 + j < C) {
                const size_t o = (size_t)(r4 + j) * p.n_slices + blockIdx.x;
                p.m[o] = run[j].m;
                p.a[o] = run[j].a;
                p.s[o] = run[j].s;
                p.g[o] = run[j].g;
                p.gi[o] = run[j].gi;
            }
        }
    }
}

// f32 head (VALU): one thread per (row, vocabulary id), workgroup = 256 ids of one row.
__global__ __launch_bounds__(256) void k_lm_head_f32(
    const float* __restrict__ Hn, int C, int d, const float* __restrict__ E, int V,
    float inv_tau, const uint8_t* __restrict__ mask, uint32_t key0, uint32_t key1, uint32_t c2,
    HeadPartials p, float* __restrict__ logits_out) {
    __shared__ Run sh[256];
    const int row = blockIdx.y;
    const int v = blockIdx.x * 256 + threadIdx.x;
    Run r = {-INFINITY, 0x7fffffff, 0.f, -INFINITY, 0x7fffffff};
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
            run_merge(x, y.m, y.a, y.s, y.g, y.gi);
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
    }
}

int lm_head_slices(int dtype, int V) {
    return dtype == kF32 ? (V + 255) / 256 : V / kHeadCols;
}

hipError_t launch_lm_head(int dtype, const void* h, int C, int d, const void* E, int V,
                          float inv_tau, const uint8_t* mask, uint64_t seed, int step, int k_blk,
                          const HeadPartials& p, float* logits_out, hipStream_t s) {
    const uint32_t key0 = (uint32_t)seed, key1 = (uint32_t)(seed >> 32);
    const uint32_t c2 = (uint32_t)step | ((uint32_t)k_blk << 16);
    if (dtype == kF32) {
        dim3 grid((V + 255) / 256, C);
        k_lm_head_f32<<<grid, 256, 0, s>>>((const float*)h, C, d, (const float*)E, V, inv_tau,
                                           mask, key0, key1, c2, p, logits_out);
    } else {
        if ((V % kHeadCols) || (d & 31)) return hipErrorInvalidValue;
        dim3 grid(V / kHeadCols, (C + kHeadRows - 1) / kHeadRows);
        k_lm_head_bf16<<<grid, 256, 0, s>>>((const bf16_t*)h, C, d, (const bf16_t*)E, V,
                                            inv_tau, mask, key0, key1, c2, p, logits_out);
    }
    return hipGetLastError();
}

}  // namespace dg
