// Streaming vocabulary epilogue of the tied LM head (device code shared by the
// head kernels).
//
// Logits L_t = Decoder(x_t, z_t, H) in R^{C x V} and p0 = Softmax(L_t / tau)
// (DiffusionGemma technical-report summary, Method: decoder and update
// equations).  The C x V logits are never stored: each wave reduces its
// 128-id vocabulary slice to per-row partials (max, lowest argmax, sum of
// exp(z - max)) and, for rows still unlocked, the Gumbel-max redraw (best
// z + G and its id) with Philox4x32-10 uniforms drawn per (vocabulary id,
// position).  With ENT it also keeps q = sum exp(z - max) (z - max), from which
// the predictive entropy of the row is log s - q / s (the entropy-bounded
// sampler ranks positions by it: technical-report summary, Method, sampler
// paragraph).  When the pass forms the self-conditioning signal z = FFW(p0 E)
// (same page, update equations) it also stores exp(z - max) of every logit in
// bf16: the posterior rows up to one factor per (row, slice).
#pragma once

#include "kernels.h"

namespace dg {

constexpr int kHeadCols = kHeadSlice;    // vocabulary ids of one partial slice (one weight slab)

struct Run {
    float m;
    int32_t a;
    float s;
    float g;
    int32_t gi;
    float q;
};

// Absorb y into x.  Rescaling a slice's sums from its max m_i to m multiplies s
// by f = exp(m_i - m) and turns q into f (q + (m_i - m) s).
template <bool ENT = false>
DG_DEV void run_merge(Run& x, float ym, int32_t ya, float ys, float yg, int32_t ygi,
                      float yq = 0.f) {
    if (ym > x.m || (ym == x.m && ya < x.a)) {
        if constexpr (ENT) {
            const float f = x.m == -INFINITY ? 0.f : __expf(x.m - ym);
            x.q = yq + (f == 0.f ? 0.f : f * fmaf(x.m - ym, x.s, x.q));
            x.s = ys + f * x.s;
        } else {
            x.s = ys + (x.m == -INFINITY ? 0.f : x.s * __expf(x.m - ym));
        }
        x.m = ym;
        x.a = ya;
    } else {
        if constexpr (ENT) {
            const float f = ym == -INFINITY ? 0.f : __expf(ym - x.m);
            x.q += f == 0.f ? 0.f : f * fmaf(ym - x.m, ys, yq);
            x.s += f * ys;
        } else {
            x.s += (ym == -INFINITY ? 0.f : ys * __expf(ym - x.m));
        }
    }
    if (yg > x.g || (yg == x.g && ygi < x.gi)) { x.g = yg; x.gi = ygi; }
}

// Gumbel noise G = -ln(-ln u) from the hardware base-2 logarithm: u >= 2^-24 and
// -ln u >= 2^-24 are normal floats, so no denormal scaling is needed.
DG_DEV float gumbel_of(uint32_t w) {
    constexpr float kLn2 = 0.69314718055994531f;
    const float t = -__builtin_amdgcn_logf(philox_open_uniform(w)) * kLn2;   // -ln u > 0
    return -__builtin_amdgcn_logf(t) * kLn2;
}

struct EpiArgs {
    int C, V, v0, rbase, g, l16;
    float inv_tau;
    const uint8_t* mask;
    uint32_t key0, key1, c2;
    HeadPartials p;
    float* logits_out;
    uint16_t* sc_w;    // bf16 [C][V] exp(z - slice max), or nullptr
};

// Epilogue of one 16-row fragment group MT of a wave's 16 x 128 tile: each lane
// holds 8 columns (ids v0 + 16 nt + l16, increasing with nt) of 4 rows.  Per row it
// takes the maximum and its first id and the Gumbel best in one pass over the 8
// columns, then the sum of exp(z - max) in a second (one exponential per element);
// the 16 lanes sharing the rows then merge.  MT is a template argument so that
// every accumulator index is static.
template <int MT, bool ENT = false>
DG_DEV void head_epilogue(const f32x4_t (&acc)[8], const EpiArgs& e) {
    constexpr float kLog2e = 1.4426950408889634f;
    const int r4 = e.rbase + 16 * MT + 4 * e.g;      // rows r4 .. r4+3 in this lane
    bool unl[4];
    bool any = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        unl[j] = (r4 + j < e.C) && e.mask[r4 + j] == 0;
        any |= unl[j];
    }
    float m[4], g[4];
    int am[4], ag[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        m[j] = -INFINITY;
        g[j] = -INFINITY;
        am[j] = 0;
        ag[j] = -1;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
        const int v = e.v0 + 16 * nt + e.l16;
        u32x4 rw = {0u, 0u, 0u, 0u};
        if (any) rw = philox4x32_10(u32x4{(uint32_t)v, (uint32_t)(r4 >> 2), e.c2, kGumbelTag},
                                    e.key0, e.key1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float z = acc[nt][j] * e.inv_tau;
            if (e.logits_out != nullptr && r4 + j < e.C) e.logits_out[(size_t)(r4 + j) * e.V + v] = z;
            if (z > m[j]) { m[j] = z; am[j] = nt; }
            if (unl[j]) {
                const uint32_t word = j == 0 ? rw.x : j == 1 ? rw.y : j == 2 ? rw.z : rw.w;
                const float gs = z + gumbel_of(word);
                if (gs > g[j]) { g[j] = gs; ag[j] = nt; }
            }
        }
    }
    Run run[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float s = 0.f, q = 0.f;
        if (m[j] != -INFINITY) {
            if constexpr (ENT) {
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) {
                    const float dz = acc[nt][j] * e.inv_tau - m[j];      // z - max, 0 at the max
                    const float ex = __builtin_amdgcn_exp2f(dz * kLog2e);
                    s += ex;
                    q = fmaf(ex, dz, q);
                }
            } else {
                const float mb = m[j] * kLog2e;
#pragma unroll
                for (int nt = 0; nt < 8; ++nt)
                    s += __builtin_amdgcn_exp2f(fmaf(acc[nt][j] * e.inv_tau, kLog2e, -mb));
            }
        }
        run[j] = Run{m[j], m[j] == -INFINITY ? 0x7fffffff : e.v0 + 16 * am[j] + e.l16, s, g[j],
                     ag[j] < 0 ? 0x7fffffff : e.v0 + 16 * ag[j] + e.l16, q};
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
            if constexpr (ENT)
                run_merge<true>(run[j], ym, ya, ys, yg, ygi, __shfl_xor(run[j].q, o, 64));
            else
                run_merge(run[j], ym, ya, ys, yg, ygi);
        }
        if (e.l16 == 0 && r4 + j < e.C) {
            const size_t o = (size_t)(r4 + j) * e.p.n_slices + e.v0 / kHeadCols;
            e.p.m[o] = run[j].m;
            e.p.a[o] = run[j].a;
            e.p.s[o] = run[j].s;
            e.p.g[o] = run[j].g;
            e.p.gi[o] = run[j].gi;
            if constexpr (ENT) e.p.q[o] = run[j].q;
        }
    }
    // Unnormalised posterior of every row for the self-conditioning signal: exp(z - m)
    // with m the slice maximum the partials keep (every lane of the 16 holds it after
    // the merge), so that p0 = exp(z - m) exp(m - lse) once lse is known.
    if (e.sc_w != nullptr) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (r4 + j >= e.C) continue;
            const float mb = run[j].m * kLog2e;
            uint16_t* row = e.sc_w + (size_t)(r4 + j) * e.V + e.v0 + e.l16;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
                row[16 * nt] = f32_to_bf16(__builtin_amdgcn_exp2f(fmaf(acc[nt][j] * e.inv_tau, kLog2e, -mb)));
        }
    }
}

}  // namespace dg
