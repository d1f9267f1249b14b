// Element-wise, routing, permutation, statistics and sampler kernels (gfx950).
//
// Method steps (DiffusionGemma technical-report summary, Method; alphasignal
// "How text diffusion actually works"):
//   canvas embedding + RMSNorm, RoPE and K/V cache write, top-k router,
//   per-expert token permutation, weighted expert combine + residual,
//   per-position LM-head statistics, and the lock / redraw sampler.
#include "kernels.h"

namespace dg {

// Packed MFMA B-operand index of logical element (n, k) of a K x N matrix:
// [N/16][K/32][64 lanes][8], lane = n%16 + 16*((k%32)/8), element k%8.
DG_DEV size_t packed_b_index(int64_t n, int64_t k, int64_t K) {
    return ((size_t)((n >> 4) * (K >> 5) + (k >> 5)) << 9) +
           ((size_t)((n & 15) + (((k & 31) >> 3) << 4)) << 3) + (size_t)(k & 7);
}

// ------------------------------------------------------------------ block reductions
template <int NT>
DG_DEV float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) t += red[i];
    return t;
}

// ------------------------------------------------------------------ embed + RMSNorm
// x[i, :] = E[canvas[i], :] (+ zadd[i, :], the self-conditioning signal, when given;
// float residual), a[i, :] = rmsnorm(x[i, :]).
// An id outside [0, V) (caller data, or the argmax of a row whose logits were
// all NaN) reads as a zero row and sets bit kBadToken of *bad; no load leaves
// the table.
template <typename T, bool PACKED>
__global__ __launch_bounds__(256) void k_embed_rmsnorm(const int32_t* __restrict__ tokens,
                                                       const T* __restrict__ E, int V, int d,
                                                       float eps, float* __restrict__ x,
                                                       T* __restrict__ a, uint8_t* __restrict__ af,
                                                       int32_t* __restrict__ bad,
                                                       const float* __restrict__ zadd) {
    __shared__ float red[4];
    const int i = blockIdx.x;
    const int64_t v = tokens[i];
    const bool valid = v >= 0 && v < V;
    if (!valid && threadIdx.x == 0) atomicOr(bad, kBadToken);
    float xs[kCombineCols];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kCombineCols; ++j) {
        const int c = threadIdx.x + 256 * j;
        float e = 0.f;
        if (valid && c < d) e = PACKED ? to_f32<T>(E[packed_b_index(v, c, d)]) : to_f32<T>(E[v * d + c]);
        if (zadd != nullptr && c < d) e += zadd[(int64_t)i * d + c];
        xs[j] = e;
        ss += e * e;
    }
    const float r = rsqrtf(block_sum<256>(ss, red) / (float)d + eps);
#pragma unroll
    for (int j = 0; j < kCombineCols; ++j) {
        const int c = threadIdx.x + 256 * j;
        if (c < d) {
            x[(int64_t)i * d + c] = xs[j];
            const T av = from_f32<T>(xs[j] * r);
            a[(int64_t)i * d + c] = av;
            if (af) *reinterpret_cast<T*>(af + frag_offset<false>(i, c, d)) = av;
        }
    }
}

// ------------------------------------------------------------------ RMSNorm
// a = rmsnorm(x) (unit gains); a8 (optional) = e4m3(a) for fp8 expert inputs.
// One block of NT threads per row, four columns per thread per pass (d % 4 == 0):
// every load of the row is issued before the reduction.  d <= 4096.
#ifndef DG_ROW_THREADS
#define DG_ROW_THREADS 1024
#endif
constexpr int kRowThreads = DG_ROW_THREADS;    // block of the row kernels (norm, combine)
template <int NT>
constexpr int row_passes() { return 1024 / NT; }   // float4 passes per thread for d = 4096

template <typename T>
DG_DEV void store4(T* dst, float4 v) {
    if constexpr (sizeof(T) == 4) {
        *reinterpret_cast<float4*>(dst) = v;
    } else {
        ushort4 u;
        u.x = f32_to_bf16(v.x);
        u.y = f32_to_bf16(v.y);
        u.z = f32_to_bf16(v.z);
        u.w = f32_to_bf16(v.w);
        *reinterpret_cast<ushort4*>(dst) = u;
    }
}

// Normalised row `row` (xs scaled by r) to a (as T), a8 (e4m3 of the rounded a) and
// af (the bf16 row in fragment order, frag_offset with K = 4 d4).
template <typename T, int NT>
DG_DEV void store_norm(const float4 (&xs)[row_passes<NT>()], float r, int d4, T* __restrict__ a,
                       uint8_t* __restrict__ a8, uint8_t* __restrict__ af, int64_t row) {
#pragma unroll
    for (int p = 0; p < row_passes<NT>(); ++p) {
        const int c4 = threadIdx.x + NT * p;
        if (c4 >= d4) break;
        const float4 v = make_float4(xs[p].x * r, xs[p].y * r, xs[p].z * r, xs[p].w * r);
        store4<T>(a + 4 * (int64_t)c4, v);
        if (af) store4<T>(reinterpret_cast<T*>(af + frag_offset<false>(row, 4 * c4, 4 * d4)), v);
        if (a8) {
            uchar4 q;
            q.x = (uint8_t)f32_to_e4m3(to_f32<T>(from_f32<T>(v.x)));
            q.y = (uint8_t)f32_to_e4m3(to_f32<T>(from_f32<T>(v.y)));
            q.z = (uint8_t)f32_to_e4m3(to_f32<T>(from_f32<T>(v.z)));
            q.w = (uint8_t)f32_to_e4m3(to_f32<T>(from_f32<T>(v.w)));
            *reinterpret_cast<uchar4*>(a8 + 4 * (int64_t)c4) = q;
        }
    }
}

template <typename T, int NT>
__global__ __launch_bounds__(NT) void k_rmsnorm(const float* __restrict__ x, int d, float eps,
                                                T* __restrict__ a, uint8_t* __restrict__ a8,
                                                uint8_t* __restrict__ af) {
    __shared__ float red[NT / 64];
    const int64_t row = blockIdx.x;
    const int d4 = d >> 2;
    const float4* xr = reinterpret_cast<const float4*>(x + row * d);
    float4 xs[row_passes<NT>()];
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < row_passes<NT>(); ++p) {
        const int c4 = threadIdx.x + NT * p;
        xs[p] = c4 < d4 ? xr[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
        ss += xs[p].x * xs[p].x + xs[p].y * xs[p].y + xs[p].z * xs[p].z + xs[p].w * xs[p].w;
    }
    const float r = rsqrtf(block_sum<NT>(ss, red) / (float)d + eps);
    store_norm<T, NT>(xs, r, d4, a + row * d, a8 ? a8 + row * d : nullptr, af, row);
}

// ------------------------------------------------------------------ RoPE + scatter
// f32 path: qkv [M, (Hq + 2 Hkv) D] -> Q [Hq][M][D] rotated, K cache rows pos0+m
// rotated, V cache rows pos0+m.  Rotate-half pairs (j, j + D/2), angle table
// [pos][D/2]; the position of token m is pos0 + m, or pos0 + m % period for a
// batch of canvases at the same positions (period = C > 0).  One block per (32
// tokens, head).  (The bf16 path rotates in the QKV GEMM's epilogue.)
constexpr int kRopeTokens = 32;

template <int D>
__global__ __launch_bounds__(256) void k_rope_scatter(const float* __restrict__ qkv, int M, int Hq,
                                                      int Hkv, int64_t pos0, int period,
                                                      const float* __restrict__ cos_t,
                                                      const float* __restrict__ sin_t,
                                                      float* __restrict__ q, float* __restrict__ kc,
                                                      float* __restrict__ vc, int64_t kv_rows) {
    const int m0 = blockIdx.x * kRopeTokens;
    const int head = blockIdx.y;             // 0..Hq-1 queries, Hq..Hq+Hkv-1 keys, then values
    constexpr int half = D >> 1;
    const int64_t ld = (int64_t)(Hq + 2 * Hkv) * D;
    const int nt = min(kRopeTokens, M - m0);
    for (int e = threadIdx.x; e < nt * half; e += 256) {
        const int mi = e / half, j = e - mi * half;
        const int m = m0 + mi;
        const int64_t row = pos0 + m;                              // cache row
        const int64_t pos = pos0 + (period > 0 ? m % period : m);  // RoPE position
        const float* src = qkv + (int64_t)m * ld + (int64_t)head * D;
        const float x1 = src[j], x2 = src[j + half];
        if (head < Hq + Hkv) {
            const float c = cos_t[pos * half + j], sn = sin_t[pos * half + j];
            const float y1 = x1 * c - x2 * sn, y2 = x2 * c + x1 * sn;
            float* dst = head < Hq ? q + ((int64_t)head * M + m) * D
                                   : kc + ((int64_t)(head - Hq) * kv_rows + row) * D;
            dst[j] = y1;
            dst[j + half] = y2;
        } else {
            float* dst = vc + ((int64_t)(head - Hq - Hkv) * kv_rows + row) * D;
            dst[j] = x1;
            dst[j + half] = x2;
        }
    }
}

// Natural [Hkv][S][D] V -> transposed key-permuted layout (for the attention entry point).
// One workgroup per (32-key block, KV head): the block's key rows are read with 16-byte
// loads into LDS (rows padded by 16 bytes), then every dimension row of the block (32 keys,
// 64 bytes, in the slot order of vt_index) is written as four 16-byte stores.  Keys past S
// are zero.  D is a multiple of 8 and at most kPackVtMaxD.
constexpr int kPackVtMaxD = 128;

__global__ __launch_bounds__(256) void k_pack_vt(const bf16_t* __restrict__ v, int S, int D,
                                                 bf16_t* __restrict__ vt, int64_t rows) {
    __shared__ __attribute__((aligned(16))) bf16_t tile[32][kPackVtMaxD + 8];
    const int64_t p0 = (int64_t)blockIdx.x * 32;
    const int h = blockIdx.y;
    const int c8n = D >> 3;
    for (int e = threadIdx.x; e < 32 * c8n; e += blockDim.x) {
        const int r = e / c8n, c8 = e % c8n;
        const int64_t p = p0 + r;
        uint4 val = uint4{0u, 0u, 0u, 0u};
        if (p < S) val = *reinterpret_cast<const uint4*>(v + ((int64_t)h * S + p) * D + 8 * c8);
        *reinterpret_cast<uint4*>(&tile[r][8 * c8]) = val;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 4 * D; e += blockDim.x) {
        const int dim = e >> 2, q0 = 8 * (e & 3);
        uint16_t o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            // output slot q holds key 16 b + 4 a + c, where q = 8 a + 4 b + c (vt_index)
            const int q = q0 + j;
            const int r = 16 * ((q >> 2) & 1) + 4 * (q >> 3) + (q & 3);
            o[j] = tile[r][dim];
        }
        uint4 w;
        w.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
        w.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
        w.z = (uint32_t)o[4] | ((uint32_t)o[5] << 16);
        w.w = (uint32_t)o[6] | ((uint32_t)o[7] << 16);
        *reinterpret_cast<uint4*>(vt + ((int64_t)h * D + dim) * rows + p0 + q0) = w;
    }
}

// K/V read-back in natural [Hkv][n][D] layout (debug / tests).
template <typename T, bool VPACKED>
__global__ void k_read_kv(const T* __restrict__ cache, int Hkv, int D, int64_t rows,
                          int64_t row0, int64_t n, T* __restrict__ dst) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)Hkv * n * D) return;
    const int t = (int)(idx % D);
    const int64_t p = (idx / D) % n;
    const int h = (int)(idx / ((int64_t)D * n));
    dst[idx] = VPACKED ? cache[vt_index(h, t, row0 + p, D, rows)]
                       : cache[((int64_t)h * rows + row0 + p) * D + t];
}

template <typename T, bool VPACKED>
__global__ void k_write_kv(T* __restrict__ cache, int Hkv, int D, int64_t rows, int64_t row0,
                           int64_t n, const T* __restrict__ src) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)Hkv * n * D) return;
    const int t = (int)(idx % D);
    const int64_t p = (idx / D) % n;
    const int h = (int)(idx / ((int64_t)D * n));
    if (VPACKED) cache[vt_index(h, t, row0 + p, D, rows)] = src[idx];
    else cache[((int64_t)h * rows + row0 + p) * D + t] = src[idx];
}

// ------------------------------------------------------------------ combine (+ RMSNorm)
// y = sum_j gates[t, j] * Y[inv[t*k + j], :] in slot order.
// MODE 0: x += y, then a = rmsnorm(x) (and a8 = e4m3(a) if given) when a != null.
// MODE 1: out = y (stored as T), no residual (the stand-alone MoE layer).
// One block of NT threads per token, four columns per thread per pass (d % 4 == 0); all of
// the token's expert rows are loaded before they are summed.
template <typename T, int MODE, int KMAX, int NT>
__global__ __launch_bounds__(NT) void k_moe_combine(const void* __restrict__ Yv, int d, int k,
                                                     const float* __restrict__ gates,
                                                     const int32_t* __restrict__ inv,
                                                     float* __restrict__ x, float eps,
                                                     T* __restrict__ a, uint8_t* __restrict__ a8,
                                                     uint8_t* __restrict__ af,
                                                     T* __restrict__ out) {
    __shared__ float red[NT / 64];
    const int64_t t = blockIdx.x;
    const int d4 = d >> 2;
    // expert outputs: float rows for f32 experts, binary16 rows otherwise (bf16 activations)
    using YT = std::conditional_t<sizeof(T) == 4, float, _Float16>;
    using Y4 = std::conditional_t<sizeof(T) == 4, float4, f16x4_t>;
    const YT* Y = static_cast<const YT*>(Yv);
    float g[KMAX];
    const Y4* yr[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        g[j] = j < k ? gates[t * k + j] : 0.f;
        yr[j] = reinterpret_cast<const Y4*>(Y + (int64_t)(j < k ? inv[t * k + j] : inv[t * k]) * d);
    }
    float4* xr = reinterpret_cast<float4*>(x + t * d);
    float4 xs[row_passes<NT>()];
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < row_passes<NT>(); ++p) {
        const int c4 = threadIdx.x + NT * p;
        if (c4 >= d4) break;
        float4 v[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j < k) {
                const Y4 yv = yr[j][c4];
                v[j] = make_float4((float)yv[0], (float)yv[1], (float)yv[2], (float)yv[3]);
            } else {
                v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {   // slot order
            if (j >= k) break;
            y.x += g[j] * v[j].x;
            y.y += g[j] * v[j].y;
            y.z += g[j] * v[j].z;
            y.w += g[j] * v[j].w;
        }
        if (MODE == 0) {
            const float4 xo = xr[c4];
            const float4 nx = make_float4(xo.x + y.x, xo.y + y.y, xo.z + y.z, xo.w + y.w);
            xr[c4] = nx;
            xs[p] = nx;
            ss += nx.x * nx.x + nx.y * nx.y + nx.z * nx.z + nx.w * nx.w;
        } else {
            store4<T>(out + t * d + 4 * c4, y);
        }
    }
    if (MODE == 0 && a != nullptr) {
        const float r = rsqrtf(block_sum<NT>(ss, red) / (float)d + eps);
        store_norm<T, NT>(xs, r, d4, a + t * d, a8 ? a8 + t * d : nullptr, af, t);
    }
}

// ------------------------------------------------------------------ canvas init
__global__ void k_canvas_init(int32_t* __restrict__ canvas, uint8_t* __restrict__ mask, int C,
                              int V, uint64_t seed, int k_blk) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= C) return;
    u32x4 c = {(uint32_t)(i >> 2), (uint32_t)k_blk, 0u, kInitTag};
    u32x4 r = philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    uint32_t w = (i & 3) == 0 ? r.x : (i & 3) == 1 ? r.y : (i & 3) == 2 ? r.z : r.w;
    if (canvas) canvas[i] = (int32_t)(((uint64_t)w * (uint64_t)V) >> 32);
    if (mask) mask[i] = 0;
}

// ------------------------------------------------------------------ LM-head statistics
// Reduce the per-slice partials of one row in a fixed tree: max with the
// lowest id on ties, sum of exp(z - max), Gumbel best with the lowest id on ties,
// and with ENT the weighted sum q = sum exp(z - max) (z - max), rescaled to a
// new max m as f (q + (m_i - m) s) with f = exp(m_i - m).
struct HeadPart { float m; int32_t a; float s; float g; int32_t gi; float q; };

template <bool ENT>
DG_DEV void head_merge(HeadPart& x, const HeadPart& y) {
    if (y.m > x.m || (y.m == x.m && y.a < x.a)) {
        const float f = (x.m == -INFINITY) ? 0.f : exp2f((x.m - y.m) * 1.4426950408889634f);
        if constexpr (ENT) x.q = y.q + (f == 0.f ? 0.f : f * fmaf(x.m - y.m, x.s, x.q));
        x.s = y.s + x.s * f;
        x.m = y.m;
        x.a = y.a;
    } else {
        const float f = (y.m == -INFINITY) ? 0.f : exp2f((y.m - x.m) * 1.4426950408889634f);
        if constexpr (ENT) x.q += f == 0.f ? 0.f : f * fmaf(y.m - x.m, y.s, y.q);
        x.s += y.s * f;
    }
    if (y.g > x.g || (y.g == x.g && y.gi < x.gi)) { x.g = y.g; x.gi = y.gi; }
}

template <bool ENT>
__global__ __launch_bounds__(256) void k_head_stats(const float* __restrict__ pm,
                                                    const int32_t* __restrict__ pa,
                                                    const float* __restrict__ ps,
                                                    const float* __restrict__ pg,
                                                    const int32_t* __restrict__ pgi,
                                                    const float* __restrict__ pq,
                                                    int n_slices, const uint8_t* __restrict__ mask,
                                                    float* __restrict__ st_m,
                                                    int32_t* __restrict__ st_a,
                                                    float* __restrict__ st_lse,
                                                    float* __restrict__ st_conf,
                                                    int32_t* __restrict__ st_draw,
                                                    float* __restrict__ st_ent,
                                                    int32_t* __restrict__ bad) {
    __shared__ HeadPart sh[4];
    const int row = blockIdx.x;
    HeadPart acc = {-INFINITY, 0x7fffffff, 0.f, -INFINITY, 0x7fffffff, 0.f};
    for (int i = threadIdx.x; i < n_slices; i += 256) {
        const int64_t o = (int64_t)row * n_slices + i;
        HeadPart p = {pm[o], pa[o], ps[o], pg[o], pgi[o], ENT ? pq[o] : 0.f};
        head_merge<ENT>(acc, p);
    }
    // within each wave by shuffles, then the four waves in order
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const HeadPart y = {__shfl_xor(acc.m, o, 64), __shfl_xor(acc.a, o, 64), __shfl_xor(acc.s, o, 64),
                            __shfl_xor(acc.g, o, 64), __shfl_xor(acc.gi, o, 64),
                            ENT ? __shfl_xor(acc.q, o, 64) : 0.f};
        head_merge<ENT>(acc, y);
    }
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        HeadPart r = sh[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) head_merge<ENT>(r, sh[w]);
        const float ls = logf(r.s);
        if constexpr (ENT) {
            const float h = ls - r.q / r.s;                    // entropy of Softmax(z), nats
            st_ent[row] = h;
            if (!isfinite(h)) atomicOr(bad, kBadNonFinite);
        }
        st_m[row] = r.m;
        st_a[row] = r.a;
        st_lse[row] = r.m + ls;
        st_conf[row] = -ls;
        st_draw[row] = mask[row] ? -1 : r.gi;
        if (!isfinite(r.m) || !isfinite(ls) || (!mask[row] && r.gi < 0)) atomicOr(bad, kBadNonFinite);
    }
}

// Posterior rows of the self-conditioning signal, in place, once every row's lse is known:
// bf16 rows hold exp(z - m_slice) (128-id slices, m_slice the partial max pm) and become
// p0 = that * exp(m_slice - lse); float rows hold the tempered logits z and become
// exp(z - lse).  One thread per 8 ids (16 bytes of bf16, two float4 of float).
template <bool BF16>
__global__ __launch_bounds__(256) void k_posterior_rows(void* __restrict__ post,
                                                        const float* __restrict__ pm, int n_slices,
                                                        const float* __restrict__ lse, int M,
                                                        int V) {
    const int v8 = V >> 3;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * v8) return;
    const int row = (int)(i / v8), c = (int)(i % v8);
    const float l = lse[row];
    if constexpr (BF16) {
        const float f = __builtin_amdgcn_exp2f((pm[(size_t)row * n_slices + (c >> 4)] - l) *
                                               1.4426950408889634f);
        uint4* p = reinterpret_cast<uint4*>(post) + i;
        uint4 v = *p;
        uint32_t* w = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float lo = bf16_to_f32((bf16_t)(w[k] & 0xffffu)) * f;
            const float hi = bf16_to_f32((bf16_t)(w[k] >> 16)) * f;
            w[k] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
        }
        *p = v;
    } else {
        float4* p = reinterpret_cast<float4*>((float*)post + (size_t)row * V) + 2 * c;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            float4 v = p[k];
            v.x = expf(v.x - l);
            v.y = expf(v.y - l);
            v.z = expf(v.z - l);
            v.w = expf(v.w - l);
            p[k] = v;
        }
    }
}

// ------------------------------------------------------------------ sampler
// Partial rank of position i among the flagged positions (keys ascending if ASC,
// else descending; ties to the lower position) over the groups of four j4 = part,
// part + 4, ...: four lanes share a position and their parts are summed by the
// caller (rank_sum4).  Tail entries past C must be unflagged.
template <bool ASC>
DG_DEV int rank_part(const float* keys, const uint8_t* flag, int C4, int i, float ki, int part) {
    int rank = 0;
#pragma unroll 4
    for (int j4 = part; j4 < C4; j4 += 4) {
        const float4 c = reinterpret_cast<const float4*>(keys)[j4];
        const uchar4 u = reinterpret_cast<const uchar4*>(flag)[j4];
        const int j = 4 * j4;
        if constexpr (ASC) {
            rank += u.x && (c.x < ki || (c.x == ki && j < i));
            rank += u.y && (c.y < ki || (c.y == ki && j + 1 < i));
            rank += u.z && (c.z < ki || (c.z == ki && j + 2 < i));
            rank += u.w && (c.w < ki || (c.w == ki && j + 3 < i));
        } else {
            rank += u.x && (c.x > ki || (c.x == ki && j < i));
            rank += u.y && (c.y > ki || (c.y == ki && j + 1 < i));
            rank += u.z && (c.z > ki || (c.z == ki && j + 2 < i));
            rank += u.w && (c.w > ki || (c.w == ki && j + 3 < i));
        }
    }
    return rank;
}

// Sum over the four adjacent lanes of a position (all four take part together).
DG_DEV int rank_sum4(int r) {
    r += __shfl_xor(r, 1, 64);
    return r + __shfl_xor(r, 2, 64);
}

// One workgroup.  Among unlocked positions, the n_s with the highest
// confidence (ties to the lower position) are locked to their argmax; the
// other unlocked positions take their Gumbel draw.  Locked ones are untouched.
__global__ __launch_bounds__(1024) void k_sampler(const float* __restrict__ conf,
                                                  const int32_t* __restrict__ amax,
                                                  const int32_t* __restrict__ draw,
                                                  int32_t* __restrict__ canvas,
                                                  uint8_t* __restrict__ mask, int C, int step,
                                                  int T) {
    // workgroup b samples canvas b of a batch (positions b C .. b C + C - 1)
    {
        const int64_t o = (int64_t)blockIdx.x * C;
        conf += o;
        amax += o;
        draw += o;
        canvas += o;
        mask += o;
    }
    __shared__ __attribute__((aligned(16))) float cf[kMaxCanvas];
    __shared__ __attribute__((aligned(16))) uint8_t un[kMaxCanvas];
    __shared__ int n_unl;
    if (threadIdx.x == 0) n_unl = 0;
    __syncthreads();
    int mine = 0;
    for (int i = threadIdx.x; i < (C + 3) / 4 * 4; i += blockDim.x) {   // tail padded locked
        const bool u = i < C && mask[i] == 0;
        cf[i] = i < C ? conf[i] : 0.f;
        un[i] = u;
        mine += u;
    }
    atomicAdd(&n_unl, mine);
    __syncthreads();
    const int nu = n_unl;
    const int quota = (C + T - 1) / T;
    const int n_s = (step == T - 1) ? nu : (quota < nu ? quota : nu);
    const int C4 = (C + 3) / 4, part = threadIdx.x & 3;
    for (int i = threadIdx.x >> 2; i < C; i += blockDim.x >> 2) {   // four lanes per position
        const bool u = un[i] != 0;
        const int rank = rank_sum4(u ? rank_part<false>(cf, un, C4, i, cf[i], part) : 0);
        if (!u || part != 0) continue;
        if (rank < n_s) {
            canvas[i] = amax[i];
            mask[i] = 1;
        } else {
            canvas[i] = draw[i];
        }
    }
}

// ------------------------------------------------------------------ entropy-bounded sampler
// One pass of the sampler of the technical-report summary (Method, the sampler
// and adaptive-stopping paragraphs), one workgroup:
//  * stop test (pass >= 1): the canvas-mean entropy, summed in float64 in
//    position order, is below theta and every position's argmax equals the
//    previous pass's; the last pass always ends the block.  Ending, every
//    unlocked position takes its argmax and locks;
//  * otherwise unlocked positions are ranked by entropy (ties to the lower
//    position) and accepted in rank order while B = (running float64 sum of
//    their entropies) - (the entropy just added, the prefix's largest) stays
//    below gamma.  Accepted positions take their Gumbel draw and lock; the
//    rest take a uniform token (Philox stream kRenoiseTag); locked ones are
//    untouched.
// prev holds the previous pass's argmax and is overwritten with this pass's.
// info: [0] 1 if the block is finished, [1] positions locked by this pass,
// [2] positions left unlocked, [3] 1 if the stop test held.  NaN entropies
// rank last (the head statistics flag them).
__global__ __launch_bounds__(1024) void k_sampler_eb(const float* __restrict__ ent,
                                                     const int32_t* __restrict__ amax,
                                                     const int32_t* __restrict__ draw,
                                                     int32_t* __restrict__ prev,
                                                     int32_t* __restrict__ canvas,
                                                     uint8_t* __restrict__ mask,
                                                     int32_t* __restrict__ info, int C, int V,
                                                     int step, int max_steps, float gamma,
                                                     float theta, uint32_t key0, uint32_t key1,
                                                     int k_blk) {
    __shared__ __attribute__((aligned(16))) float hs[kMaxCanvas];
    __shared__ __attribute__((aligned(16))) uint8_t un[kMaxCanvas];
    __shared__ __attribute__((aligned(16))) float h_sorted[kMaxCanvas];
    __shared__ int16_t rank_of[kMaxCanvas];
    __shared__ int n_unl, n_diff, n_acc, stop;
    const int tid = threadIdx.x;
    if (tid == 0) {
        n_unl = 0;
        n_diff = 0;
    }
    __syncthreads();
    int mine = 0, diff = 0;
    for (int i = tid; i < (C + 3) / 4 * 4; i += blockDim.x) {   // tail padded locked
        const bool u = i < C && mask[i] == 0;
        float h = i < C ? ent[i] : 0.f;
        if (h != h) h = INFINITY;
        hs[i] = h;
        un[i] = u;
        mine += u;
        if (i < C && step > 0) diff += prev[i] != amax[i];
    }
    if (mine) atomicAdd(&n_unl, mine);
    if (diff) atomicAdd(&n_diff, diff);
    __syncthreads();
    const int C4 = (C + 3) / 4, part = tid & 3;
    for (int i = tid >> 2; i < C; i += blockDim.x >> 2) {   // four lanes per position
        const bool u = un[i] != 0;
        const float hi = hs[i];
        const int rank = rank_sum4(u ? rank_part<true>(hs, un, C4, i, hi, part) : 0);
        if (u && part == 0) {
            rank_of[i] = (int16_t)rank;
            h_sorted[rank] = hi;
        }
    }
    __syncthreads();
    const float4* hs4 = reinterpret_cast<const float4*>(hs);
    const float4* hq4 = reinterpret_cast<const float4*>(h_sorted);
    if (tid == 0) {
        // position order; the padded tail adds zeros
        double acc = 0.0;
#pragma unroll 8
        for (int g = 0; g < C4; ++g) {
            const float4 v = hs4[g];
            acc += (double)v.x;
            acc += (double)v.y;
            acc += (double)v.z;
            acc += (double)v.w;
        }
        const bool rule = step >= 1 && n_diff == 0 && acc / (double)C < (double)theta;
        stop = rule ? 2 : (step == max_steps - 1 ? 1 : 0);
    } else if (tid == 64) {
        // rank order, four sorted entropies per LDS read with the next four in flight
        const int nu = n_unl;
        int n = nu > 0 ? 1 : 0;
        double run = 0.0;
        float4 v = hq4[0];
        for (int g = 0; 4 * g < nu; ++g) {
            const float4 nxt = hq4[(g + 1) < kMaxCanvas / 4 ? g + 1 : g];
            const float w4[4] = {v.x, v.y, v.z, v.w};
            bool go = true;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = 4 * g + q;
                if (k >= nu) break;
                const double hk = (double)w4[q];
                run += hk;
                if (k == 0) continue;
                if (run - hk < (double)gamma) {
                    n = k + 1;
                } else {
                    go = false;
                    break;
                }
            }
            if (!go) break;
            v = nxt;
        }
        n_acc = n;
    }
    __syncthreads();
    const bool fin = stop != 0;
    const int na = n_acc, nu = n_unl;
    for (int i = tid; i < C; i += blockDim.x) {
        const int32_t a = amax[i];
        prev[i] = a;
        if (!un[i]) continue;
        if (fin) {
            canvas[i] = a;
            mask[i] = 1;
        } else if (rank_of[i] < na) {
            canvas[i] = draw[i];
            mask[i] = 1;
        } else {
            const u32x4 r = philox4x32_10(u32x4{(uint32_t)(i >> 2), (uint32_t)k_blk, (uint32_t)step,
                                                kRenoiseTag}, key0, key1);
            const uint32_t w = (i & 3) == 0 ? r.x : (i & 3) == 1 ? r.y : (i & 3) == 2 ? r.z : r.w;
            canvas[i] = (int32_t)(((uint64_t)w * (uint64_t)V) >> 32);
        }
    }
    if (tid == 0) {
        const int locked_now = fin ? nu : na;
        info[0] = fin || nu - locked_now == 0;
        info[1] = locked_now;
        info[2] = nu - locked_now;
        info[3] = stop == 2;
    }
}

// ------------------------------------------------------------------ weight packing
// src [K][N] (SRC_KN) or [N][K] (!SRC_KN), 16-bit elements -> packed B operand.
// The destination column group of source group g is g * gstride + goff (the
// gate / up interleave of the first expert GEMM uses gstride 2).
// Pair-tiled group order of a 128-column head: group gi (dims 16 gi ..) goes to
// group 4 ((gi % 4) / 2) + 2 (gi / 4) + gi % 2, so tile t (groups 4t..4t+3) holds
// dims 32t..32t+31 and their rotary partners 64 + 32t..64 + 32t + 31.
DG_DEV int64_t rope_pair_group(int64_t g) {
    const int64_t gi = g & 7;
    return (g & ~(int64_t)7) + 4 * ((gi & 3) >> 1) + 2 * (gi >> 2) + (gi & 1);
}

template <bool SRC_KN>
__global__ void k_pack_b16(const uint16_t* __restrict__ src, int K, int N, int gstride, int goff,
                           uint16_t* __restrict__ dst, int rope_hd) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)K * N) return;
    int64_t n, kk;
    if (SRC_KN) { kk = idx / N; n = idx % N; } else { n = idx / K; kk = idx % K; }
    const int64_t g = rope_hd == 128 ? rope_pair_group(n >> 4) : (n >> 4);
    const int64_t dn = (g * gstride + goff) * 16 + (n & 15);
    dst[packed_b_index(dn, kk, K)] = src[idx];
}

// e4m3 codes [K][N] -> packed [N/16][K/64][64 lanes][16 bytes]; byte b < 8 holds
// k = 64*kb + 8*(lane/16) + b, byte b >= 8 holds k = 64*kb + 32 + 8*(lane/16) + b - 8.
__global__ void k_pack_b8(const uint8_t* __restrict__ src, int K, int N, int gstride, int goff,
                          uint8_t* __restrict__ dst) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)K * N) return;
    const int64_t kk = idx / N, n = idx % N;
    const int64_t dn = ((n >> 4) * gstride + goff) * 16 + (n & 15);
    const int64_t kb = kk >> 6, r = kk & 63;
    const int half = (int)(r >> 5), g = (int)((r & 31) >> 3), b = (int)(r & 7);
    const int lane = (int)(dn & 15) + 16 * g;
    dst[((((dn >> 4) * (K >> 6) + kb) * 64 + lane) << 4) + half * 8 + b] = src[idx];
}

// Column scales of the interleaved gate/up weights follow the same group map.
__global__ void k_scatter_scales(const float* __restrict__ src, int N, int gstride, int goff,
                                 float* __restrict__ dst) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    dst[((n >> 4) * gstride + goff) * 16 + (n & 15)] = src[n];
}

__global__ void k_cast_e4m3(const bf16_t* __restrict__ x, int64_t n, uint8_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = (uint8_t)f32_to_e4m3(bf16_to_f32(x[i]));
}

__global__ void k_fill_u32(uint32_t* p, uint32_t v, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// ================================================================== launchers
#define LAUNCH_CHECK() return hipGetLastError()

hipError_t launch_embed_rmsnorm(int dtype, bool packed, const int32_t* tokens, const void* E,
                                int V, int C, int d, float eps, float* x, void* a, void* af,
                                int32_t* bad, hipStream_t s, const float* zadd) {
    if (C == 0) return hipSuccess;
    if (dtype == kF32)
        k_embed_rmsnorm<float, false><<<C, 256, 0, s>>>(tokens, (const float*)E, V, d, eps, x,
                                                        (float*)a, nullptr, bad, zadd);
    else if (packed)
        k_embed_rmsnorm<bf16_t, true><<<C, 256, 0, s>>>(tokens, (const bf16_t*)E, V, d, eps, x,
                                                        (bf16_t*)a, (uint8_t*)af, bad, zadd);
    else
        k_embed_rmsnorm<bf16_t, false><<<C, 256, 0, s>>>(tokens, (const bf16_t*)E, V, d, eps, x,
                                                         (bf16_t*)a, (uint8_t*)af, bad, zadd);
    LAUNCH_CHECK();
}

// ------------------------------------------------------------------ self-conditioning FFW
// H[r, f] = silu(h1[r, f]) * h1[r, F + f]: the gated hidden layer of the feed-forward
// block of the self-conditioning signal (gate columns first, then up).  bf16: H in
// MFMA fragment order (K = F) for the down projection; f32: natural rows.  One thread
// per four columns (F % 4 == 0).
template <bool FRAG>
__global__ __launch_bounds__(256) void k_swiglu_rows(const float* __restrict__ h1, int M, int F,
                                                     void* __restrict__ H) {
    const int f4 = F >> 2;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * f4) return;
    const int r = (int)(i / f4), c = (int)(i % f4) * 4;
    const float4 g = *reinterpret_cast<const float4*>(h1 + (size_t)r * 2 * F + c);
    const float4 u = *reinterpret_cast<const float4*>(h1 + (size_t)r * 2 * F + F + c);
    float4 h;
    h.x = g.x / (1.0f + expf(-g.x)) * u.x;
    h.y = g.y / (1.0f + expf(-g.y)) * u.y;
    h.z = g.z / (1.0f + expf(-g.z)) * u.z;
    h.w = g.w / (1.0f + expf(-g.w)) * u.w;
    if constexpr (FRAG) {
        ushort4 b;
        b.x = f32_to_bf16(h.x);
        b.y = f32_to_bf16(h.y);
        b.z = f32_to_bf16(h.z);
        b.w = f32_to_bf16(h.w);
        *reinterpret_cast<ushort4*>((uint8_t*)H + frag_offset<false>(r, c, F)) = b;
    } else {
        *reinterpret_cast<float4*>((float*)H + (size_t)r * F + c) = h;
    }
}

hipError_t launch_swiglu_rows(int dtype, const float* h1, int M, int F, void* H, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if (F & (dtype == kF32 ? 3 : 31)) return hipErrorInvalidValue;
    const int64_t n = (int64_t)M * (F / 4);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (dtype == kF32) k_swiglu_rows<false><<<blocks, 256, 0, s>>>(h1, M, F, H);
    else k_swiglu_rows<true><<<blocks, 256, 0, s>>>(h1, M, F, H);
    LAUNCH_CHECK();
}

hipError_t launch_rmsnorm(int dtype, const float* x, int M, int d, float eps, void* a,
                          uint8_t* a8, void* af, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if ((d & 3) || d > 4096) return hipErrorInvalidValue;
    if (dtype == kF32)
        k_rmsnorm<float, kRowThreads><<<M, kRowThreads, 0, s>>>(x, d, eps, (float*)a, a8, nullptr);
    else
        k_rmsnorm<bf16_t, kRowThreads><<<M, kRowThreads, 0, s>>>(x, d, eps, (bf16_t*)a, a8, (uint8_t*)af);
    LAUNCH_CHECK();
}

template <int D>
static void rope_d(const float* qkv, int M, int Hq, int Hkv, int64_t pos0, int period,
                   const float* cos_t, const float* sin_t, void* q, void* kc, void* vc,
                   int64_t kv_rows, hipStream_t s) {
    dim3 grid((M + kRopeTokens - 1) / kRopeTokens, Hq + 2 * Hkv);
    k_rope_scatter<D><<<grid, 256, 0, s>>>(qkv, M, Hq, Hkv, pos0, period, cos_t, sin_t, (float*)q,
                                           (float*)kc, (float*)vc, kv_rows);
}

hipError_t launch_rope_scatter(int dtype, const float* qkv, int M, int Hq, int Hkv, int D,
                               int64_t pos0, int period, const float* cos_t, const float* sin_t,
                               void* q, void* kc, void* vc, int64_t kv_rows, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if (period < 0) return hipErrorInvalidValue;
    if (dtype == kF32) {
        if (D == 64) rope_d<64>(qkv, M, Hq, Hkv, pos0, period, cos_t, sin_t, q, kc, vc, kv_rows, s);
        else if (D == 128) rope_d<128>(qkv, M, Hq, Hkv, pos0, period, cos_t, sin_t, q, kc, vc, kv_rows, s);
        else return hipErrorInvalidValue;
    } else {
        return hipErrorInvalidValue;   // bf16: RoPE runs in the QKV GEMM's epilogue (kEpiRope)
    }
    LAUNCH_CHECK();
}

hipError_t launch_pack_vt(const void* v, int Hkv, int S, int D, void* vt, int64_t rows,
                          hipStream_t s) {
    if (Hkv <= 0 || rows <= 0) return hipSuccess;
    if ((D & 7) || D > kPackVtMaxD || (rows & 31) || rows < S) return hipErrorInvalidValue;
    k_pack_vt<<<dim3((unsigned)(rows / 32), Hkv), 256, 0, s>>>((const bf16_t*)v, S, D, (bf16_t*)vt, rows);
    LAUNCH_CHECK();
}

hipError_t launch_read_kv(int dtype, bool vpacked, const void* cache, int Hkv, int D,
                          int64_t rows, int64_t row0, int64_t n, void* dst, hipStream_t s) {
    int64_t total = (int64_t)Hkv * n * D;
    if (total <= 0) return hipSuccess;
    unsigned blocks = (unsigned)((total + 255) / 256);
    if (dtype == kF32)
        k_read_kv<float, false><<<blocks, 256, 0, s>>>((const float*)cache, Hkv, D, rows, row0,
                                                       n, (float*)dst);
    else if (vpacked)
        k_read_kv<bf16_t, true><<<blocks, 256, 0, s>>>((const bf16_t*)cache, Hkv, D, rows, row0,
                                                       n, (bf16_t*)dst);
    else
        k_read_kv<bf16_t, false><<<blocks, 256, 0, s>>>((const bf16_t*)cache, Hkv, D, rows,
                                                        row0, n, (bf16_t*)dst);
    LAUNCH_CHECK();
}

hipError_t launch_write_kv(int dtype, bool vpacked, void* cache, int Hkv, int D, int64_t rows,
                           int64_t row0, int64_t n, const void* src, hipStream_t s) {
    int64_t total = (int64_t)Hkv * n * D;
    if (total <= 0) return hipSuccess;
    unsigned blocks = (unsigned)((total + 255) / 256);
    if (dtype == kF32)
        k_write_kv<float, false><<<blocks, 256, 0, s>>>((float*)cache, Hkv, D, rows, row0, n,
                                                        (const float*)src);
    else if (vpacked)
        k_write_kv<bf16_t, true><<<blocks, 256, 0, s>>>((bf16_t*)cache, Hkv, D, rows, row0, n,
                                                        (const bf16_t*)src);
    else
        k_write_kv<bf16_t, false><<<blocks, 256, 0, s>>>((bf16_t*)cache, Hkv, D, rows, row0, n,
                                                         (const bf16_t*)src);
    LAUNCH_CHECK();
}

template <typename T, int MODE, int KMAX>
static void combine_k(const void* Y, int M, int d, int k, const float* gates, const int32_t* inv,
                      float* x, float eps, void* a, uint8_t* a8, void* af, void* out,
                      hipStream_t s) {
    k_moe_combine<T, MODE, KMAX, kRowThreads><<<M, kRowThreads, 0, s>>>(Y, d, k, gates, inv, x, eps,
                                                                        (T*)a, a8, (uint8_t*)af,
                                                                        (T*)out);
}

template <typename T, int MODE>
static void combine_m(const void* Y, int M, int d, int k, const float* gates, const int32_t* inv,
                      float* x, float eps, void* a, uint8_t* a8, void* af, void* out,
                      hipStream_t s) {
    if (k <= 2) combine_k<T, MODE, 2>(Y, M, d, k, gates, inv, x, eps, a, a8, af, out, s);
    else if (k <= 4) combine_k<T, MODE, 4>(Y, M, d, k, gates, inv, x, eps, a, a8, af, out, s);
    else if (k <= 8) combine_k<T, MODE, 8>(Y, M, d, k, gates, inv, x, eps, a, a8, af, out, s);
    else combine_k<T, MODE, kMaxTopK>(Y, M, d, k, gates, inv, x, eps, a, a8, af, out, s);
}

hipError_t launch_moe_combine(int dtype, int mode, const void* Y, int M, int d, int k,
                              const float* gates, const int32_t* inv, float* x, float eps,
                              void* a, uint8_t* a8, void* af, void* out, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if ((d & 3) || d > 4096 || k < 1 || k > kMaxTopK) return hipErrorInvalidValue;
    if (dtype == kF32) {
        if (mode == 0) combine_m<float, 0>(Y, M, d, k, gates, inv, x, eps, a, a8, nullptr, nullptr, s);
        else combine_m<float, 1>(Y, M, d, k, gates, inv, x, eps, nullptr, nullptr, nullptr, out, s);
    } else {
        if (mode == 0) combine_m<bf16_t, 0>(Y, M, d, k, gates, inv, x, eps, a, a8, af, nullptr, s);
        else combine_m<bf16_t, 1>(Y, M, d, k, gates, inv, x, eps, nullptr, nullptr, nullptr, out, s);
    }
    LAUNCH_CHECK();
}

hipError_t launch_canvas_init(int32_t* canvas, uint8_t* mask, int C, int V, uint64_t seed,
                              int k_blk, hipStream_t s) {
    k_canvas_init<<<(C + 255) / 256, 256, 0, s>>>(canvas, mask, C, V, seed, k_blk);
    LAUNCH_CHECK();
}

hipError_t launch_head_stats(const HeadPartials& p, int C, const uint8_t* mask, float* st_m,
                             int32_t* st_a, float* st_lse, float* st_conf, int32_t* st_draw,
                             float* st_ent, int32_t* bad, hipStream_t s,
                             const PosteriorRows& post) {
    if (C <= 0) return hipSuccess;
    if ((p.q == nullptr) != (st_ent == nullptr)) return hipErrorInvalidValue;
    if (post.rows != nullptr) {
        if (post.dtype == kBF16 ? (post.V % kHeadSlice || p.n_slices != post.V / kHeadSlice)
                                : (post.dtype != kF32 || post.V % 8))
            return hipErrorInvalidValue;
    }
    auto k = p.q ? k_head_stats<true> : k_head_stats<false>;
    k<<<C, 256, 0, s>>>(p.m, p.a, p.s, p.g, p.gi, p.q, p.n_slices, mask, st_m, st_a, st_lse,
                        st_conf, st_draw, st_ent, bad);
    if (post.rows == nullptr) LAUNCH_CHECK();
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)C * (post.V / 8);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (post.dtype == kBF16)
        k_posterior_rows<true><<<blocks, 256, 0, s>>>(post.rows, p.m, p.n_slices, st_lse, C, post.V);
    else
        k_posterior_rows<false><<<blocks, 256, 0, s>>>(post.rows, p.m, p.n_slices, st_lse, C, post.V);
    LAUNCH_CHECK();
}

hipError_t launch_sampler(const float* conf, const int32_t* amax, const int32_t* draw,
                          int32_t* canvas, uint8_t* mask, int C, int B, int step, int T,
                          hipStream_t s) {
    if (C <= 0 || C > kMaxCanvas || B <= 0) return hipErrorInvalidValue;
    k_sampler<<<B, 1024, 0, s>>>(conf, amax, draw, canvas, mask, C, step, T);
    LAUNCH_CHECK();
}

hipError_t launch_sampler_eb(const float* ent, const int32_t* amax, const int32_t* draw,
                             int32_t* prev, int32_t* canvas, uint8_t* mask, int32_t* info, int C,
                             int V, int step, int max_steps, float gamma, float theta,
                             uint64_t seed, int k_blk, hipStream_t s) {
    if (C <= 0 || C > kMaxCanvas || V <= 0 || step < 0 || step >= max_steps)
        return hipErrorInvalidValue;
    k_sampler_eb<<<1, 1024, 0, s>>>(ent, amax, draw, prev, canvas, mask, info, C, V, step,
                                    max_steps, gamma, theta, (uint32_t)seed,
                                    (uint32_t)(seed >> 32), k_blk);
    LAUNCH_CHECK();
}

hipError_t launch_pack_b16(const void* src, bool src_kn, int K, int N, int gstride, int goff,
                           void* dst, hipStream_t s, int rope_hd) {
    if (rope_hd != 0 && (rope_hd != 128 || N % 128 != 0 || gstride != 1 || goff % 8 != 0))
        return hipErrorInvalidValue;
    int64_t total = (int64_t)K * N;
    unsigned blocks = (unsigned)((total + 255) / 256);
    if (src_kn)
        k_pack_b16<true><<<blocks, 256, 0, s>>>((const uint16_t*)src, K, N, gstride, goff,
                                                (uint16_t*)dst, rope_hd);
    else
        k_pack_b16<false><<<blocks, 256, 0, s>>>((const uint16_t*)src, K, N, gstride, goff,
                                                 (uint16_t*)dst, rope_hd);
    LAUNCH_CHECK();
}

// MX FP4 weights into the fragment and stage orders of mx_code_bytes / mx_scale_bytes.
// Codes: one thread per destination byte (source group gs, k-step, lane, byte t): rows
// 128 ks + 32 (l / 16) + 2 t and + 1 of column 16 gs + l % 16, zero past K.  Scales: one
// thread per (source group, k-step, lane).
__global__ void k_pack_mx_codes(const uint8_t* __restrict__ src, int K, int N, int KS, int gstride,
                                int goff, uint8_t* __restrict__ dst) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)(N / 16) * KS * 1024;
    if (idx >= total) return;
    const int t = (int)(idx & 15), lane = (int)((idx >> 4) & 63);
    const int64_t rest = idx >> 10;
    const int ks = (int)(rest % KS), gs = (int)(rest / KS);
    const int n = 16 * gs + (lane & 15);
    const int k0 = 128 * ks + 32 * (lane >> 4) + 2 * t;
    auto nib = [&](int k) -> uint32_t {
        if (k >= K) return 0u;
        return (src[(size_t)k * (N / 2) + n / 2] >> (4 * (n & 1))) & 0xFu;
    };
    const int64_t G = (int64_t)gs * gstride + goff;
    dst[((G * KS + ks) * 64 + lane) * 16 + t] = (uint8_t)(nib(k0) | (nib(k0 + 1) << 4));
}

__global__ void k_pack_mx_scales(const uint8_t* __restrict__ src, int K, int N, int KS, int gstride,
                                 int goff, uint8_t* __restrict__ dst) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)(N / 16) * KS * 64;
    if (idx >= total) return;
    const int lane = (int)(idx & 63);
    const int64_t rest = idx >> 6;
    const int ks = (int)(rest % KS), gs = (int)(rest / KS);
    const int n = 16 * gs + (lane & 15);
    const int kb = 4 * ks + (lane >> 4);
    const int64_t G = (int64_t)gs * gstride + goff;
    const int64_t slab = G >> 3, i = G & 7;
    const int NSt = (KS + 1) / 2;
    dst[((slab * NSt + ks / 2) * 64 + lane) * 16 + 8 * (ks & 1) + i] =
        kb < K / 32 ? src[(size_t)kb * N + n] : (uint8_t)127;
}

hipError_t launch_pack_mx(const uint8_t* codes, const uint8_t* scales, int K, int N, int gstride,
                          int goff, int n_dst_groups, void* dst_codes, uint8_t* dst_scales,
                          hipStream_t s) {
    if (K <= 0 || K % 32 || N % 16 || gstride < 1 || goff < 0 || goff >= gstride ||
        (int64_t)(N / 16 - 1) * gstride + goff >= n_dst_groups)
        return hipErrorInvalidValue;
    const int KS = (K + 127) / 128;
    const int64_t nc = (int64_t)(N / 16) * KS * 1024, ns = (int64_t)(N / 16) * KS * 64;
    k_pack_mx_codes<<<(unsigned)((nc + 255) / 256), 256, 0, s>>>(codes, K, N, KS, gstride, goff,
                                                                 (uint8_t*)dst_codes);
    k_pack_mx_scales<<<(unsigned)((ns + 255) / 256), 256, 0, s>>>(scales, K, N, KS, gstride, goff,
                                                                  dst_scales);
    LAUNCH_CHECK();
}

hipError_t launch_pack_b8(const void* src, int K, int N, int gstride, int goff, void* dst,
                          hipStream_t s) {
    int64_t total = (int64_t)K * N;
    k_pack_b8<<<(unsigned)((total + 255) / 256), 256, 0, s>>>((const uint8_t*)src, K, N,
                                                              gstride, goff, (uint8_t*)dst);
    LAUNCH_CHECK();
}

hipError_t launch_scatter_scales(const float* src, int N, int gstride, int goff, float* dst,
                                 hipStream_t s) {
    k_scatter_scales<<<(N + 255) / 256, 256, 0, s>>>(src, N, gstride, goff, dst);
    LAUNCH_CHECK();
}

hipError_t launch_fill_u32(void* p, uint32_t v, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    k_fill_u32<<<(unsigned)((n + 255) / 256), 256, 0, s>>>((uint32_t*)p, v, n);
    LAUNCH_CHECK();
}

hipError_t launch_cast_e4m3(const void* x, int64_t n, uint8_t* out, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    k_cast_e4m3<<<(unsigned)((n + 255) / 256), 256, 0, s>>>((const bf16_t*)x, n, out);
    LAUNCH_CHECK();
}

}  // namespace dg
