// C ABI of the canvas-denoising library: handle, weight re-layout, KV cache,
// and the orchestration of prefill / denoise pass / block / commit.
//
// Stages follow the generation pipeline of the DiffusionGemma technical-report
// summary (Method): the causal encoder fills the KV cache from the prompt
// (prefill), the decoder refines the canvas with bidirectional attention over
// [KV cache || canvas] (denoise pass), and the finished canvas is encoded
// causally and appended to the cache (commit).  Positions follow the P + K*C
// layout (same page, Dataset, "Example and sequence structure").
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dg.h"
#include "kernels.h"

using namespace dg;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

#define HIP_TRY(expr)                                                                       \
    do {                                                                                    \
        hipError_t e_ = (expr);                                                             \
        if (e_ != hipSuccess)                                                               \
            return fail(DG_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));           \
    } while (0)

#define DG_TRY(expr)                                                                        \
    do {                                                                                    \
        int r_ = (expr);                                                                    \
        if (r_ != DG_OK) return r_;                                                         \
    } while (0)

constexpr int kPrefillChunk = 4096;   // tokens per causal-encoder chunk
constexpr int kRouterSplit = 8;       // K split of the router GEMM

size_t dsize(int dt) { return dt == kF32 ? 4 : dt == kBF16 ? 2 : 1; }

}  // namespace

struct dg_handle {
    dg_model_cfg cfg;
    int L, d, Hq, Hkv, D, E, k, F, V, C;
    int B_max = 1;          // canvases one batched pass can hold
    int rows_max = 0;       // C * B_max: rows of the per-pass buffers
    int last_rows = 0;      // rows of the last pass (what the captures hold)
    int act, edt;
    int64_t max_ctx, kv_rows;
    int max_tokens;
    int qkv_n;

    std::vector<void*> allocs;

    void* embed = nullptr;
    std::vector<void*> wqkv, wo, wr, w1, wu, w2;
    std::vector<float*> s1, s2;
    std::vector<uint8_t*> x1, x2;  // MX FP4 experts: E8M0 block scales in stage order
    std::vector<uint8_t> loaded;   // per (layer, kind) dense flags and per expert flags
    bool ready = false;

    void* kcache = nullptr;   // [L][Hkv][kv_rows][D]
    void* vcache = nullptr;   // f32: same as K; bf16: [L][Hkv][D][kv_rows] transposed-permuted
    float* cos_t = nullptr;
    float* sin_t = nullptr;

    float* x = nullptr;
    void* a = nullptr;
    uint8_t* a8 = nullptr;
    float* qkv = nullptr;
    void* q = nullptr;
    void* attn_o = nullptr;
    void* part = nullptr;     // attention split partials
    size_t part_bytes = 0;
    float* rlog = nullptr;
    int32_t* idx = nullptr;
    float* gates = nullptr;
    int32_t* counts = nullptr;
    int32_t* base = nullptr;
    int32_t* offsets = nullptr;
    int32_t* perm_token = nullptr;
    int32_t* inv = nullptr;
    void* Xf = nullptr;      // fp8 expert GEMM 1 activations in fragment order
    void* Af = nullptr;      // dense-projection activations in fragment order (bf16)
    void* H = nullptr;
    float* Y = nullptr;      // expert outputs: float rows (f32 experts) or binary16 rows
    int4* work_items = nullptr;      // the first GEMM's items, then the second's
    int work_cap1 = 0;               // capacity of the first list
    int32_t* work_count = nullptr;

    HeadPartials hp{};
    float* st_m = nullptr;
    int32_t* st_a = nullptr;
    float* st_lse = nullptr;
    float* st_conf = nullptr;
    int32_t* st_draw = nullptr;
    float* st_ent = nullptr;      // predictive entropy per position (entropy-bounded passes)
    float* hp_q = nullptr;        // entropy partials [C][n_slices]
    int32_t* eb_prev = nullptr;   // argmax of the previous entropy-bounded pass
    int32_t* eb_info = nullptr;   // [4] outcome of the last entropy-bounded pass
    int32_t* bad = nullptr;
    float* logits_cap = nullptr;
    int32_t* cap_idx = nullptr;
    float* cap_gates = nullptr;
    float* cap_hidden = nullptr;
    void* cap_attn = nullptr;
    float* cap_rlog = nullptr;
    uint32_t cap_mask = 0;    // captures recorded by the next passes (buffers allocated)
    bool cap(uint32_t bit) const { return (cap_mask & bit) != 0; }
    int32_t* blk_canvas = nullptr;
    uint8_t* blk_mask = nullptr;

    // self-conditioning (cfg.self_cond): weights, the vocabulary-packed copy of E,
    // the posterior rows of the last pass and the signal chain u -> h1 -> H -> z
    bool sc = false;
    int Fsc = 0;
    void* sc_w1 = nullptr;      // bf16: packed [d][2 Fsc] gate | up columns; f32: Wg [d][Fsc]
    void* sc_wu = nullptr;      // f32: Wu [d][Fsc]
    void* sc_w2 = nullptr;      // bf16: packed [Fsc][d]; f32: Wd [Fsc][d]
    void* embed_kn = nullptr;   // bf16: E packed as the B operand of a [V] x [d] product
    void* sc_post = nullptr;    // posterior rows [rows_max][V] (bf16 or float)
    float* sc_part = nullptr;   // stream-K partial tiles of the contraction
    float* sc_u = nullptr;      // p0 E, float [rows_max][d]
    void* sc_uf = nullptr;      // bf16 fragment order of u
    float* sc_h1 = nullptr;     // [rows_max][2 Fsc] gate | up pre-activations
    void* sc_hf = nullptr;      // gated hidden layer (bf16 fragment order, or float rows)
    float* sc_z = nullptr;      // the signal the next pass reads, float [rows_max][d]

    void* stage = nullptr;
    size_t stage_bytes = 0;

    int64_t n_ctx = 0;
    int k_blk = 0;
    bool prefilled = false;

    // layer stack of a denoise pass as a HIP graph, captured for one context
    // length (the attention and RoPE launches depend on it) and replayed
    bool use_graphs = true;
    hipStream_t gstream = nullptr;   // capture stream (default priority)
    hipGraphExec_t gexec = nullptr;
    int64_t g_nctx = -1;
    int g_rows = -1;

    // per-kernel-class event timing
    bool prof = false;
    std::vector<hipEvent_t> ev;
    std::vector<int> ev_cls;
    int ev_used = 0;

    int alloc(void** p, size_t bytes) {
        if (bytes == 0) bytes = 256;
        const hipError_t e = hipMalloc(p, bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            *p = nullptr;
            return fail(DG_ENOMEM, "hipMalloc of %zu bytes failed: %s", bytes, hipGetErrorString(e));
        }
        allocs.push_back(*p);
        if (hipMemset(*p, 0, bytes) != hipSuccess) return fail(DG_EHIP, "hipMemset failed");
        return DG_OK;
    }
    template <typename T>
    int allocT(T** p, size_t count) {
        void* v = nullptr;
        int r = alloc(&v, count * sizeof(T));
        *p = (T*)v;
        return r;
    }

    size_t kv_layer_elems() const { return (size_t)Hkv * kv_rows * D; }
    void* klayer(int l) const { return (char*)kcache + (size_t)l * kv_layer_elems() * dsize(act); }
    void* vlayer(int l) const { return (char*)vcache + (size_t)l * kv_layer_elems() * dsize(act); }

    // loaded flags: [L][5 dense] then [L][3][E], then the three self-conditioning tensors
    uint8_t& dense_flag(int l, int kind) { return loaded[1 + l * 5 + kind]; }
    uint8_t& expert_flag(int l, int which, int e) {
        return loaded[1 + L * 5 + ((size_t)l * 3 + which) * E + e];
    }
    uint8_t& sc_flag(int which) { return loaded[1 + (size_t)L * 5 + (size_t)L * 3 * E + which]; }
};

// =========================================================================== helpers
static int validate_cfg(const dg_model_cfg* c) {
    if (!c) return fail(DG_EINVAL, "cfg is NULL");
    if (c->n_layers <= 0 || c->d_model <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
        c->head_dim <= 0 || c->n_experts <= 0 || c->top_k <= 0 || c->d_ff <= 0 ||
        c->vocab <= 0 || c->canvas <= 0 || c->max_ctx <= 0)
        return fail(DG_EINVAL, "all sizes must be positive");
    if (c->n_q_heads % c->n_kv_heads) return fail(DG_EINVAL, "n_q_heads %% n_kv_heads != 0");
    if (c->top_k > c->n_experts || c->top_k > 16) return fail(DG_EINVAL, "top_k must be <= E and <= 16");
    if (c->n_experts > 256 || c->n_experts % 4)
        return fail(DG_EINVAL, "n_experts must be a multiple of 4, at most 256");
    if (c->canvas > kMaxCanvas) return fail(DG_EINVAL, "canvas must be <= %d", kMaxCanvas);
    if (c->max_batch < 0 || (int64_t)c->canvas * (c->max_batch > 1 ? c->max_batch : 1) > 65536)
        return fail(DG_EINVAL, "max_batch must be >= 0 and max_batch * canvas <= 65536");
    if (c->head_dim & 1) return fail(DG_EINVAL, "head_dim must be even");
    if (c->d_model > 256 * kCombineCols || c->d_model % 4)
        return fail(DG_EINVAL, "d_model must be a multiple of 4, at most %d", 256 * kCombineCols);
    if (c->head_dim > 128) return fail(DG_EINVAL, "head_dim must be <= 128");
    if (c->max_ctx < c->canvas) return fail(DG_EINVAL, "max_ctx must hold at least one canvas");
    if (!(c->temperature > 0.f)) return fail(DG_EINVAL, "temperature must be > 0");
    if (c->self_cond != 0 && c->self_cond != 1) return fail(DG_EINVAL, "self_cond must be 0 or 1");
    if (c->sc_ff < 0) return fail(DG_EINVAL, "sc_ff must be >= 0");
    if (c->self_cond) {
        const int fsc = c->sc_ff > 0 ? c->sc_ff : c->d_model;
        if (c->act_dtype == DG_BF16 && fsc % 64)
            return fail(DG_EINVAL, "bf16 self-conditioning needs sc_ff a multiple of 64");
        if (c->act_dtype != DG_BF16 && (fsc % 4 || c->vocab % 8))
            return fail(DG_EINVAL, "f32 self-conditioning needs sc_ff %% 4 == 0 and vocab %% 8 == 0");
    }
    if (!(c->rope_base > 0.0)) return fail(DG_EINVAL, "rope_base must be > 0");
    if (c->act_dtype == DG_F32) {
        if (c->expert_dtype != DG_F32) return fail(DG_EINVAL, "f32 activations need f32 experts");
        if (c->head_dim != 64 && c->head_dim != 128) return fail(DG_EINVAL, "f32 head_dim must be 64 or 128");
    } else if (c->act_dtype == DG_BF16) {
        if (c->expert_dtype != DG_BF16 && c->expert_dtype != DG_FP8_E4M3 &&
            c->expert_dtype != DG_MXFP4)
            return fail(DG_EINVAL, "bf16 activations need bf16, e4m3 or MX FP4 experts");
        if (c->expert_dtype == DG_MXFP4 && c->d_model % 128)
            return fail(DG_EINVAL, "MX FP4 experts need d_model a multiple of 128");
        if (c->head_dim != 128) return fail(DG_EINVAL, "bf16 path needs head_dim 128");
        if (c->d_model % 64 || c->d_ff % 64) return fail(DG_EINVAL, "bf16 path needs d_model and d_ff multiples of 64");
        if (c->vocab % 128) return fail(DG_EINVAL, "bf16 path needs vocab multiple of 128");
        if ((c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim % 64 || c->n_experts % 64)
            return fail(DG_EINVAL, "bf16 path needs (Hq+2Hkv)*D and E multiples of 64");
    } else {
        return fail(DG_EINVAL, "act_dtype must be DG_F32 or DG_BF16");
    }
    return DG_OK;
}

static int ensure_ready(dg_handle* h) {
    if (h->ready) return DG_OK;
    for (size_t i = 0; i < h->loaded.size(); ++i)
        if (!h->loaded[i]) return fail(DG_ESTATE, "weights not fully loaded (slot %zu missing)", i);
    h->ready = true;
    return DG_OK;
}

// fp8 and MX FP4 experts read e4m3 copies of the normed activations.
static bool e4m3_inputs(const dg_handle* h) { return h->edt == kFP8 || h->edt == kMX; }

static ExpertWeights expert_weights(dg_handle* h, int l) {
    ExpertWeights w;
    w.w1 = h->w1[l];
    w.wu = h->wu.empty() ? nullptr : h->wu[l];
    w.w2 = h->w2[l];
    w.s1 = h->s1.empty() ? nullptr : h->s1[l];
    w.s2 = h->s2.empty() ? nullptr : h->s2[l];
    w.x1 = h->x1.empty() ? nullptr : h->x1[l];
    w.x2 = h->x2.empty() ? nullptr : h->x2[l];
    return w;
}

// Row padding of the permuted entries: one MFMA row tile for the bf16/fp8 expert
// GEMMs (their activation fragments are 16 rows of one expert), none for f32.
static int moe_pad(const dg_handle* h) { return h->edt == kF32 ? 1 : kMoePad; }

// Expert-GEMM work list for a batch of n tokens (grid bound from n * k entries).
static MoeWork moe_work(dg_handle* h, int n) {
    MoeWork w;
    w.items = h->work_items;
    w.items2 = h->work_items + h->work_cap1;
    w.count = h->work_count;
    w.max_items = (n * h->k + kMoeItemRows - 1) / kMoeItemRows + h->E;
    w.max_items2 = (n * h->k + kMoeRows - 1) / kMoeRows + h->E;
    return w;
}

// Drop the captured layer-stack graph (weights or context changed).
static void drop_graph(dg_handle* h) {
    if (h->gexec) (void)hipGraphExecDestroy(h->gexec);
    h->gexec = nullptr;
    h->g_nctx = -1;
    h->g_rows = -1;
}

// Allocate the capture buffers a mask needs (once) and make it the active mask.
static int alloc_captures(dg_handle* h, uint32_t mask) {
    const size_t L = h->L, C = h->rows_max, k = h->k;
    if ((mask & DG_CAP_LOGITS) && !h->logits_cap) DG_TRY(h->allocT(&h->logits_cap, C * h->V));
    if ((mask & DG_CAP_ROUTING) && !h->cap_idx) {
        DG_TRY(h->allocT(&h->cap_idx, L * C * k));
        DG_TRY(h->allocT(&h->cap_gates, L * C * k));
    }
    if ((mask & DG_CAP_HIDDEN) && !h->cap_hidden) DG_TRY(h->allocT(&h->cap_hidden, L * C * h->d));
    if ((mask & DG_CAP_ATTN) && !h->cap_attn)
        DG_TRY(h->alloc(&h->cap_attn, L * C * h->Hq * h->D * dsize(h->act)));
    if ((mask & DG_CAP_ROUTER_LOGITS) && !h->cap_rlog) DG_TRY(h->allocT(&h->cap_rlog, L * C * h->E));
    h->cap_mask = mask;
    return DG_OK;
}

#define K_TRY(expr) HIP_TRY(expr)

// Event pair around one launch of a timed kernel class (no-op unless profiling).
struct ProfScope {
    dg_handle* h;
    hipStream_t s;
    int slot = -1;
    ProfScope(dg_handle* hh, int cls, hipStream_t ss) : h(hh), s(ss) {
        if (h->prof && h->ev_used + 2 <= (int)h->ev.size()) {
            slot = h->ev_used;
            h->ev_used += 2;
            h->ev_cls[slot] = cls;
            (void)hipEventRecord(h->ev[slot], s);
        }
    }
    ~ProfScope() {
        if (slot >= 0) (void)hipEventRecord(h->ev[slot + 1], s);
    }
};

// MoE block of one layer on h->a (and h->a8) for n tokens: router -> permute ->
// expert GEMMs.  Leaves Y, gates, inv ready for the combine.
static int run_moe(dg_handle* h, int l, int n, const void* xin, const uint8_t* xin8,
                   hipStream_t s) {
    // the router GEMM is narrow (N = E): split K over workgroups; top-k adds the partials
    const int ksplit = (h->act == kBF16 && !h->cap(DG_CAP_ROUTER_LOGITS)) ? kRouterSplit : 1;
    {
        ProfScope p(h, DG_PROF_DENSE, s);
        K_TRY(launch_gemm(h->act, kEpiStoreF32, xin, h->d, n, h->wr[l], h->d, h->E, h->rlog, h->E,
                          s, ksplit));
    }
    K_TRY(launch_router_permute(h->rlog, ksplit, n, h->E, h->k, h->idx, h->gates, h->counts,
                                h->base, h->offsets, h->perm_token, h->inv, moe_work(h, n),
                                moe_pad(h), s));
    ExpertWeights w = expert_weights(h, l);
    const int rows = (int)moe_rows_cap(n, h->k, h->E, moe_pad(h));
    const bool e4 = h->edt == kFP8 || h->edt == kMX;
    const void* X1 = e4 ? (const void*)xin8 : xin;
    // fp8 and MX FP4 experts take their e4m3 inputs gathered into fragment order; the
    // bf16 GEMM reads the token rows in place
    if (e4)
        K_TRY(launch_moe_gather8(X1, h->d, h->perm_token, h->offsets, h->E, rows, h->Xf, s,
                                 h->edt == kMX));
    {
        ProfScope p(h, DG_PROF_MOE_GEMM1, s);
        K_TRY(launch_moe_gemm1(h->edt, w, X1, h->perm_token, h->offsets, h->E, h->d, h->F, rows,
                               moe_work(h, n), h->Xf, h->H, s));
    }
    {
        ProfScope p(h, DG_PROF_MOE_GEMM2, s);
        K_TRY(launch_moe_gemm2(h->edt, w, h->H, h->offsets, h->E, h->d, h->F, rows,
                               moe_work(h, n), h->Y, h->bad, s));
    }
    return DG_OK;
}

// One transformer layer for n tokens at positions pos0..pos0+n-1 (x, a hold the
// residual and its norm).  Keys: cache rows [0, pos0 + n).  kv_only: stop after
// writing K/V (the last encoder layer).
// period > 0: the n rows are n / period canvases at the same positions pos0..pos0 +
// period - 1 (a batched decoder pass); canvas b's cache rows are pos0 + b period +
// i, and its queries see the context rows [0, pos0) and its own rows.
static int run_layer(dg_handle* h, int l, int n, int64_t pos0, bool causal, bool kv_only,
                     hipStream_t s, bool capture = false, int period = 0) {
    if (h->act == kBF16) {
        // Af: a in fragment order, from the norm that wrote it.  The QKV weights are
        // pair-tiled (rope_hd 128), so the GEMM's epilogue applies RoPE and writes Q
        // and the K/V cache rows itself.
        ProfScope p(h, DG_PROF_DENSE, s);
        RopeArgs ra;
        ra.Hq = h->Hq;
        ra.Hkv = h->Hkv;
        ra.pos0 = pos0;
        ra.period = period;
        ra.cos_t = h->cos_t;
        ra.sin_t = h->sin_t;
        ra.q = h->q;
        ra.kc = h->klayer(l);
        ra.vc = h->vlayer(l);
        ra.kv_rows = h->kv_rows;
        K_TRY(launch_gemm_frag(kEpiRope, h->Af, n, h->wqkv[l], h->d, h->qkv_n, nullptr, 0, s, 1,
                               &ra));
    } else {
        {
            ProfScope p(h, DG_PROF_DENSE, s);
            K_TRY(launch_gemm(h->act, kEpiStoreF32, h->a, h->d, n, h->wqkv[l], h->d, h->qkv_n,
                              h->qkv, h->qkv_n, s));
        }
        K_TRY(launch_rope_scatter(h->act, h->qkv, n, h->Hq, h->Hkv, h->D, pos0, period, h->cos_t,
                                  h->sin_t, h->q, h->klayer(l), h->vlayer(l), h->kv_rows, s));
    }
    if (kv_only) return DG_OK;
    AttnArgs aa;
    aa.q = h->q;
    aa.k = h->klayer(l);
    aa.v = h->vlayer(l);
    // bf16: the output projection reads the fragment-order copy; the row-order one is
    // written only for the attention capture
    aa.of = h->act == kBF16 ? h->Af : nullptr;
    aa.o = h->act == kBF16 && !(capture && h->cap(DG_CAP_ATTN)) ? nullptr : h->attn_o;
    aa.Hq = h->Hq;
    aa.Hkv = h->Hkv;
    aa.M = n;
    aa.S = (int)(pos0 + (period > 0 ? period : n));
    aa.ctx = period > 0 ? pos0 : 0;
    aa.canvas = period;
    aa.D = h->D;
    aa.kv_rows = h->kv_rows;
    aa.v_rows = h->kv_rows;
    aa.scale = 1.0f / sqrtf((float)h->D);
    aa.causal = causal ? 1 : 0;
    aa.q_pos0 = pos0;
    aa.part = h->part;
    aa.part_bytes = h->part_bytes;
    aa.bad = h->bad;
    {
        ProfScope p(h, DG_PROF_ATTENTION, s);
        K_TRY(launch_attention(h->act, aa, s));
    }
    if (capture && h->cap(DG_CAP_ATTN)) {
        const size_t b = (size_t)n * h->Hq * h->D * dsize(h->act);
        HIP_TRY(hipMemcpyAsync((char*)h->cap_attn + (size_t)l * b, h->attn_o, b,
                               hipMemcpyDeviceToDevice, s));
    }
    {
        ProfScope p(h, DG_PROF_DENSE, s);
        if (h->act == kBF16) {   // Af: the attention output in fragment order
            K_TRY(launch_gemm_frag(kEpiAddF32, h->Af, n, h->wo[l], h->Hq * h->D, h->d, h->x, h->d, s));
        } else {
            K_TRY(launch_gemm(h->act, kEpiAddF32, h->attn_o, h->Hq * h->D, n, h->wo[l],
                              h->Hq * h->D, h->d, h->x, h->d, s));
        }
    }
    K_TRY(launch_rmsnorm(h->act, h->x, n, h->d, h->cfg.rms_eps, h->a,
                         e4m3_inputs(h) ? h->a8 : nullptr, nullptr, s));
    DG_TRY(run_moe(h, l, n, h->a, h->a8, s));
    if (capture && h->cap(DG_CAP_ROUTER_LOGITS))
        HIP_TRY(hipMemcpyAsync(h->cap_rlog + (size_t)l * n * h->E, h->rlog, (size_t)n * h->E * 4,
                               hipMemcpyDeviceToDevice, s));
    // residual add, then the next norm (next layer's input, or the final norm)
    K_TRY(launch_moe_combine(h->act, 0, h->Y, n, h->d, h->k, h->gates, h->inv, h->x,
                             h->cfg.rms_eps, h->a, e4m3_inputs(h) ? h->a8 : nullptr, h->Af,
                             nullptr, s));
    return DG_OK;
}

// Causal encoder over n tokens at positions pos0.. (prefill chunk or commit).
static int encode(dg_handle* h, const int32_t* tokens, int n, int64_t pos0, hipStream_t s) {
    K_TRY(launch_embed_rmsnorm(h->act, h->act == kBF16, tokens, h->embed, h->V, n, h->d,
                               h->cfg.rms_eps, h->x, h->a, h->Af, h->bad, s));
    for (int l = 0; l < h->L; ++l)
        DG_TRY(run_layer(h, l, n, pos0, true, l == h->L - 1, s));
    return DG_OK;
}

// =========================================================================== C ABI
extern "C" {

const char* dg_last_error(void) { return g_err.c_str(); }

int dg_create(const dg_model_cfg* cfg, dg_handle** out) {
    g_err.clear();
    if (!out) return fail(DG_EINVAL, "out is NULL");
    *out = nullptr;
    DG_TRY(validate_cfg(cfg));
    dg_handle* h = new dg_handle();
    h->cfg = *cfg;
    h->L = cfg->n_layers;
    h->d = cfg->d_model;
    h->Hq = cfg->n_q_heads;
    h->Hkv = cfg->n_kv_heads;
    h->D = cfg->head_dim;
    h->E = cfg->n_experts;
    h->k = cfg->top_k;
    h->F = cfg->d_ff;
    h->V = cfg->vocab;
    h->C = cfg->canvas;
    h->B_max = cfg->max_batch > 1 ? cfg->max_batch : 1;
    h->rows_max = h->C * h->B_max;
    h->act = cfg->act_dtype == DG_F32 ? kF32 : kBF16;
    h->edt = cfg->expert_dtype == DG_F32 ? kF32 : cfg->expert_dtype == DG_BF16 ? kBF16
           : cfg->expert_dtype == DG_MXFP4 ? kMX : kFP8;
    h->max_ctx = cfg->max_ctx;
    h->kv_rows = (cfg->max_ctx + 31) & ~(int64_t)31;
    h->max_tokens = std::max(h->rows_max, kPrefillChunk);
    h->qkv_n = (h->Hq + 2 * h->Hkv) * h->D;
    h->sc = cfg->self_cond != 0;
    h->Fsc = h->sc ? (cfg->sc_ff > 0 ? cfg->sc_ff : cfg->d_model) : 0;
    h->loaded.assign(1 + (size_t)h->L * 5 + (size_t)h->L * 3 * h->E, 0);
    if (h->sc) h->loaded.resize(h->loaded.size() + 3, 0);

    auto cleanup = [&](int r) {
        dg_destroy(h);
        return r;
    };
    const size_t as = dsize(h->act), es = dsize(h->edt);
    const size_t L = h->L, d = h->d, E = h->E, F = h->F, V = h->V, k = h->k;
    const size_t T = h->max_tokens;
    int r;
#define A_TRY(call) do { if ((r = (call)) != DG_OK) return cleanup(r); } while (0)
    A_TRY(h->alloc(&h->embed, V * d * as));
    h->wqkv.resize(L);
    h->wo.resize(L);
    h->wr.resize(L);
    h->w1.resize(L);
    h->w2.resize(L);
    if (h->edt == kF32) h->wu.resize(L);
    if (h->edt == kFP8) {
        h->s1.resize(L);
        h->s2.resize(L);
    }
    if (h->edt == kMX) {
        h->x1.resize(L);
        h->x2.resize(L);
    }
    for (size_t l = 0; l < L; ++l) {
        A_TRY(h->alloc(&h->wqkv[l], d * h->qkv_n * as));
        A_TRY(h->alloc(&h->wo[l], (size_t)h->Hq * h->D * d * as));
        A_TRY(h->alloc(&h->wr[l], d * E * as));
        if (h->edt == kMX) {
            A_TRY(h->alloc(&h->w1[l], E * mx_code_bytes(h->d, 2 * h->F)));
            A_TRY(h->alloc(&h->w2[l], E * mx_code_bytes(h->F, h->d)));
            A_TRY(h->allocT(&h->x1[l], E * mx_scale_bytes(h->d, 2 * h->F)));
            A_TRY(h->allocT(&h->x2[l], E * mx_scale_bytes(h->F, h->d)));
            continue;
        }
        A_TRY(h->alloc(&h->w1[l], E * d * F * es * (h->edt == kF32 ? 1 : 2)));
        if (h->edt == kF32) A_TRY(h->alloc(&h->wu[l], E * d * F * es));
        A_TRY(h->alloc(&h->w2[l], E * F * d * es));
        if (h->edt == kFP8) {
            A_TRY(h->allocT(&h->s1[l], E * 2 * F));
            A_TRY(h->allocT(&h->s2[l], E * d));
        }
    }
    const size_t kv = L * (size_t)h->Hkv * h->kv_rows * h->D * as;
    A_TRY(h->alloc(&h->kcache, kv));
    A_TRY(h->alloc(&h->vcache, kv));
    // RoPE tables in double precision, stored as float: angle = pos * base^(-2j/D)
    {
        const int half = h->D / 2;
        std::vector<float> c((size_t)h->kv_rows * half), sn((size_t)h->kv_rows * half);
        std::vector<double> theta(half);
        for (int j = 0; j < half; ++j) theta[j] = pow(cfg->rope_base, -2.0 * j / h->D);
        for (int64_t p = 0; p < h->kv_rows; ++p)
            for (int j = 0; j < half; ++j) {
                const double ang = (double)p * theta[j];
                c[(size_t)p * half + j] = (float)cos(ang);
                sn[(size_t)p * half + j] = (float)sin(ang);
            }
        A_TRY(h->allocT(&h->cos_t, c.size()));
        A_TRY(h->allocT(&h->sin_t, sn.size()));
        if (hipMemcpy(h->cos_t, c.data(), c.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
            hipMemcpy(h->sin_t, sn.data(), sn.size() * 4, hipMemcpyHostToDevice) != hipSuccess)
            return cleanup(fail(DG_EHIP, "RoPE table upload failed"));
    }
    A_TRY(h->allocT(&h->x, T * d));
    A_TRY(h->alloc(&h->a, T * d * as));
    if (h->edt == kFP8 || h->edt == kMX) A_TRY(h->allocT(&h->a8, T * d));
    if (h->act == kF32) A_TRY(h->allocT(&h->qkv, T * h->qkv_n));   // bf16: RoPE in the QKV epilogue
    A_TRY(h->alloc(&h->q, T * h->Hq * h->D * as));
    A_TRY(h->alloc(&h->attn_o, T * h->Hq * h->D * as));
    // split-KV partials, sized for the largest split call of any batch size
    h->part_bytes = h->act == kF32 ? 256 : attention_part_bytes_bound(h->D);
    A_TRY(h->alloc(&h->part, h->part_bytes));
    A_TRY(h->allocT(&h->rlog, T * E * kRouterSplit));
    A_TRY(h->allocT(&h->idx, T * k));
    A_TRY(h->allocT(&h->gates, T * k));
    const size_t n_chunks = (T * k + kPermChunk - 1) / kPermChunk;
    A_TRY(h->allocT(&h->counts, n_chunks * E));
    A_TRY(h->allocT(&h->base, n_chunks * E));
    const size_t rows = (size_t)moe_rows_cap(T, h->k, h->E, moe_pad(h));
    const size_t esz = h->edt == kF32 ? 4 : h->edt == kBF16 ? 2 : 1;
    A_TRY(h->allocT(&h->offsets, E + 1));
    A_TRY(h->allocT(&h->perm_token, rows));
    A_TRY(h->allocT(&h->inv, T * k));
    h->work_cap1 = (T * k + kMoeItemRows - 1) / kMoeItemRows + E;
    A_TRY(h->allocT(&h->work_items, (size_t)h->work_cap1 + (T * k + kMoeRows - 1) / kMoeRows + E));
    A_TRY(h->allocT(&h->work_count, 4));   // item counts and the two GEMMs' unit counters
    if (h->edt == kFP8 || h->edt == kMX) A_TRY(h->alloc(&h->Xf, rows * d * esz));
    if (h->act == kBF16)
        A_TRY(h->alloc(&h->Af, (T + 15) / 16 * 16 * std::max<size_t>(d, (size_t)h->Hq * h->D) * 2));
    // MX: H in the 128-column k-steps of the block-scaled MFMA; columns past F stay zero
    A_TRY(h->alloc(&h->H, rows * (h->edt == kMX ? (F + 127) / 128 * 128 : F) * esz));
    A_TRY(h->allocT(&h->Y, rows * d));
    const int ns = lm_head_slices(h->act, h->V);
    h->hp.n_slices = ns;
    A_TRY(h->allocT(&h->hp.m, (size_t)h->rows_max * ns));
    A_TRY(h->allocT(&h->hp.a, (size_t)h->rows_max * ns));
    A_TRY(h->allocT(&h->hp.s, (size_t)h->rows_max * ns));
    A_TRY(h->allocT(&h->hp.g, (size_t)h->rows_max * ns));
    A_TRY(h->allocT(&h->hp.gi, (size_t)h->rows_max * ns));
    A_TRY(h->allocT(&h->st_m, h->rows_max));
    A_TRY(h->allocT(&h->st_a, h->rows_max));
    A_TRY(h->allocT(&h->st_lse, h->rows_max));
    A_TRY(h->allocT(&h->st_conf, h->rows_max));
    A_TRY(h->allocT(&h->st_draw, h->rows_max));
    A_TRY(h->allocT(&h->st_ent, h->rows_max));
    A_TRY(h->allocT(&h->hp_q, (size_t)h->rows_max * ns));
    A_TRY(h->allocT(&h->eb_prev, h->C));
    A_TRY(h->allocT(&h->eb_info, 4));
    A_TRY(h->allocT(&h->bad, 1));
    A_TRY(h->allocT(&h->blk_canvas, h->rows_max));
    A_TRY(h->allocT(&h->blk_mask, h->rows_max));
    if (h->sc) {
        const size_t Fs = h->Fsc, R = h->rows_max, Rp = (R + 15) / 16 * 16;
        if (h->act == kBF16) {
            A_TRY(h->alloc(&h->sc_w1, d * 2 * Fs * 2));
            A_TRY(h->alloc(&h->sc_w2, Fs * d * 2));
            A_TRY(h->alloc(&h->embed_kn, V * d * 2));
            A_TRY(h->alloc(&h->sc_post, R * V * 2));
            A_TRY(h->allocT(&h->sc_part, sc_part_floats(h->rows_max, h->d, h->V)));
            A_TRY(h->alloc(&h->sc_uf, Rp * d * 2));
            A_TRY(h->alloc(&h->sc_hf, Rp * Fs * 2));
        } else {
            A_TRY(h->alloc(&h->sc_w1, d * Fs * 4));
            A_TRY(h->alloc(&h->sc_wu, d * Fs * 4));
            A_TRY(h->alloc(&h->sc_w2, Fs * d * 4));
            A_TRY(h->alloc(&h->sc_post, R * V * 4));
            A_TRY(h->alloc(&h->sc_hf, R * Fs * 4));
        }
        A_TRY(h->allocT(&h->sc_u, R * d));
        A_TRY(h->allocT(&h->sc_h1, R * 2 * Fs));
        A_TRY(h->allocT(&h->sc_z, R * d));
    }
    A_TRY(alloc_captures(h, cfg->capture_mask));
#undef A_TRY
    *out = h;
    return DG_OK;
}

void dg_destroy(dg_handle* h) {
    if (!h) return;
    (void)hipDeviceSynchronize();
    if (h->gexec) (void)hipGraphExecDestroy(h->gexec);
    if (h->gstream) (void)hipStreamDestroy(h->gstream);
    for (hipEvent_t e : h->ev) (void)hipEventDestroy(e);
    for (void* p : h->allocs) (void)hipFree(p);
    if (h->stage) (void)hipFree(h->stage);
    delete h;
}

static int stage_upload(dg_handle* h, const void* src, size_t bytes, void** dev) {
    if (bytes > h->stage_bytes) {
        if (h->stage) (void)hipFree(h->stage);
        h->stage = nullptr;
        h->stage_bytes = 0;
        if (hipMalloc(&h->stage, bytes) != hipSuccess) {
            (void)hipGetLastError();
            return fail(DG_ENOMEM, "staging allocation of %zu bytes failed", bytes);
        }
        h->stage_bytes = bytes;
    }
    HIP_TRY(hipMemcpy(h->stage, src, bytes, hipMemcpyHostToDevice));
    *dev = h->stage;
    return DG_OK;
}

int dg_load_tensor(dg_handle* h, int32_t kind, int32_t layer, int32_t expert,
                   const void* host_src, size_t bytes, const void* host_scales) {
    g_err.clear();
    if (!h || !host_src) return fail(DG_EINVAL, "NULL handle or source");
    if (kind < DG_T_EMBED || kind > DG_T_SC_WD) return fail(DG_EINVAL, "bad tensor kind %d", kind);
    const bool is_sc = kind >= DG_T_SC_WG;
    if (is_sc && !h->sc) return fail(DG_EINVAL, "self-conditioning tensors need cfg.self_cond");
    const bool is_exp = kind >= DG_T_WG && !is_sc;
    if (kind != DG_T_EMBED && !is_sc && (layer < 0 || layer >= h->L))
        return fail(DG_EINVAL, "bad layer %d", layer);
    HIP_TRY(hipDeviceSynchronize());
    drop_graph(h);
    if (is_exp && (expert < -1 || expert >= h->E)) return fail(DG_EINVAL, "bad expert %d", expert);
    const int dt = is_exp ? h->edt : h->act;
    const size_t es = dsize(dt);
    const int nexp = (is_exp && expert < 0) ? h->E : 1;
    const int e0 = (is_exp && expert >= 0) ? expert : 0;
    int K = 0, N = 0;
    switch (kind) {
        case DG_T_EMBED: K = h->d; N = h->V; break;
        case DG_T_WQ: K = h->d; N = h->Hq * h->D; break;
        case DG_T_WK: case DG_T_WV: K = h->d; N = h->Hkv * h->D; break;
        case DG_T_WO: K = h->Hq * h->D; N = h->d; break;
        case DG_T_WR: K = h->d; N = h->E; break;
        case DG_T_WG: case DG_T_WU: K = h->d; N = h->F; break;
        case DG_T_WD: K = h->F; N = h->d; break;
        case DG_T_SC_WG: case DG_T_SC_WU: K = h->d; N = h->Fsc; break;
        case DG_T_SC_WD: K = h->Fsc; N = h->d; break;
    }
    // MX FP4: two E2M1 codes per byte
    const size_t per = dt == kMX ? (size_t)K * N / 2 : (size_t)K * N * es;
    if (bytes != per * nexp)
        return fail(DG_EINVAL, "tensor kind %d: expected %zu bytes, got %zu", kind, per * nexp, bytes);
    if ((dt == kFP8 || dt == kMX) && !host_scales)
        return fail(DG_EINVAL, "e4m3 and MX FP4 tensors need their scales");
    void* src = nullptr;
    DG_TRY(stage_upload(h, host_src, bytes, &src));
    hipStream_t s = 0;
    if (kind == DG_T_EMBED) {
        if (dt == kF32) HIP_TRY(hipMemcpy(h->embed, src, bytes, hipMemcpyDeviceToDevice));
        else HIP_TRY(launch_pack_b16(src, false, K, N, 1, 0, h->embed, s));
        // the self-conditioning contraction runs over the vocabulary: [V] x [d]
        if (dt != kF32 && h->sc) HIP_TRY(launch_pack_b16(src, true, N, K, 1, 0, h->embed_kn, s));
        h->loaded[0] = 1;
    } else if (is_sc) {
        const int which = kind - DG_T_SC_WG;   // 0 gate, 1 up, 2 down
        if (dt == kF32) {
            void* dst = which == 0 ? h->sc_w1 : which == 1 ? h->sc_wu : h->sc_w2;
            HIP_TRY(hipMemcpy(dst, src, bytes, hipMemcpyDeviceToDevice));
        } else if (which < 2) {   // gate columns 0..Fsc-1, up columns Fsc..2Fsc-1
            HIP_TRY(launch_pack_b16(src, true, K, N, 1, which * (h->Fsc / 16), h->sc_w1, s));
        } else {
            HIP_TRY(launch_pack_b16(src, true, K, N, 1, 0, h->sc_w2, s));
        }
        h->sc_flag(which) = 1;
    } else if (!is_exp) {
        void* dst = nullptr;
        int col0 = 0, ldn = N;
        if (kind == DG_T_WQ || kind == DG_T_WK || kind == DG_T_WV) {
            dst = h->wqkv[layer];
            ldn = h->qkv_n;
            col0 = kind == DG_T_WQ ? 0 : kind == DG_T_WK ? h->Hq * h->D : (h->Hq + h->Hkv) * h->D;
        } else if (kind == DG_T_WO) dst = h->wo[layer];
        else dst = h->wr[layer];
        if (dt == kF32)
            HIP_TRY(hipMemcpy2D((float*)dst + col0, (size_t)ldn * 4, src, (size_t)N * 4,
                                (size_t)N * 4, K, hipMemcpyDeviceToDevice));
        else   // Q, K and V columns pair-tiled for the QKV GEMM's RoPE epilogue
            HIP_TRY(launch_pack_b16(src, true, K, N, 1, col0 / 16, dst, s, kind <= DG_T_WV ? 128 : 0));
        h->dense_flag(layer, kind - DG_T_WQ) = 1;
    } else {
        const int which = kind - DG_T_WG;   // 0 gate, 1 up, 2 down
        std::vector<float> dummy;
        float* sdev = nullptr;
        if (dt == kFP8 || dt == kMX) {
            // scales are small: upload them through a temporary allocation (MX: one E8M0
            // byte per 32 rows of a column)
            const size_t sb = dt == kMX ? (size_t)(K / 32) * N * nexp : (size_t)N * nexp * 4;
            if (hipMalloc(&sdev, sb) != hipSuccess) return fail(DG_ENOMEM, "scale staging failed");
            if (hipMemcpy(sdev, host_scales, sb, hipMemcpyHostToDevice) != hipSuccess) {
                (void)hipFree(sdev);
                return fail(DG_EHIP, "scale upload failed");
            }
        }
        int rc = DG_OK;
        for (int i = 0; i < nexp && rc == DG_OK; ++i) {
            const int e = e0 + i;
            const char* se = (const char*)src + per * i;
            hipError_t he = hipSuccess;
            if (dt == kF32) {
                void* dst = which == 0 ? h->w1[layer] : which == 1 ? h->wu[layer] : h->w2[layer];
                he = hipMemcpy((char*)dst + per * e, se, per, hipMemcpyDeviceToDevice);
            } else if (dt == kMX) {
                const uint8_t* sx = (const uint8_t*)sdev + (size_t)(K / 32) * N * i;
                if (which < 2)   // gate and up interleaved per 16 columns, as for bf16
                    he = launch_pack_mx((const uint8_t*)se, sx, K, N, 2, which, 2 * N / 16,
                                        (char*)h->w1[layer] + (size_t)e * mx_code_bytes(K, 2 * N),
                                        h->x1[layer] + (size_t)e * mx_scale_bytes(K, 2 * N), s);
                else
                    he = launch_pack_mx((const uint8_t*)se, sx, K, N, 1, 0, N / 16,
                                        (char*)h->w2[layer] + (size_t)e * mx_code_bytes(K, N),
                                        h->x2[layer] + (size_t)e * mx_scale_bytes(K, N), s);
            } else if (dt == kBF16) {
                if (which < 2) {
                    char* dst = (char*)h->w1[layer] + (size_t)e * 2 * per;
                    he = launch_pack_b16(se, true, K, N, 2, which, dst, s);
                } else {
                    he = launch_pack_b16(se, true, K, N, 1, 0, (char*)h->w2[layer] + per * e, s);
                }
            } else {
                if (which < 2) {
                    char* dst = (char*)h->w1[layer] + (size_t)e * 2 * per;
                    he = launch_pack_b8(se, K, N, 2, which, dst, s);
                    if (he == hipSuccess)
                        he = launch_scatter_scales(sdev + (size_t)N * i, N, 2, which,
                                                   h->s1[layer] + (size_t)e * 2 * N, s);
                } else {
                    he = launch_pack_b8(se, K, N, 1, 0, (char*)h->w2[layer] + per * e, s);
                    if (he == hipSuccess)
                        he = hipMemcpy(h->s2[layer] + (size_t)e * N, sdev + (size_t)N * i,
                                       (size_t)N * 4, hipMemcpyDeviceToDevice);
                }
            }
            if (he != hipSuccess) rc = fail(DG_EHIP, "expert load failed: %s", hipGetErrorString(he));
            else h->expert_flag(layer, which, e) = 1;
        }
        if (hipDeviceSynchronize() != hipSuccess && rc == DG_OK) rc = fail(DG_EHIP, "load sync failed");
        if (sdev) (void)hipFree(sdev);
        return rc;
    }
    HIP_TRY(hipDeviceSynchronize());
    return DG_OK;
}

int dg_set_graphs(dg_handle* h, int32_t enable) {
    g_err.clear();
    if (!h) return fail(DG_EINVAL, "NULL handle");
    HIP_TRY(hipDeviceSynchronize());
    h->use_graphs = enable != 0;
    if (!h->use_graphs) drop_graph(h);
    return DG_OK;
}

int dg_set_capture(dg_handle* h, uint32_t capture_mask) {
    g_err.clear();
    if (!h) return fail(DG_EINVAL, "NULL handle");
    if (capture_mask & ~(uint32_t)63) return fail(DG_EINVAL, "unknown capture bits");
    HIP_TRY(hipDeviceSynchronize());
    return alloc_captures(h, capture_mask);
}

int dg_profile_begin(dg_handle* h, int32_t max_launches) {
    g_err.clear();
    if (!h || max_launches <= 0) return fail(DG_EINVAL, "bad profile arguments");
    while ((int)h->ev.size() < 2 * max_launches) {
        hipEvent_t e;
        HIP_TRY(hipEventCreate(&e));
        h->ev.push_back(e);
    }
    h->ev_cls.assign(h->ev.size(), -1);
    h->ev_used = 0;
    h->prof = true;
    return DG_OK;
}

int dg_profile_end(dg_handle* h, double* total_ms, int32_t* counts) {
    g_err.clear();
    if (!h || !total_ms || !counts) return fail(DG_EINVAL, "NULL argument");
    h->prof = false;
    HIP_TRY(hipDeviceSynchronize());
    for (int c = 0; c < DG_PROF_N; ++c) {
        total_ms[c] = 0.0;
        counts[c] = 0;
    }
    for (int i = 0; i + 1 < h->ev_used; i += 2) {
        float ms = 0.f;
        HIP_TRY(hipEventElapsedTime(&ms, h->ev[i], h->ev[i + 1]));
        const int c = h->ev_cls[i];
        if (c >= 0 && c < DG_PROF_N) {
            total_ms[c] += ms;
            counts[c] += 1;
        }
    }
    h->ev_used = 0;
    return DG_OK;
}

int dg_set_self_cond(dg_handle* h, const float* d_z, int32_t rows, void* stream) {
    g_err.clear();
    if (!h || !d_z) return fail(DG_EINVAL, "NULL handle or signal");
    if (!h->sc) return fail(DG_ESTATE, "self-conditioning is off");
    if (rows < 0 || rows > h->rows_max)
        return fail(DG_EINVAL, "rows %d outside [0, %d]", rows, h->rows_max);
    HIP_TRY(hipMemcpyAsync(h->sc_z, d_z, (size_t)rows * h->d * 4, hipMemcpyDeviceToDevice,
                           (hipStream_t)stream));
    return DG_OK;
}

int dg_reset_context(dg_handle* h) {
    if (!h) return fail(DG_EINVAL, "NULL handle");
    drop_graph(h);
    h->n_ctx = 0;
    h->k_blk = 0;
    h->prefilled = false;
    return DG_OK;
}

int dg_set_state(dg_handle* h, int64_t n_ctx, int32_t k_blk) {
    g_err.clear();
    if (!h) return fail(DG_EINVAL, "NULL handle");
    if (n_ctx < 0 || n_ctx + h->C > h->max_ctx || k_blk < 0)
        return fail(DG_EINVAL, "need 0 <= n_ctx, n_ctx + C <= max_ctx %lld and k_blk >= 0",
                    (long long)h->max_ctx);
    DG_TRY(ensure_ready(h));
    h->n_ctx = n_ctx;
    h->k_blk = k_blk;
    h->prefilled = true;
    return DG_OK;
}

int dg_get_state(dg_handle* h, int64_t* n_ctx, int32_t* k_blk) {
    if (!h) return fail(DG_EINVAL, "NULL handle");
    if (n_ctx) *n_ctx = h->n_ctx;
    if (k_blk) *k_blk = h->k_blk;
    return DG_OK;
}

int dg_prefill_prompt_kv(dg_handle* h, const int32_t* d_prompt_ids, int32_t P, void* stream) {
    g_err.clear();
    if (!h) return fail(DG_EINVAL, "NULL handle");
    if (P < 0) return fail(DG_EINVAL, "P must be >= 0");
    if (P > 0 && !d_prompt_ids) return fail(DG_EINVAL, "NULL prompt ids");
    if ((int64_t)P + h->C > h->max_ctx)
        return fail(DG_ECAPACITY, "prompt %d plus one canvas %d exceeds max_ctx %lld", P, h->C,
                    (long long)h->max_ctx);
    DG_TRY(ensure_ready(h));
    hipStream_t s = (hipStream_t)stream;
    for (int c0 = 0; c0 < P; c0 += kPrefillChunk) {
        const int n = std::min(kPrefillChunk, P - c0);
        DG_TRY(encode(h, d_prompt_ids + c0, n, c0, s));
    }
    h->n_ctx = P;
    h->k_blk = 0;
    h->prefilled = true;
    return DG_OK;
}

int dg_commit_canvas(dg_handle* h, const int32_t* d_canvas, void* stream) {
    g_err.clear();
    if (!h || !d_canvas) return fail(DG_EINVAL, "NULL handle or canvas");
    if (!h->prefilled) return fail(DG_ESTATE, "commit before prefill");
    if (h->n_ctx + h->C > h->max_ctx)
        return fail(DG_ECAPACITY, "commit would exceed max_ctx %lld", (long long)h->max_ctx);
    DG_TRY(ensure_ready(h));
    DG_TRY(encode(h, d_canvas, h->C, h->n_ctx, (hipStream_t)stream));
    h->n_ctx += h->C;
    h->k_blk += 1;
    return DG_OK;
}

// The L decoder layers of a denoise pass over the canvas at n_ctx, as one HIP
// graph replayed on stream s.  Captured on the handle's own stream the first
// time for this context length.  The kernels record no memset nodes.
static int run_layers_graph(dg_handle* h, int B, hipStream_t s) {
    const int rows = B * h->C;
    if (!h->gexec || h->g_nctx != h->n_ctx || h->g_rows != rows) {
        drop_graph(h);
        if (!h->gstream) HIP_TRY(hipStreamCreateWithFlags(&h->gstream, hipStreamNonBlocking));
        HIP_TRY(hipStreamBeginCapture(h->gstream, hipStreamCaptureModeThreadLocal));
        int rc = DG_OK;
        for (int l = 0; l < h->L && rc == DG_OK; ++l)
            rc = run_layer(h, l, rows, h->n_ctx, false, false, h->gstream, false,
                           B > 1 ? h->C : 0);
        hipGraph_t g = nullptr;
        const hipError_t e = hipStreamEndCapture(h->gstream, &g);
        if (rc != DG_OK || e != hipSuccess) {
            if (g) (void)hipGraphDestroy(g);
            (void)hipGetLastError();
            return rc != DG_OK ? rc : fail(DG_EHIP, "graph capture failed: %s", hipGetErrorString(e));
        }
        const hipError_t ei = hipGraphInstantiate(&h->gexec, g, nullptr, nullptr, 0);
        (void)hipGraphDestroy(g);
        if (ei != hipSuccess) {
            h->gexec = nullptr;
            return fail(DG_EHIP, "graph instantiation failed: %s", hipGetErrorString(ei));
        }
        h->g_nctx = h->n_ctx;
        h->g_rows = rows;
    }
    HIP_TRY(hipGraphLaunch(h->gexec, s));
    return DG_OK;
}

// Decoder over the canvas, LM head at temperature 1 / inv_tau and the per-position
// statistics (with the predictive entropy when ent is set): everything of a pass
// but the sampler.
// B canvases of C rows each (B > 1: a batch at the same positions, see run_layer).
// The next pass's self-conditioning signal from the posterior rows the head and its
// statistics left in sc_post: u = p0 E (the contraction over the vocabulary), then
// z = (silu(u Wg) * (u Wu)) Wd.
static int run_self_cond(dg_handle* h, int rows, hipStream_t s) {
    const int d = h->d, F = h->Fsc;
    if (h->act == kBF16) {
        {
            ProfScope p(h, DG_PROF_SELF_COND, s);
            K_TRY(launch_sc_expect((const uint16_t*)h->sc_post, rows, h->V, h->embed_kn, d,
                                   h->sc_part, s));
        }
        K_TRY(launch_sc_reduce(h->sc_part, rows, d, h->V, h->sc_u, h->sc_uf, s));
        K_TRY(launch_gemm_frag(kEpiStoreF32, h->sc_uf, rows, h->sc_w1, d, 2 * F, h->sc_h1, 2 * F, s));
        K_TRY(launch_swiglu_rows(kBF16, h->sc_h1, rows, F, h->sc_hf, s));
        K_TRY(launch_gemm_frag(kEpiStoreF32, h->sc_hf, rows, h->sc_w2, F, d, h->sc_z, d, s));
    } else {
        {
            ProfScope p(h, DG_PROF_SELF_COND, s);
            K_TRY(launch_gemm(kF32, kEpiStoreF32, h->sc_post, h->V, rows, h->embed, h->V, d,
                              h->sc_u, d, s));
        }
        K_TRY(launch_gemm(kF32, kEpiStoreF32, h->sc_u, d, rows, h->sc_w1, d, F, h->sc_h1, 2 * F, s));
        K_TRY(launch_gemm(kF32, kEpiStoreF32, h->sc_u, d, rows, h->sc_wu, d, F, h->sc_h1 + F,
                          2 * F, s));
        K_TRY(launch_swiglu_rows(kF32, h->sc_h1, rows, F, h->sc_hf, s));
        K_TRY(launch_gemm(kF32, kEpiStoreF32, (const float*)h->sc_hf, F, rows, h->sc_w2, F, d,
                          h->sc_z, d, s));
    }
    return DG_OK;
}

// sc_out: also form the self-conditioning signal of the next pass (cfg.self_cond).
static int decode_and_head(dg_handle* h, const int32_t* d_canvas, const uint8_t* d_locked_mask,
                           int32_t step, float inv_tau, uint64_t seed, bool ent, hipStream_t s,
                           int B = 1, bool sc_out = false) {
    if (!h->prefilled) return fail(DG_ESTATE, "denoise step before prefill");
    if (h->n_ctx + (int64_t)B * h->C > h->max_ctx)
        return fail(DG_ECAPACITY, "%d canvas(es) at %lld exceed max_ctx %lld", B,
                    (long long)h->n_ctx, (long long)h->max_ctx);
    DG_TRY(ensure_ready(h));
    const int C = B * h->C;        // rows of this pass
    const int period = B > 1 ? h->C : 0;
    h->last_rows = C;
    sc_out = sc_out && h->sc;
    // the first pass of a block takes z = 0, later ones the previous pass's signal
    K_TRY(launch_embed_rmsnorm(h->act, h->act == kBF16, d_canvas, h->embed, h->V, C, h->d,
                               h->cfg.rms_eps, h->x, h->a, h->Af, h->bad, s,
                               h->sc && step > 0 ? h->sc_z : nullptr));
    const uint32_t per_layer = DG_CAP_ROUTING | DG_CAP_HIDDEN | DG_CAP_ATTN | DG_CAP_ROUTER_LOGITS;
    if (h->use_graphs && !h->prof && !(h->cap_mask & per_layer)) {
        DG_TRY(run_layers_graph(h, B, s));
    } else for (int l = 0; l < h->L; ++l) {
        DG_TRY(run_layer(h, l, C, h->n_ctx, false, false, s, true, period));
        if (h->cap(DG_CAP_ROUTING)) {
            HIP_TRY(hipMemcpyAsync(h->cap_idx + (size_t)l * C * h->k, h->idx,
                                   (size_t)C * h->k * 4, hipMemcpyDeviceToDevice, s));
            HIP_TRY(hipMemcpyAsync(h->cap_gates + (size_t)l * C * h->k, h->gates,
                                   (size_t)C * h->k * 4, hipMemcpyDeviceToDevice, s));
        }
        if (h->cap(DG_CAP_HIDDEN))
            HIP_TRY(hipMemcpyAsync(h->cap_hidden + (size_t)l * C * h->d, h->x,
                                   (size_t)C * h->d * 4, hipMemcpyDeviceToDevice, s));
    }
    HeadPartials hp = h->hp;
    hp.q = ent ? h->hp_q : nullptr;
    // self-conditioning: bf16 heads store exp(z - slice max) per logit, the f32 head
    // the tempered logits; the statistics kernel turns them into p0 in place
    const bool f32_post = sc_out && h->act == kF32;
    float* logits_out = f32_post ? (float*)h->sc_post : h->cap(DG_CAP_LOGITS) ? h->logits_cap : nullptr;
    {
        ProfScope p(h, DG_PROF_LM_HEAD, s);
        K_TRY(launch_lm_head(h->act, h->a, h->Af, C, h->d, h->embed, h->V, inv_tau, d_locked_mask,
                             seed, step, h->k_blk, hp, logits_out, s,
                             sc_out && h->act == kBF16 ? (uint16_t*)h->sc_post : nullptr));
    }
    if (f32_post && h->cap(DG_CAP_LOGITS))
        HIP_TRY(hipMemcpyAsync(h->logits_cap, h->sc_post, (size_t)C * h->V * 4,
                               hipMemcpyDeviceToDevice, s));
    PosteriorRows post;
    if (sc_out) {
        post.rows = h->sc_post;
        post.dtype = h->act;
        post.V = h->V;
    }
    K_TRY(launch_head_stats(hp, C, d_locked_mask, h->st_m, h->st_a, h->st_lse, h->st_conf,
                            h->st_draw, ent ? h->st_ent : nullptr, h->bad, s, post));
    if (sc_out) DG_TRY(run_self_cond(h, C, s));
    return DG_OK;
}

int dg_denoise_step(dg_handle* h, int32_t* d_canvas, uint8_t* d_locked_mask, int32_t step,
                    int32_t T, uint64_t seed, void* stream) {
    g_err.clear();
    if (!h || !d_canvas || !d_locked_mask) return fail(DG_EINVAL, "NULL handle, canvas or mask");
    if (T <= 0 || step < 0 || step >= T) return fail(DG_EINVAL, "need 0 <= step < T (step %d, T %d)", step, T);
    hipStream_t s = (hipStream_t)stream;
    DG_TRY(decode_and_head(h, d_canvas, d_locked_mask, step, 1.0f / h->cfg.temperature, seed,
                           false, s, 1, step < T - 1));
    K_TRY(launch_sampler(h->st_conf, h->st_a, h->st_draw, d_canvas, d_locked_mask, h->C, 1, step,
                         T, s));
    return DG_OK;
}

// A batch of canvases is B canvases continuing the same context at the same
// positions: each attends to the context and to itself (not to the others), and
// canvas b draws its Philox uniforms as positions b C .. b C + C - 1 of one long
// canvas, so a batch of one is dg_denoise_step.
static int check_batch(dg_handle* h, int32_t B) {
    if (B < 1 || B > h->B_max) return fail(DG_EINVAL, "batch %d outside [1, %d] (max_batch)", B, h->B_max);
    if (B > 1 && h->act == kBF16 && (h->C % 256 || (h->n_ctx & 31)))
        return fail(DG_EINVAL, "batched bf16 passes need canvas %% 256 == 0 and a context length "
                               "that is a multiple of 32 (n_ctx %lld)", (long long)h->n_ctx);
    return DG_OK;
}

int dg_denoise_step_batch(dg_handle* h, int32_t* d_canvas, uint8_t* d_locked_mask, int32_t B,
                          int32_t step, int32_t T, uint64_t seed, void* stream) {
    g_err.clear();
    if (!h || !d_canvas || !d_locked_mask) return fail(DG_EINVAL, "NULL handle, canvas or mask");
    if (T <= 0 || step < 0 || step >= T) return fail(DG_EINVAL, "need 0 <= step < T (step %d, T %d)", step, T);
    DG_TRY(check_batch(h, B));
    hipStream_t s = (hipStream_t)stream;
    DG_TRY(decode_and_head(h, d_canvas, d_locked_mask, step, 1.0f / h->cfg.temperature, seed,
                           false, s, B, step < T - 1));
    K_TRY(launch_sampler(h->st_conf, h->st_a, h->st_draw, d_canvas, d_locked_mask, h->C, B, step,
                         T, s));
    return DG_OK;
}

static int check_eb_params(const dg_eb_params* p, int32_t step) {
    if (!p) return fail(DG_EINVAL, "NULL sampler parameters");
    if (!(p->tau_max > 0.f) || !(p->tau_min > 0.f) || !std::isfinite(p->tau_max) ||
        !std::isfinite(p->tau_min))
        return fail(DG_EINVAL, "temperatures must be finite and > 0");
    if (std::isnan(p->gamma) || std::isnan(p->theta)) return fail(DG_EINVAL, "NaN threshold");
    if (p->max_steps <= 0) return fail(DG_EINVAL, "max_steps must be > 0");
    if (step < 0 || step >= p->max_steps)
        return fail(DG_EINVAL, "need 0 <= step < max_steps (step %d, max_steps %d)", step,
                    p->max_steps);
    return DG_OK;
}

// tau_s falls linearly from tau_max at pass 0 to tau_min at pass max_steps - 1.
static double eb_tau(const dg_eb_params* p, int32_t step) {
    if (p->max_steps <= 1) return (double)p->tau_min;
    const double t = (double)(p->max_steps - 1 - step) / (double)(p->max_steps - 1);
    return (double)p->tau_min + ((double)p->tau_max - (double)p->tau_min) * t;
}

int dg_eb_sample(const float* d_entropy, const int32_t* d_argmax, const int32_t* d_draw,
                 int32_t* d_prev_argmax, int32_t* d_canvas, uint8_t* d_locked_mask,
                 int32_t* d_info, int32_t C, int32_t V, int32_t step, const dg_eb_params* p,
                 uint64_t seed, int32_t k_blk, void* stream) {
    g_err.clear();
    if (!d_entropy || !d_argmax || !d_draw || !d_prev_argmax || !d_canvas || !d_locked_mask ||
        !d_info)
        return fail(DG_EINVAL, "NULL buffer");
    if (C <= 0 || C > kMaxCanvas) return fail(DG_EINVAL, "need 0 < C <= %d", kMaxCanvas);
    if (V <= 0 || k_blk < 0) return fail(DG_EINVAL, "need V > 0 and k_blk >= 0");
    DG_TRY(check_eb_params(p, step));
    K_TRY(launch_sampler_eb(d_entropy, d_argmax, d_draw, d_prev_argmax, d_canvas, d_locked_mask,
                            d_info, C, V, step, p->max_steps, p->gamma, p->theta, seed, k_blk,
                            (hipStream_t)stream));
    return DG_OK;
}

int dg_denoise_step_eb(dg_handle* h, int32_t* d_canvas, uint8_t* d_locked_mask, int32_t step,
                       const dg_eb_params* p, uint64_t seed, int32_t* d_info, void* stream) {
    g_err.clear();
    if (!h || !d_canvas || !d_locked_mask) return fail(DG_EINVAL, "NULL handle, canvas or mask");
    DG_TRY(check_eb_params(p, step));
    hipStream_t s = (hipStream_t)stream;
    DG_TRY(decode_and_head(h, d_canvas, d_locked_mask, step, (float)(1.0 / eb_tau(p, step)), seed,
                           true, s, 1, step < p->max_steps - 1));
    K_TRY(launch_sampler_eb(h->st_ent, h->st_a, h->st_draw, h->eb_prev, d_canvas, d_locked_mask,
                            d_info ? d_info : h->eb_info, h->C, h->V, step, p->max_steps, p->gamma,
                            p->theta, seed, h->k_blk, s));
    return DG_OK;
}

static int check_bad(dg_handle* h, hipStream_t s) {
    int32_t bad = 0;
    HIP_TRY(hipMemcpyAsync(&bad, h->bad, 4, hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
    if (bad) {
        HIP_TRY(launch_fill_u32(h->bad, 0u, 1, s));
        HIP_TRY(hipStreamSynchronize(s));
        if (bad & kBadToken) return fail(DG_ETOKEN, "a token id outside [0, %d) was embedded", h->V);
        if (bad & kBadNonFinite) return fail(DG_ENONFINITE, "non-finite logits statistics");
        return fail(DG_ENONFINITE, "an expert output or attention split average exceeded the "
                                   "binary16 range (|value| >= 65520) and was saturated");
    }
    return DG_OK;
}

int dg_check_finite(dg_handle* h, void* stream) {
    g_err.clear();
    if (!h) return fail(DG_EINVAL, "NULL handle");
    return check_bad(h, (hipStream_t)stream);
}

int dg_init_canvas(dg_handle* h, int32_t* d_canvas, uint8_t* d_locked_mask, uint64_t seed,
                   void* stream) {
    g_err.clear();
    if (!h) return fail(DG_EINVAL, "NULL handle");
    if (!d_canvas && !d_locked_mask) return DG_OK;
    hipStream_t s = (hipStream_t)stream;
    K_TRY(launch_canvas_init(d_canvas, d_locked_mask, h->C, h->V, seed, h->k_blk, s));
    return DG_OK;
}

int dg_init_canvas_batch(dg_handle* h, int32_t* d_canvas, uint8_t* d_locked_mask, int32_t B,
                         uint64_t seed, void* stream) {
    g_err.clear();
    if (!h) return fail(DG_EINVAL, "NULL handle");
    if (B < 1 || B > h->B_max) return fail(DG_EINVAL, "batch %d outside [1, %d]", B, h->B_max);
    if (!d_canvas && !d_locked_mask) return DG_OK;
    K_TRY(launch_canvas_init(d_canvas, d_locked_mask, B * h->C, h->V, seed, h->k_blk,
                             (hipStream_t)stream));
    return DG_OK;
}

int dg_generate_block_batch(dg_handle* h, int32_t* d_out_tokens, int32_t B, int32_t T,
                            uint64_t seed, void* stream) {
    g_err.clear();
    if (!h || !d_out_tokens) return fail(DG_EINVAL, "NULL handle or output");
    if (T <= 0) return fail(DG_EINVAL, "T must be > 0");
    if (!h->prefilled) return fail(DG_ESTATE, "generate before prefill");
    DG_TRY(check_batch(h, B));
    if (h->n_ctx + (int64_t)B * h->C > h->max_ctx)
        return fail(DG_ECAPACITY, "%d canvases at %lld exceed max_ctx %lld", B,
                    (long long)h->n_ctx, (long long)h->max_ctx);
    DG_TRY(ensure_ready(h));
    hipStream_t s = (hipStream_t)stream;
    K_TRY(launch_canvas_init(h->blk_canvas, h->blk_mask, B * h->C, h->V, seed, h->k_blk, s));
    for (int st = 0; st < T; ++st)
        DG_TRY(dg_denoise_step_batch(h, h->blk_canvas, h->blk_mask, B, st, T, seed, stream));
    HIP_TRY(hipMemcpyAsync(d_out_tokens, h->blk_canvas, (size_t)B * h->C * 4,
                           hipMemcpyDeviceToDevice, s));
    return check_bad(h, s);
}

int dg_generate_block(dg_handle* h, int32_t* d_out_tokens, int32_t T, uint64_t seed,
                      int32_t commit, void* stream) {
    g_err.clear();
    if (!h || !d_out_tokens) return fail(DG_EINVAL, "NULL handle or output");
    if (T <= 0) return fail(DG_EINVAL, "T must be > 0");
    if (!h->prefilled) return fail(DG_ESTATE, "generate before prefill");
    if (h->n_ctx + h->C > h->max_ctx)
        return fail(DG_ECAPACITY, "canvas at %lld exceeds max_ctx %lld", (long long)h->n_ctx,
                    (long long)h->max_ctx);
    DG_TRY(ensure_ready(h));
    hipStream_t s = (hipStream_t)stream;
    K_TRY(launch_canvas_init(h->blk_canvas, h->blk_mask, h->C, h->V, seed, h->k_blk, s));
    for (int st = 0; st < T; ++st)
        DG_TRY(dg_denoise_step(h, h->blk_canvas, h->blk_mask, st, T, seed, stream));
    HIP_TRY(hipMemcpyAsync(d_out_tokens, h->blk_canvas, (size_t)h->C * 4,
                           hipMemcpyDeviceToDevice, s));
    if (commit) DG_TRY(dg_commit_canvas(h, h->blk_canvas, stream));
    return check_bad(h, s);
}

int dg_generate_block_eb(dg_handle* h, int32_t* d_out_tokens, const dg_eb_params* p,
                         uint64_t seed, int32_t commit, int32_t* n_steps, void* stream) {
    g_err.clear();
    if (!h || !d_out_tokens) return fail(DG_EINVAL, "NULL handle or output");
    DG_TRY(check_eb_params(p, 0));
    if (!h->prefilled) return fail(DG_ESTATE, "generate before prefill");
    if (h->n_ctx + h->C > h->max_ctx)
        return fail(DG_ECAPACITY, "canvas at %lld exceeds max_ctx %lld", (long long)h->n_ctx,
                    (long long)h->max_ctx);
    DG_TRY(ensure_ready(h));
    hipStream_t s = (hipStream_t)stream;
    K_TRY(launch_canvas_init(h->blk_canvas, h->blk_mask, h->C, h->V, seed, h->k_blk, s));
    int32_t info[4] = {0, 0, 0, 0};
    int st = 0;
    while (st < p->max_steps) {
        DG_TRY(dg_denoise_step_eb(h, h->blk_canvas, h->blk_mask, st, p, seed, h->eb_info, stream));
        ++st;
        HIP_TRY(hipMemcpyAsync(info, h->eb_info, sizeof(info), hipMemcpyDeviceToHost, s));
        HIP_TRY(hipStreamSynchronize(s));
        if (info[0]) break;
    }
    if (n_steps) *n_steps = st;
    HIP_TRY(hipMemcpyAsync(d_out_tokens, h->blk_canvas, (size_t)h->C * 4,
                           hipMemcpyDeviceToDevice, s));
    if (commit) DG_TRY(dg_commit_canvas(h, h->blk_canvas, stream));
    return check_bad(h, s);
}

int dg_get_capture(dg_handle* h, uint32_t what, int32_t layer, void* d_dst, size_t bytes,
                   void* stream) {
    g_err.clear();
    if (!h || !d_dst) return fail(DG_EINVAL, "NULL handle or destination");
    hipStream_t s = (hipStream_t)stream;
    const size_t C = h->last_rows > 0 ? h->last_rows : h->C;   // rows of the last pass
    if (what == DG_CAP_STATS) {
        if (bytes != C * 4 * 5) return fail(DG_EINVAL, "stats capture is %zu bytes", C * 20);
        char* d = (char*)d_dst;
        HIP_TRY(hipMemcpyAsync(d, h->st_m, C * 4, hipMemcpyDeviceToDevice, s));
        HIP_TRY(hipMemcpyAsync(d + C * 4, h->st_a, C * 4, hipMemcpyDeviceToDevice, s));
        HIP_TRY(hipMemcpyAsync(d + C * 8, h->st_lse, C * 4, hipMemcpyDeviceToDevice, s));
        HIP_TRY(hipMemcpyAsync(d + C * 12, h->st_conf, C * 4, hipMemcpyDeviceToDevice, s));
        HIP_TRY(hipMemcpyAsync(d + C * 16, h->st_draw, C * 4, hipMemcpyDeviceToDevice, s));
        return DG_OK;
    }
    if (what == DG_CAP_ENTROPY) {
        if (bytes != C * 4) return fail(DG_EINVAL, "entropy capture is %zu bytes", C * 4);
        HIP_TRY(hipMemcpyAsync(d_dst, h->st_ent, C * 4, hipMemcpyDeviceToDevice, s));
        return DG_OK;
    }
    if (what == DG_CAP_SELFCOND) {
        if (!h->sc) return fail(DG_ESTATE, "self-conditioning is off");
        if (layer != 0 && layer != 1) return fail(DG_EINVAL, "layer 0 (u) or 1 (z)");
        if (bytes != C * h->d * 4) return fail(DG_EINVAL, "self-conditioning capture is %zu bytes", C * h->d * 4);
        HIP_TRY(hipMemcpyAsync(d_dst, layer == 0 ? h->sc_u : h->sc_z, bytes, hipMemcpyDeviceToDevice, s));
        return DG_OK;
    }
    if (what == DG_CAP_LOGITS) {
        if (!h->logits_cap) return fail(DG_ESTATE, "logits capture not enabled");
        if (bytes != C * h->V * 4) return fail(DG_EINVAL, "logits capture is %zu bytes", C * h->V * 4);
        HIP_TRY(hipMemcpyAsync(d_dst, h->logits_cap, bytes, hipMemcpyDeviceToDevice, s));
        return DG_OK;
    }
    if (layer < 0 || layer >= h->L) return fail(DG_EINVAL, "bad layer %d", layer);
    if (what == DG_CAP_ROUTING) {
        if (!h->cap_idx) return fail(DG_ESTATE, "routing capture not enabled");
        const size_t n = C * h->k * 4;
        if (bytes != 2 * n) return fail(DG_EINVAL, "routing capture is %zu bytes", 2 * n);
        HIP_TRY(hipMemcpyAsync(d_dst, h->cap_idx + (size_t)layer * C * h->k, n,
                               hipMemcpyDeviceToDevice, s));
        HIP_TRY(hipMemcpyAsync((char*)d_dst + n, h->cap_gates + (size_t)layer * C * h->k, n,
                               hipMemcpyDeviceToDevice, s));
        return DG_OK;
    }
    if (what == DG_CAP_ATTN) {
        if (!h->cap_attn) return fail(DG_ESTATE, "attention capture not enabled");
        const size_t n = C * h->Hq * h->D * dsize(h->act);
        if (bytes != n) return fail(DG_EINVAL, "attention capture is %zu bytes", n);
        HIP_TRY(hipMemcpyAsync(d_dst, (char*)h->cap_attn + (size_t)layer * n, n,
                               hipMemcpyDeviceToDevice, s));
        return DG_OK;
    }
    if (what == DG_CAP_ROUTER_LOGITS) {
        if (!h->cap_rlog) return fail(DG_ESTATE, "router logits capture not enabled");
        const size_t n = C * h->E * 4;
        if (bytes != n) return fail(DG_EINVAL, "router logits capture is %zu bytes", n);
        HIP_TRY(hipMemcpyAsync(d_dst, h->cap_rlog + (size_t)layer * C * h->E, n,
                               hipMemcpyDeviceToDevice, s));
        return DG_OK;
    }
    if (what == DG_CAP_HIDDEN) {
        if (!h->cap_hidden) return fail(DG_ESTATE, "hidden capture not enabled");
        const size_t n = C * h->d * 4;
        if (bytes != n) return fail(DG_EINVAL, "hidden capture is %zu bytes", n);
        HIP_TRY(hipMemcpyAsync(d_dst, h->cap_hidden + (size_t)layer * C * h->d, n,
                               hipMemcpyDeviceToDevice, s));
        return DG_OK;
    }
    return fail(DG_EINVAL, "unknown capture %u", what);
}

int dg_get_kv(dg_handle* h, int32_t layer, int32_t which, int64_t row0, int64_t n, void* d_dst,
              void* stream) {
    g_err.clear();
    if (!h || !d_dst) return fail(DG_EINVAL, "NULL handle or destination");
    if (layer < 0 || layer >= h->L || (which != 0 && which != 1)) return fail(DG_EINVAL, "bad layer or which");
    if (row0 < 0 || n < 0 || row0 + n > h->kv_rows) return fail(DG_EINVAL, "rows out of range");
    const bool vp = which == 1 && h->act == kBF16;
    HIP_TRY(launch_read_kv(h->act, vp, which ? h->vlayer(layer) : h->klayer(layer), h->Hkv, h->D,
                           h->kv_rows, row0, n, d_dst, (hipStream_t)stream));
    return DG_OK;
}

int dg_set_kv(dg_handle* h, int32_t layer, int32_t which, int64_t row0, int64_t n,
              const void* d_src, void* stream) {
    g_err.clear();
    if (!h || !d_src) return fail(DG_EINVAL, "NULL handle or source");
    if (layer < 0 || layer >= h->L || (which != 0 && which != 1)) return fail(DG_EINVAL, "bad layer or which");
    if (row0 < 0 || n < 0 || row0 + n > h->max_ctx) return fail(DG_EINVAL, "rows out of range");
    const bool vp = which == 1 && h->act == kBF16;
    HIP_TRY(launch_write_kv(h->act, vp, which ? h->vlayer(layer) : h->klayer(layer), h->Hkv, h->D,
                            h->kv_rows, row0, n, d_src, (hipStream_t)stream));
    return DG_OK;
}

// ---------------------------------------------------------------- kernel-level entry points
namespace {
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Rows of the transposed V copy a bf16 attention call packs (a multiple of 32).
int64_t attn_vt_rows(int32_t S) { return ((int64_t)S + 31) & ~(int64_t)31; }

int check_attention_args(int32_t Hq, int32_t Hkv, int32_t M, int32_t S, int32_t D,
                         int32_t causal, int32_t q_pos0, int32_t dtype) {
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || M <= 0 || S <= 0 || D <= 0 || q_pos0 < 0)
        return fail(DG_EINVAL, "bad attention sizes");
    if (dtype != DG_F32 && dtype != DG_BF16) return fail(DG_EINVAL, "dtype must be DG_F32 or DG_BF16");
    if (dtype == DG_F32 && D != 64 && D != 128) return fail(DG_EINVAL, "f32 needs D 64 or 128");
    if (dtype == DG_BF16 && D != 128) return fail(DG_EINVAL, "bf16 needs D 128");
    if (causal && (int64_t)q_pos0 + M > S) return fail(DG_EINVAL, "causal queries beyond the keys");
    return DG_OK;
}

// Workspace of a bf16 call: the transposed, key-permuted copy of V, then the split
// partials.  f32 calls need none.
size_t attention_ws_bytes(int32_t Hq, int32_t Hkv, int32_t M, int32_t S, int32_t D, int32_t dtype) {
    if (dtype != DG_BF16) return 0;
    return align256((size_t)Hkv * D * attn_vt_rows(S) * 2) +
           attention_part_bytes(kBF16, Hq, Hkv, M, S, D);
}

// The attention call on a workspace of ws_bytes at d_ws (sizes already checked).
int run_attention(const void* d_q, const void* d_k, const void* d_v, void* d_o, int32_t Hq,
                  int32_t Hkv, int32_t M, int32_t S, int32_t D, float scale, int32_t causal,
                  int32_t q_pos0, int32_t dtype, void* d_ws, size_t ws_bytes, hipStream_t s) {
    AttnArgs aa;
    aa.q = d_q;
    aa.k = d_k;
    aa.v = d_v;
    aa.o = d_o;
    aa.Hq = Hq;
    aa.Hkv = Hkv;
    aa.M = M;
    aa.S = S;
    aa.D = D;
    aa.kv_rows = S;
    aa.v_rows = S;
    aa.scale = scale;
    aa.causal = causal;
    aa.q_pos0 = q_pos0;
    const int dt = dtype == DG_F32 ? kF32 : kBF16;
    if (dt == kBF16) {
        const int64_t rows = attn_vt_rows(S);
        const size_t vb = align256((size_t)Hkv * D * rows * 2);
        HIP_TRY(launch_pack_vt(d_v, Hkv, S, D, d_ws, rows, s));
        aa.v = d_ws;
        aa.v_rows = rows;
        aa.part = (char*)d_ws + vb;
        aa.part_bytes = ws_bytes - vb;
    }
    HIP_TRY(launch_attention(dt, aa, s));
    return DG_OK;
}
}  // namespace

int dg_attention_workspace_size(int32_t Hq, int32_t Hkv, int32_t M, int32_t S, int32_t D,
                                int32_t causal, int32_t q_pos0, int32_t dtype, size_t* bytes) {
    g_err.clear();
    if (!bytes) return fail(DG_EINVAL, "NULL bytes");
    DG_TRY(check_attention_args(Hq, Hkv, M, S, D, causal, q_pos0, dtype));
    *bytes = attention_ws_bytes(Hq, Hkv, M, S, D, dtype);
    return DG_OK;
}

int dg_attention(const void* d_q, const void* d_k, const void* d_v, void* d_o, int32_t Hq,
                 int32_t Hkv, int32_t M, int32_t S, int32_t D, float scale, int32_t causal,
                 int32_t q_pos0, int32_t dtype, void* d_workspace, size_t workspace_bytes,
                 void* stream) {
    g_err.clear();
    if (!d_q || !d_k || !d_v || !d_o) return fail(DG_EINVAL, "NULL tensor");
    DG_TRY(check_attention_args(Hq, Hkv, M, S, D, causal, q_pos0, dtype));
    const size_t need = attention_ws_bytes(Hq, Hkv, M, S, D, dtype);
    if (need > 0 && (!d_workspace || workspace_bytes < need))
        return fail(DG_EINVAL, "attention workspace of %zu bytes needed, %zu given", need,
                    d_workspace ? workspace_bytes : (size_t)0);
    return run_attention(d_q, d_k, d_v, d_o, Hq, Hkv, M, S, D, scale, causal, q_pos0, dtype,
                         d_workspace, workspace_bytes, (hipStream_t)stream);
}

// Scratch of dg_attention_noalloc: a file-scope device array, one copy per GPU the
// library runs on, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (resolved on the first call there).
int scratch_address(void** out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(DG_EINVAL, "device %d beyond the scratch table", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(DG_EHIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return DG_OK;
}
}  // namespace

int dg_attention_noalloc(const void* d_q, const void* d_k, const void* d_v, void* d_o, int32_t Hq,
                         int32_t Hkv, int32_t M, int32_t S, int32_t D, float scale,
                         int32_t causal, int32_t q_pos0, int32_t dtype, void* stream) {
    g_err.clear();
    if (!d_q || !d_k || !d_v || !d_o) return fail(DG_EINVAL, "NULL tensor");
    DG_TRY(check_attention_args(Hq, Hkv, M, S, D, causal, q_pos0, dtype));
    const size_t need = attention_ws_bytes(Hq, Hkv, M, S, D, dtype);
    if (need > kNoAllocScratchBytes)
        return fail(DG_EINVAL, "attention needs %zu bytes of scratch, the static scratch holds %zu",
                    need, kNoAllocScratchBytes);
    void* ws = nullptr;
    if (need > 0) DG_TRY(scratch_address(&ws));
    return run_attention(d_q, d_k, d_v, d_o, Hq, Hkv, M, S, D, scale, causal, q_pos0, dtype, ws,
                         kNoAllocScratchBytes, (hipStream_t)stream);
}

int dg_moe_layer(dg_handle* h, int32_t layer, const void* d_x, int32_t n_tokens, void* d_y,
                 int32_t* d_idx, float* d_gates, void* stream) {
    g_err.clear();
    if (!h || !d_x || !d_y) return fail(DG_EINVAL, "NULL handle or tensor");
    if (layer < 0 || layer >= h->L) return fail(DG_EINVAL, "bad layer %d", layer);
    if (n_tokens <= 0 || n_tokens > h->max_tokens)
        return fail(DG_EINVAL, "n_tokens must be in [1, %d]", h->max_tokens);
    for (int kind = 0; kind < 3; ++kind)
        for (int e = 0; e < h->E; ++e)
            if (!h->expert_flag(layer, kind, e)) return fail(DG_ESTATE, "experts of layer %d not loaded", layer);
    if (!h->dense_flag(layer, DG_T_WR - DG_T_WQ)) return fail(DG_ESTATE, "router of layer %d not loaded", layer);
    hipStream_t s = (hipStream_t)stream;
    const uint8_t* x8 = nullptr;
    if (e4m3_inputs(h)) {
        K_TRY(launch_cast_e4m3(d_x, (int64_t)n_tokens * h->d, h->a8, s));
        x8 = h->a8;
    }
    DG_TRY(run_moe(h, layer, n_tokens, d_x, x8, s));
    K_TRY(launch_moe_combine(h->act, 1, h->Y, n_tokens, h->d, h->k, h->gates, h->inv, nullptr,
                             0.f, nullptr, nullptr, nullptr, d_y, s));
    if (d_idx) HIP_TRY(hipMemcpyAsync(d_idx, h->idx, (size_t)n_tokens * h->k * 4, hipMemcpyDeviceToDevice, s));
    if (d_gates) HIP_TRY(hipMemcpyAsync(d_gates, h->gates, (size_t)n_tokens * h->k * 4, hipMemcpyDeviceToDevice, s));
    return DG_OK;
}

}  // extern "C"
