// Kernel launchers of the gfx950 canvas-denoising library (internal interface).
#pragma once

#include "common.h"

namespace dg {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kFP8 = 2;
constexpr int kMX = 3;    // MX FP4 expert weights (E2M1 + E8M0 per 32 along K), e4m3 inputs

constexpr int kPermChunk = 1024;   // entries per permutation workgroup
constexpr int kMaxCanvas = 1024;   // sampler capacity (one workgroup)
// Bits of the handle's sticky error word.
constexpr int32_t kBadNonFinite = 1;   // a row's logits statistics were not finite
constexpr int32_t kBadToken = 2;       // a token id outside [0, V) was embedded
constexpr int32_t kBadRange = 4;       // an expert output or attention split average saturated
                                       // at the binary16 range (|value| >= 65520)
constexpr int kMaxTopK = 16;       // experts per token
constexpr int kCombineCols = 16;   // combine: columns per thread, d <= 256 * 16
constexpr int kMoeRows = 256;      // rows one expert-GEMM workgroup covers (a whole canvas)
#ifndef DG_MOE_ITEM_ROWS
#define DG_MOE_ITEM_ROWS 128
#endif
// Rows of one work item of the first expert GEMM.  Below kMoeRows an expert with
// many rows is split over several workgroups (its weights are read once per
// item), which shortens the longest unit; the second GEMM (K = d_ff, short
// units) keeps whole-canvas items.
constexpr int kMoeItemRows = DG_MOE_ITEM_ROWS;
static_assert(kMoeItemRows % 16 == 0 && kMoeItemRows <= kMoeRows, "work item rows");
constexpr int kMaxRouterSplit = 8; // K split of the router GEMM (partials summed in top-k)
constexpr int kMoePad = 16;        // expert row padding of the MFMA expert GEMMs (one row tile)

// Permuted-row capacity for n tokens, k experts each, E experts, rows padded to pad.
inline int64_t moe_rows_cap(int64_t n, int k, int E, int pad) { return n * k + (int64_t)E * (pad - 1); }

// Expert-GEMM work lists built by the permutation: item i of `items` covers rows
// [row0, row0 + kMoeItemRows) of expert e (clipped to the expert's count), item i
// of `items2` rows [row0, row0 + kMoeRows).
struct MoeWork {
    int4* items;       // {e, row0, first row of e, end of e's padded rows}, first GEMM
    int4* items2;      // the same for the second GEMM
    int32_t* count;    // [0] number of valid items; [1], [2] unit counters of the two
                       // persistent expert GEMMs (zeroed by the kernel that writes [0]);
                       // [3] number of valid items2
    int max_items;     // grid bound: ceil(entries / kMoeItemRows) + E
    int max_items2;    // grid bound: ceil(entries / kMoeRows) + E
};

// Byte offset of element (row, col) of a [rows][K] matrix stored in MFMA
// A-operand fragment order: [row / 16][k-step][lane = 16 g + row % 16][16 bytes].
// bf16: k-step of 32 columns, lane group g = (col % 32) / 8, element col % 8.
// e4m3: k-step of 64 columns, the lane's 16 bytes hold columns 8 g..8 g+7 (low
// half) and 32 + 8 g..32 + 8 g + 7 (high half) of the k-step.  A 16-row x k-step
// fragment set is one contiguous 1 KiB, so an MFMA operand load is one
// coalesced 16-byte load per lane.
template <bool FP8>
DG_DEV size_t frag_offset(int64_t row, int col, int K) {
    const int KB = FP8 ? (K >> 6) : (K >> 5);
    const int kb = FP8 ? (col >> 6) : (col >> 5);
    const int g = (col & 31) >> 3;
    const int byte = FP8 ? (8 * ((col >> 5) & 1) + (col & 7)) : 2 * (col & 7);
    return ((size_t)((row >> 4) * KB + kb) * 64 + 16 * g + (row & 15)) * 16 + byte;
}

// Byte offset of element (row, col) of an e4m3 [rows][K] matrix (K a multiple of 128)
// in the A-operand order of the block-scaled 16x16x128 MFMA: [row / 16][k-step of
// 128][lane = 16 g + row % 16][32 bytes]; the lane's byte j holds column
// 16 g + 64 (j / 16) + j % 16 of the k-step (two runs of 16 consecutive columns).
DG_DEV size_t frag_offset_mx(int64_t row, int col, int K) {
    const int KS = K >> 7, ks = col >> 7, kk = col & 127;
    const int g = (kk & 63) >> 4, j = 16 * (kk >> 6) + (kk & 15);
    return ((size_t)((row >> 4) * KS + ks) * 64 + 16 * g + (row & 15)) * 32 + j;
}

// Transposed, key-permuted V cache: Vt[h][dim][slot], rows padded to a multiple
// of 32.  Within each 32-key block, key 16*hi + 4*g + j sits at slot 8*g + 4*hi + j,
// so one 16-byte load gives a lane exactly the 8 keys its MFMA operand needs.
DG_DEV size_t vt_index(int64_t h, int64_t dim, int64_t pos, int64_t D, int64_t rows) {
    const int64_t r = pos & 31;
    const int64_t slot = (pos & ~(int64_t)31) + 8 * ((r & 15) >> 2) + 4 * (r >> 4) + (r & 3);
    return (size_t)((h * D + dim) * rows + slot);
}

// Vocabulary ids of one partial slice of the bf16 LM head (one 128-column weight slab).
constexpr int kHeadSlice = 128;

// Per (row, vocabulary slice) partial statistics of the LM head, [C][n_slices] each.
struct HeadPartials {
    float* m;       // max tempered logit
    int32_t* a;     // lowest id attaining it
    float* s;       // sum exp(z - m)
    float* g;       // best Gumbel-perturbed score (-inf for locked rows)
    int32_t* gi;    // its id
    float* q;       // sum exp(z - m) (z - m), for the predictive entropy; nullptr: not kept
    int n_slices;
};

// ---------------------------------------------------------------- misc
// The row-normalising kernels also write the bf16 rows in fragment order to af
// (frag_offset, K = d) when af is given (bf16 only).
// zadd (optional, float [C][d]): the self-conditioning signal added to the embedding.
hipError_t launch_embed_rmsnorm(int dtype, bool packed, const int32_t* tokens, const void* E,
                                int V, int C, int d, float eps, float* x, void* a, void* af,
                                int32_t* bad, hipStream_t s, const float* zadd = nullptr);
hipError_t launch_rmsnorm(int dtype, const float* x, int M, int d, float eps, void* a,
                          uint8_t* a8, void* af, hipStream_t s);
// Token m sits at RoPE position pos0 + m (period 0) or pos0 + m % period, and in
// cache row pos0 + m.
hipError_t launch_rope_scatter(int dtype, const float* qkv, int M, int Hq, int Hkv, int D,
                               int64_t pos0, int period, const float* cos_t, const float* sin_t,
                               void* q, void* kc, void* vc, int64_t kv_rows, hipStream_t s);
hipError_t launch_pack_vt(const void* v, int Hkv, int S, int D, void* vt, int64_t rows,
                          hipStream_t s);
hipError_t launch_read_kv(int dtype, bool vpacked, const void* cache, int Hkv, int D,
                          int64_t rows, int64_t row0, int64_t n, void* dst, hipStream_t s);
hipError_t launch_write_kv(int dtype, bool vpacked, void* cache, int Hkv, int D, int64_t rows,
                           int64_t row0, int64_t n, const void* src, hipStream_t s);
// logits: nsplit partial sums [nsplit][M][E], added in order.  Each expert's
// rows start at a multiple of pad (kMoePad for the MFMA expert GEMMs, 1 for
// f32); padding rows have perm_token = -1.  perm_token holds moe_rows_cap rows.
hipError_t launch_router_permute(const float* logits, int nsplit, int M, int E, int k, int32_t* idx,
                                 float* gates, int32_t* counts, int32_t* base, int32_t* offsets,
                                 int32_t* perm_token, int32_t* inv, const MoeWork& work, int pad,
                                 hipStream_t s);
hipError_t launch_moe_combine(int dtype, int mode, const void* Y, int M, int d, int k,
                              const float* gates, const int32_t* inv, float* x, float eps,
                              void* a, uint8_t* a8, void* af, void* out, hipStream_t s);
hipError_t launch_canvas_init(int32_t* canvas, uint8_t* mask, int C, int V, uint64_t seed,
                              int k_blk, hipStream_t s);
// st_ent (entropy per row) is written when p.q is kept, and must be given exactly then.
// post (optional, rows [C][V]): turned in place into the posterior p0 of each row once
// its log-sum-exp is known: bf16 rows hold exp(z - m) of their 128-id slice (the head
// epilogue's sc output), f32 rows the tempered logits z.
struct PosteriorRows {
    void* rows = nullptr;
    int dtype = 0;     // kBF16: exp(z - slice max), kF32: z
    int V = 0;
};
hipError_t launch_head_stats(const HeadPartials& p, int C, const uint8_t* mask, float* st_m,
                             int32_t* st_a, float* st_lse, float* st_conf, int32_t* st_draw,
                             float* st_ent, int32_t* bad, hipStream_t s,
                             const PosteriorRows& post = PosteriorRows{});
// H[r][f] = silu(h1[r][f]) * h1[r][F + f] (h1 float [M][2F]); bf16: H in MFMA fragment
// order (frag_offset, K = F, rows padded to 16); f32: H natural float [M][F].
hipError_t launch_swiglu_rows(int dtype, const float* h1, int M, int F, void* H, hipStream_t s);
// B canvases of C positions each, one workgroup per canvas.
hipError_t launch_sampler(const float* conf, const int32_t* amax, const int32_t* draw,
                          int32_t* canvas, uint8_t* mask, int C, int B, int step, int T,
                          hipStream_t s);
// One pass of the entropy-bounded sampler (k_sampler_eb); C <= kMaxCanvas.
hipError_t launch_sampler_eb(const float* ent, const int32_t* amax, const int32_t* draw,
                             int32_t* prev, int32_t* canvas, uint8_t* mask, int32_t* info, int C,
                             int V, int step, int max_steps, float gamma, float theta,
                             uint64_t seed, int k_blk, hipStream_t s);
// rope_hd > 0 (128): the 16-column groups of every rope_hd-column head are
// reordered so that each 64-column tile holds 32 rotary pairs (dims j and
// j + 64 for j in one 32-dim quarter), see kEpiRope.
hipError_t launch_pack_b16(const void* src, bool src_kn, int K, int N, int gstride, int goff,
                           void* dst, hipStream_t s, int rope_hd = 0);
hipError_t launch_pack_b8(const void* src, int K, int N, int gstride, int goff, void* dst,
                          hipStream_t s);
hipError_t launch_scatter_scales(const float* src, int N, int gstride, int goff, float* dst,
                                 hipStream_t s);
hipError_t launch_fill_u32(void* p, uint32_t v, int64_t n, hipStream_t s);
hipError_t launch_cast_e4m3(const void* x_bf16, int64_t n, uint8_t* out, hipStream_t s);

// ---------------------------------------------------------------- GEMMs
// Epilogue modes of the dense GEMM.
constexpr int kEpiStoreF32 = 0;   // C[m, n] = acc
constexpr int kEpiAddF32 = 1;     // C[m, n] += acc (residual add, single writer)
constexpr int kEpiRope = 2;       // QKV with pair-tiled columns: RoPE, bf16 Q, K and V cache writes

// The QKV epilogue's destinations (head dim 128): Q bf16 [Hq][M][128], the K
// cache bf16 [Hkv][kv_rows][128] and the V cache transposed (vt_index), rows
// pos0 + m; cos/sin tables [position][64].
struct RopeArgs {
    int Hq = 0, Hkv = 0;
    int64_t pos0 = 0;
    int period = 0;        // > 0: token m at RoPE position pos0 + m % period (cache row pos0 + m)
    const float* cos_t = nullptr;
    const float* sin_t = nullptr;
    void* q = nullptr;
    void* kc = nullptr;
    void* vc = nullptr;
    int64_t kv_rows = 0;
};

// C = A[M, K] B[K, N].  bf16: A row-major (lda), B packed (see packed_b_index).
// f32: A row-major, B row-major [K, N].  bf16 with ksplit > 1 (store epilogue
// only): partial sums over ksplit K ranges at C + z * M * ldc, z < ksplit.
hipError_t launch_gemm(int dtype, int epi, const void* A, int lda, int M, const void* B, int K,
                       int N, float* C, int ldc, hipStream_t s, int ksplit = 1);
// The same product (bf16) with A in MFMA A-fragment order ([row/16][K/32][64][16 B],
// rows padded to 16), as written by the kernel that produces A.
// epi = kEpiRope: B packed with rope_hd = 128, N = (Hq + 2 Hkv) * 128, C unused.
hipError_t launch_gemm_frag(int epi, const void* Af, int M, const void* B, int K, int N, float* C,
                            int ldc, hipStream_t s, int ksplit = 1,
                            const RopeArgs* rope = nullptr);

// Expert GEMMs over the permuted entries (offsets[e]..offsets[e+1] belong to expert e).
// GEMM 1: H[entry, :F] = silu(x Wg_e) * (x Wu_e), x = X[perm_token[entry]].
//   bf16: X bf16 [*, d] natural token rows, read in place through perm_token;
//         W1 packed with interleaved gate/up groups; H bf16.
//   fp8 : Xf e4m3 in MFMA A-operand fragment order (launch_moe_gather8:
//         [row / 16][k-step][lane][16 bytes], padding rows zero); W1 packed
//         e4m3 + column scales (2F); H e4m3.
//   f32 : X f32, Wg/Wu row-major [E][d][F], H f32.
//   bf16/fp8 write H in fragment order for GEMM 2; rows padded to kMoePad,
//   max_rows = moe_rows_cap.
// GEMM 2: Y[entry, :d] = H[entry] Wd_e (binary16 rows, f32 for f32 experts).
struct ExpertWeights {
    const void* w1;        // bf16/fp8/MX packed gate|up, or f32 Wg
    const void* wu;        // f32 Wu (f32 path only)
    const void* w2;        // down projection (packed or row-major)
    const float* s1;       // fp8 column scales of w1 [E][2F] (interleaved)
    const float* s2;       // fp8 column scales of w2 [E][d]
    const uint8_t* x1 = nullptr;   // MX: E8M0 block scales of w1 in stage order (mx_scale_bytes)
    const uint8_t* x2 = nullptr;   // MX: the same for w2
};

// MX FP4 expert weights.  Codes of a [K][N] matrix (K padded to Kp, a multiple of 128)
// as B-operand fragments of the block-scaled 16x16x128 MFMA: [N/16 groups][Kp/128
// k-steps][64 lanes][16 bytes], lane l of group G holding column 16 G + l % 16 at rows
// 128 ks + 32 (l / 16) + 0..31, two per byte (even row in the low nibble): the same
// 1 KiB chunk per (group, k-step) as the bf16 and e4m3 weights.  The E8M0 scales in the
// order the expert GEMM reads them, one 16-byte load per lane per stage of two
// k-steps: [N/128 slabs][ceil(Kp/256) stages][64 lanes][2 k-steps][8 groups], the byte
// of (k-step ks, group i) being the scale of rows 32 (4 ks + l / 16) .. + 31 of column
// 16 (8 slab + i) + l % 16 (127 past K).  gstride / goff place source group g at
// destination group g * gstride + goff (gate and up interleaved per 16 columns).
inline size_t mx_code_bytes(int K, int N) { return (size_t)N / 16 * ((K + 127) / 128) * 1024; }
inline size_t mx_scale_bytes(int K, int N) {
    return (size_t)((N + 127) / 128) * (((K + 127) / 128 + 1) / 2) * 1024;
}
hipError_t launch_pack_mx(const uint8_t* codes, const uint8_t* scales, int K, int N, int gstride,
                          int goff, int n_dst_groups, void* dst_codes, uint8_t* dst_scales,
                          hipStream_t s);
// fp8 GEMM 1's activation fragments: Xf = X[perm_token] (e4m3) in MFMA A-operand
// order, padding rows zero.
// mx: the MX FP4 experts' activation order (frag_offset_mx) instead.
hipError_t launch_moe_gather8(const void* X, int d, const int32_t* perm_token,
                              const int32_t* offsets, int E, int max_rows, void* Xf, hipStream_t s,
                              bool mx = false);
hipError_t launch_moe_gemm1(int dtype, const ExpertWeights& w, const void* X,
                            const int32_t* perm_token, const int32_t* offsets, int E, int d,
                            int F, int max_rows, const MoeWork& work, void* Xf, void* H,
                            hipStream_t s);
// bad (optional): kBadRange is set when a binary16 output saturates.
hipError_t launch_moe_gemm2(int dtype, const ExpertWeights& w, const void* H,
                            const int32_t* offsets, int E, int d, int F, int max_rows,
                            const MoeWork& work, float* Y, int32_t* bad, hipStream_t s);

// LM head: per (row, slice) partial max / argmax / sum-exp / Gumbel best of
// z = (h E^T) / tau over the vocabulary.  Gumbel noise for rows with mask == 0.
// bf16: hf, when given, holds the same rows in MFMA fragment order (frag_offset,
// K = d) and the head runs on the streamed-weight pipeline of the expert GEMMs.
// sc_w (optional, bf16 [C][V]): exp(z - m) of every logit, m the max of its 128-id
// slice (the unnormalised posterior rows that launch_head_stats rescales).
hipError_t launch_lm_head(int dtype, const void* h, const void* hf, int C, int d, const void* E,
                          int V, float inv_tau, const uint8_t* mask, uint64_t seed, int step,
                          int k_blk, const HeadPartials& p, float* logits_out, hipStream_t s,
                          uint16_t* sc_w = nullptr);
hipError_t launch_head_wide(const void* hf, int C, int d, const void* E, int V, float inv_tau,
                            const uint8_t* mask, uint32_t key0, uint32_t key1, uint32_t c2,
                            const HeadPartials& p, float* logits_out, hipStream_t s,
                            uint16_t* sc_w = nullptr);
int lm_head_slices(int dtype, int V);

// ---------------------------------------------------------------- self-conditioning
// u = P E over the vocabulary: P bf16 [M][V] (natural rows), E packed as the B
// operand of a [K = V] x [N = d] product (launch_pack_b16 with src_kn, K = V, N = d).
// Stream-K: the (256-row block, 128-column slab, k-step) space is cut into `grid`
// equal ranges, one per workgroup, each spanning at most two (block, slab) units;
// every range stores its partial tiles, and launch_sc_reduce adds them in range
// order (deterministic).  part holds sc_part_floats(M, d, V) floats.
int sc_grid(int M, int d, int V);
size_t sc_part_floats(int M, int d, int V);
hipError_t launch_sc_expect(const uint16_t* P, int M, int V, const void* Ep, int d, float* part,
                            hipStream_t s);
// u (float [M][d]) and uf (bf16 fragment order, K = d, rows padded to 16) from the partials.
hipError_t launch_sc_reduce(const float* part, int M, int d, int V, float* u, void* uf,
                            hipStream_t s);

// ---------------------------------------------------------------- attention
// q [Hq][M][D]; K [Hkv][rows][D]; V natural [Hkv][rows][D] (f32) or
// transposed-permuted (bf16, vt_index); O [M][Hq*D].  Keys 0..S-1.
struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;               // O in row order; bf16 may pass null when of is given
    void* of = nullptr;    // optional bf16 copy of O in fragment order (frag_offset, K = Hq D)
    int Hq, Hkv, M, S, D;
    int64_t kv_rows;       // row capacity per head of K (and of f32 V)
    int64_t v_rows;        // row capacity per head of the bf16 transposed V (multiple of 32)
    float scale;
    int causal;
    int64_t q_pos0;
    void* part = nullptr;  // split partials workspace (attention_part_bytes): binary16
                           // averages [split][Hq][M][D], then float (max, sum) pairs
    size_t part_bytes = 0; // bytes available at part
    int32_t* bad = nullptr; // optional: kBadRange when a binary16 split average saturates
    // A batch of canvases at the same positions (canvas > 0, decoder only): queries
    // m of canvas b = m / canvas see keys 0..S-1 where key j < ctx is cache row j
    // (the shared context) and key j >= ctx is row j + b * canvas (the canvas's own
    // rows); S = ctx + canvas.  bf16 needs canvas % 256 == 0 and ctx % 32 == 0.
    int64_t ctx = 0;
    int canvas = 0;
};
hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t s);
// Bytes of split partials a call with these sizes needs (0 when it runs unsplit).
size_t attention_part_bytes(int dtype, int Hq, int Hkv, int M, int S, int D);
// Query rows x splits of any split call stay below this bound, whatever M and S:
// a handle sized for it never runs short.
constexpr int64_t kAttnMaxPartRows = 131072;
inline size_t attention_part_bytes_bound(int D) {
    return (size_t)kAttnMaxPartRows * D * 2 + 256 + (size_t)kAttnMaxPartRows * 8;
}

}  // namespace dg
