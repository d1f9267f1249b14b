/*
 * dg.h — C ABI of the MI355X (gfx950) canvas-denoising library (libdg.so).
 *
 * The library runs the parallel canvas-denoising step of block discrete
 * diffusion as described for DiffusionGemma:
 *   - "DiffusionGemma" technical-report summary (hyper.ai paper page),
 *     section Method: the three-stage generation pipeline (causal encoder
 *     fills the KV cache from the prompt; the decoder refines a noisy canvas
 *     with bidirectional attention across the canvas and attention to the KV
 *     cache; the finished canvas goes back through the encoder and is
 *     appended to the cache), the decoder logits equation L_t in R^{C x V},
 *     and the update equations (tempered softmax, Step map);
 *   - same page, section Dataset, "Example and sequence structure": the
 *     P + K*C layout of prompt tokens and canvases;
 *   - "Google's DiffusionGemma Generates 256 Tokens at Once" (alphasignal),
 *     "How text diffusion actually works": canvas initialised with random
 *     tokens, passes that lock high-confidence tokens and refine the rest,
 *     convergence after T passes.
 *
 * Conventions
 *   - Every function returns DG_OK (0) or a negative status; the message of
 *     the last failure on the calling thread is in dg_last_error().
 *   - Argument errors are detected before any work is enqueued and leave the
 *     handle unchanged.
 *   - Work is enqueued asynchronously on the caller's HIP stream (a
 *     hipStream_t passed as void*, NULL = the default stream).  No call
 *     synchronises the host except dg_load_tensor (which copies from host
 *     memory) and the entry points documented as synchronous.
 *   - Pointers prefixed d_ are device pointers owned by the caller; they must
 *     stay valid until the enqueued work completes.  Host pointers are read
 *     before the call returns.
 *   - The handle owns weights, the KV cache and all workspace (device memory
 *     allocated in dg_create).  A handle is not thread-safe: use it from one
 *     host thread and one stream at a time.
 *   - Token ids are int32 in [0, vocab); lock masks are uint8 in {0, 1}.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
#define DG_OK 0
#define DG_EINVAL (-1)      /* bad argument: null pointer, out-of-range value, size mismatch */
#define DG_ENOMEM (-2)      /* device allocation failed */
#define DG_EHIP (-3)        /* a HIP runtime call failed (message has the HIP error) */
#define DG_ECAPACITY (-4)   /* the KV cache cannot hold n_ctx + canvas rows */
#define DG_ESTATE (-5)      /* call out of order: no prompt prefilled, weights missing */
#define DG_ENONFINITE (-6)  /* non-finite logits statistics were produced */
#define DG_ETOKEN (-7)      /* a token id outside [0, V) was read (it embeds as a zero row) */

/* ---------------------------------------------------------------- dtypes */
#define DG_F32 0
#define DG_BF16 1
#define DG_FP8_E4M3 2       /* OCP FP8 E4M3 (bias 7, max 448); expert weights only */
#define DG_MXFP4 3          /* OCP MX FP4: E2M1 elements, one E8M0 scale per 32 along the
                               contraction; expert weights only (the pages' 4-bit deployment,
                               alphasignal, the FP8 / 4-bit quantisation paragraph) */

/* ---------------------------------------------------------------- tensors
 * Logical layouts are [in, out] row-major (y = x W):
 *   DG_T_EMBED [V, d]        token embedding, also the tied LM head (logits = h E^T)
 *   DG_T_WQ    [d, Hq*D]     query projection
 *   DG_T_WK    [d, Hkv*D]    key projection
 *   DG_T_WV    [d, Hkv*D]    value projection
 *   DG_T_WO    [Hq*D, d]     attention output projection
 *   DG_T_WR    [d, E]        router
 *   DG_T_WG    [d, F]        expert gate projection (one expert)
 *   DG_T_WU    [d, F]        expert up projection   (one expert)
 *   DG_T_WD    [F, d]        expert down projection (one expert)
 *   DG_T_SC_WG [d, Fsc]      self-conditioning block, gate projection (cfg.self_cond)
 *   DG_T_SC_WU [d, Fsc]      self-conditioning block, up projection
 *   DG_T_SC_WD [Fsc, d]      self-conditioning block, down projection
 * Element type: act_dtype for the non-expert tensors, expert_dtype for
 * DG_T_WG / DG_T_WU / DG_T_WD.  bf16 is passed as its 16-bit pattern,
 * e4m3 as its 8-bit code plus one float scale per output column. */
#define DG_T_EMBED 0
#define DG_T_WQ 1
#define DG_T_WK 2
#define DG_T_WV 3
#define DG_T_WO 4
#define DG_T_WR 5
#define DG_T_WG 6
#define DG_T_WU 7
#define DG_T_WD 8
#define DG_T_SC_WG 9
#define DG_T_SC_WU 10
#define DG_T_SC_WD 11

/* ---------------------------------------------------------------- captures
 * Debug captures of the last dg_denoise_step, enabled per handle by
 * capture_mask.  Layouts, with C the rows of that pass (the canvas, or
 * B * canvas after a batched pass):
 *   DG_CAP_LOGITS   float [C, V] tempered logits of the last pass
 *   DG_CAP_STATS    per position, 5 arrays of C elements in this order:
 *                   float m (max tempered logit), int32 argmax,
 *                   float lse, float conf (= m - lse), int32 redraw token
 *                   (-1 where the position was locked on entry)
 *   DG_CAP_ROUTING  per layer: int32 idx [C, k] then float gates [C, k]
 *   DG_CAP_HIDDEN   per layer: float residual stream [C, d] after the layer
 *   DG_CAP_ATTN     per layer: attention output [C, Hq*D] in act_dtype
 *   DG_CAP_ROUTER_LOGITS per layer: float router logits [C, E]
 *   DG_CAP_ENTROPY  float [C] predictive entropy (nats) per position of the
 *                   last dg_denoise_step_eb pass; always available (no
 *                   capture_mask bit needed)
 */
#define DG_CAP_LOGITS 1u
#define DG_CAP_STATS 2u
#define DG_CAP_ROUTING 4u
#define DG_CAP_HIDDEN 8u
#define DG_CAP_ATTN 16u
#define DG_CAP_ROUTER_LOGITS 32u
#define DG_CAP_ENTROPY 64u
/* DG_CAP_SELFCOND (cfg.self_cond; always kept, no capture bit needed): float
 * [C, d] of the last pass that formed the self-conditioning signal, layer 0
 * selecting u = p0 E and layer 1 the signal z = FFW(u) the next pass reads. */
#define DG_CAP_SELFCOND 128u

typedef struct dg_model_cfg {
    int32_t n_layers;      /* L */
    int32_t d_model;       /* d, multiple of 4, at most 4096 (bf16/fp8: multiple of 64) */
    int32_t n_q_heads;     /* Hq, multiple of n_kv_heads */
    int32_t n_kv_heads;    /* Hkv */
    int32_t head_dim;      /* D: 64 or 128 (bf16 path: 128) */
    int32_t n_experts;     /* E */
    int32_t top_k;         /* k <= E, k <= 16 */
    int32_t d_ff;          /* F, expert hidden width, multiple of 64 for bf16/fp8 */
    int32_t vocab;         /* V (bf16 path: multiple of 128) */
    int32_t canvas;        /* C, canvas length (<= 1024) */
    int64_t max_ctx;       /* KV rows per layer: >= P + K*C */
    double rope_base;      /* RoPE base (rotate-half pairs, absolute positions) */
    float rms_eps;         /* RMSNorm epsilon (unit gains) */
    float temperature;     /* tau > 0: p0 = softmax(logits / tau) */
    int32_t act_dtype;     /* DG_F32 or DG_BF16: activations, KV cache, dense weights */
    int32_t expert_dtype;  /* DG_F32, DG_BF16, DG_FP8_E4M3 or DG_MXFP4 (the last two need
                              act_dtype DG_BF16; DG_MXFP4 needs d_model % 128 == 0) */
    uint32_t capture_mask; /* DG_CAP_* bits */
    int32_t max_batch;     /* canvases one batched pass holds (dg_denoise_step_batch); 0 or 1:
                              single canvases only.  max_batch * canvas <= 65536 */
    int32_t self_cond;     /* 1: self-conditioning (see "self-conditioning" below), 0: off */
    int32_t sc_ff;         /* Fsc, hidden width of its feed-forward block (0: d_model);
                              multiple of 64 (bf16) or of 4 (f32; then vocab % 8 == 0) */
} dg_model_cfg;

typedef struct dg_handle dg_handle;

/* Create a handle: validates cfg, allocates weights, KV cache
 * ([L][Hkv][max_ctx][D] for K and for V), RoPE tables and workspace on the
 * current HIP device.  *out receives the handle.  Synchronous. */
int dg_create(const dg_model_cfg* cfg, dg_handle** out);

/* Free everything the handle owns.  Waits for the device.  NULL is a no-op. */
void dg_destroy(dg_handle* h);

/* Message of the last failure on this thread ("" if none). */
const char* dg_last_error(void);

/* Copy one logical tensor from host memory into the handle, re-laid out for
 * the kernels.  kind = DG_T_*; layer in [0, L) (ignored for DG_T_EMBED);
 * expert in [0, E) for expert tensors (-1: all E at once, [E, in, out]),
 * else ignored.  bytes must equal the tensor size in its storage type.
 * host_scales: e4m3 experts: float per output column (F for WG/WU, d for WD);
 * MX FP4 experts: the codes are [in][out / 2] bytes (two E2M1 per byte, the
 * even output column in the low nibble) and host_scales holds uint8 E8M0
 * exponents [in / 32][out] (one per 32 rows of a column, value 2^(s - 127));
 * NULL otherwise.  Synchronous. */
int dg_load_tensor(dg_handle* h, int32_t kind, int32_t layer, int32_t expert,
                   const void* host_src, size_t bytes, const void* host_scales);

/* Stage 1 (technical report, Method, generation pipeline): run the causal
 * encoder over P prompt ids (d_prompt_ids, device int32 [P]) and fill K/V
 * rows 0..P-1 of every layer.  Resets the context: afterwards n_ctx = P and
 * the canvas index k_blk = 0.  P >= 0 (P = 0 gives an empty context).
 * Prompt ids outside [0, V) embed as zero rows; dg_check_finite reports them. */
int dg_prefill_prompt_kv(dg_handle* h, const int32_t* d_prompt_ids, int32_t P, void* stream);

/* Stage 2, one denoise pass over the canvas at positions n_ctx..n_ctx+C-1:
 * logits = Decoder(canvas, KV cache) with bidirectional attention over
 * [KV cache || canvas]; p0 = softmax(logits / tau); among unlocked positions
 * the n_s with the highest confidence log max p0 (ties to the lower
 * position) are locked to their argmax token (ties to the lower id), where
 * n_s = min(ceil(C/T), #unlocked) and n_s = #unlocked at step T-1; every
 * other unlocked position is redrawn from p0 by Gumbel-max with Philox4x32-10
 * uniforms (key = seed; counter (v, i>>2, step | k_blk<<16, 0x47554D42),
 * word i&3, u = (2*(word>>9)+1) * 2^-24).  Locked positions are not written.
 * d_canvas: device int32 [C], updated in place; d_locked_mask: device uint8
 * [C], updated in place.  0 <= step < T.  Needs a prefilled context
 * (DG_ESTATE otherwise) and room for C rows (DG_ECAPACITY).  Asynchronous:
 * canvas ids outside [0, V) and non-finite statistics are reported later by
 * dg_check_finite or dg_generate_block. */
int dg_denoise_step(dg_handle* h, int32_t* d_canvas, uint8_t* d_locked_mask, int32_t step,
                    int32_t T, uint64_t seed, void* stream);

/* Canvas initialisation alone (alphasignal, "How text diffusion actually
 * works", step 1; technical report, Method, forward process at kappa = 0):
 * d_canvas[i] = uniform token from Philox (counter (i>>2, k_blk, 0,
 * 0x494E4954), word i&3, token = word*V >> 32), d_locked_mask[i] = 0, for
 * the handle's current canvas index k_blk.  Either pointer may be NULL. */
int dg_init_canvas(dg_handle* h, int32_t* d_canvas, uint8_t* d_locked_mask, uint64_t seed,
                   void* stream);

/* One 256-token block (technical report, Method, block-autoregressive
 * generation): initialise the canvas uniformly over [0, V) with Philox
 * (counter (i>>2, k_blk, 0, 0x494E4954), word i&3, token = word*V >> 32),
 * run T denoise passes, write the canvas to d_out_tokens (device int32 [C]);
 * if commit != 0, run stage 3 (the causal encoder over the final canvas,
 * appending its K/V; n_ctx += C, k_blk += 1).  Synchronous only if the
 * handle checks the non-finite flag (always: it reads one int at the end). */
int dg_generate_block(dg_handle* h, int32_t* d_out_tokens, int32_t T, uint64_t seed,
                      int32_t commit, void* stream);

/* ---------------------------------------------------------------- batched canvases
 * B canvases (1 <= B <= cfg.max_batch) denoised in one pass (the technical-report
 * summary's Experiment, inference analysis: the method's advantage is largest at
 * low batch, its throughput at large batch lower; the alphasignal page, "The
 * numbers", low-to-medium batch).  The B canvases continue the same context at
 * the same positions n_ctx..n_ctx+C-1, as independent samples of the next
 * block: every canvas attends bidirectionally to the context and to itself,
 * never to another canvas of the batch; its K/V rows go to cache rows n_ctx + b*C
 * + i, so n_ctx + B*C <= max_ctx.  Canvas b draws its Philox uniforms as
 * positions b*C .. b*C+C-1 of one long canvas (same counters as dg_denoise_step
 * and dg_init_canvas otherwise), so a batch of one equals the single-canvas
 * calls.  The lock schedule runs per canvas.  Buffers are [B][C] (canvas b at
 * offset b*C).  bf16 activations need canvas % 256 == 0 and n_ctx % 32 == 0
 * when B > 1.  Errors and asynchrony as dg_denoise_step. */
int dg_denoise_step_batch(dg_handle* h, int32_t* d_canvas, uint8_t* d_locked_mask, int32_t B,
                          int32_t step, int32_t T, uint64_t seed, void* stream);

/* The initial canvases of a batch (dg_init_canvas over B*C positions); either
 * pointer may be NULL. */
int dg_init_canvas_batch(dg_handle* h, int32_t* d_canvas, uint8_t* d_locked_mask, int32_t B,
                         uint64_t seed, void* stream);

/* B blocks at once: the initial canvases of the batch, T batched passes, the B
 * canvases written to d_out_tokens (device int32 [B][C]).  No commit (commit one
 * of them with dg_commit_canvas).  Synchronous as dg_generate_block. */
int dg_generate_block_batch(dg_handle* h, int32_t* d_out_tokens, int32_t B, int32_t T,
                            uint64_t seed, void* stream);

/* ---------------------------------------------------------------- entropy-bounded sampler
 * The sampler of the technical-report summary (Method, the paragraphs on the
 * sampler and on adaptive stopping; Experiment, the recommended sampler:
 * tau 0.8 -> 0.4, at most 48 passes, separate thresholds for selection and
 * stopping, whose values the pages do not give). */
typedef struct dg_eb_params {
    float tau_max;       /* temperature at pass 0 (0.8) */
    float tau_min;       /* temperature at pass max_steps - 1 (0.4) */
    float gamma;         /* selection tolerance on the bound B, nats */
    float theta;         /* stop threshold on the canvas-mean entropy, nats */
    int32_t max_steps;   /* passes at most (48) */
} dg_eb_params;

/* One sampler pass given its statistics (all device buffers of C elements):
 * d_entropy float H_i, d_argmax int32, d_draw int32 (Gumbel-max draw at
 * tau_s), d_prev_argmax int32 in/out (the previous pass's argmax; ignored at
 * step 0, overwritten with d_argmax), d_canvas int32 and d_locked_mask uint8
 * in/out, d_info int32 [4] out: finished (0/1), positions locked by this
 * pass, positions left unlocked, 1 if the stop test held.
 *   Stop test (step >= 1): sum_i H_i (float64, in position order) / C < theta
 *   and d_argmax equals d_prev_argmax everywhere.  It, or step = max_steps-1,
 *   locks every unlocked position to its argmax and finishes the block.
 *   Otherwise unlocked positions are ranked by H ascending (ties to the lower
 *   position; NaN last) and accepted in rank order while B stays below
 *   gamma, B = (float64 running sum of the accepted entropies in rank order)
 *   minus the entropy just added (the largest so far); the first candidate
 *   always is.  Accepted positions take d_draw and lock; the other unlocked
 *   ones take a uniform token: Philox4x32-10, key = seed, counter (i>>2,
 *   k_blk, step, 0x524E5345), word i&3, token = word*V >> 32.  A pass that
 *   leaves nothing unlocked also finishes the block.
 * 0 < C <= 1024, V > 0, 0 <= step < max_steps; tau_max, tau_min unused here.
 * The caller owns every buffer; nothing is allocated.  Asynchronous. */
int dg_eb_sample(const float* d_entropy, const int32_t* d_argmax, const int32_t* d_draw,
                 int32_t* d_prev_argmax, int32_t* d_canvas, uint8_t* d_locked_mask,
                 int32_t* d_info, int32_t C, int32_t V, int32_t step, const dg_eb_params* p,
                 uint64_t seed, int32_t k_blk, void* stream);

/* One pass of stage 2 with the entropy-bounded sampler: the decoder as in
 * dg_denoise_step, the LM head at tau_s = tau_min + (tau_max - tau_min) *
 * (max_steps-1-step) / (max_steps-1) (tau_min if max_steps = 1), the
 * per-position entropy H_i of softmax(logits / tau_s) kept by the head's
 * streaming epilogue, the Gumbel-max draw of unlocked positions at tau_s
 * (the dg_denoise_step stream), then dg_eb_sample with the handle's own
 * previous-argmax buffer.  d_info: device int32 [4] as in dg_eb_sample, or
 * NULL to keep it in the handle.  Passes of one block must run in order from
 * step 0.  Errors and asynchrony as dg_denoise_step. */
int dg_denoise_step_eb(dg_handle* h, int32_t* d_canvas, uint8_t* d_locked_mask, int32_t step,
                       const dg_eb_params* p, uint64_t seed, int32_t* d_info, void* stream);

/* One block with the entropy-bounded sampler: the initial canvas of
 * dg_generate_block, then dg_denoise_step_eb passes until one finishes the
 * block (reads 16 bytes back after each pass), then the output copy and the
 * optional commit as in dg_generate_block.  *n_steps (if not NULL) receives
 * the number of passes run.  Synchronous. */
int dg_generate_block_eb(dg_handle* h, int32_t* d_out_tokens, const dg_eb_params* p,
                         uint64_t seed, int32_t commit, int32_t* n_steps, void* stream);

/* ---------------------------------------------------------------- self-conditioning
 * The decoder's continuous input z_t that feeds its previous predictions back
 * (technical-report summary, Method: decoder equation L_t = Decoder(x_t, z_t, H)
 * and the update equations p0 = Softmax(L_t / tau_t), z = FFW(p0 E); Dataset,
 * "How the data is used": a zero state in half of the training examples).
 * With cfg.self_cond = 1 (and the DG_T_SC_* tensors loaded):
 *   - z is added to the canvas token embedding before the first layer;
 *   - a pass with step 0 takes z = 0; a pass with step > 0 reads the z the
 *     handle holds (that of the previous pass, or dg_set_self_cond);
 *   - every pass but the last of its block (step < T-1, entropy-bounded:
 *     step < max_steps-1) forms the next signal from its own logits:
 *     p0 = Softmax(L / tau) at the pass's temperature, u = p0 E over the whole
 *     vocabulary, z = (silu(u Wg) * (u Wu)) Wd with the DG_T_SC_* weights.
 * So the passes of one block (or batch) run in order on one handle.  bf16:
 * p0, u and the hidden layer are stored in bf16, z in float; the contraction
 * reads a second copy of E packed over the vocabulary (V d bf16 more device
 * memory).  The signal rows of a batch are [B][C][d]. */

/* Overwrite the signal the next pass with step > 0 reads: d_z device float
 * [rows, d], rows <= max_batch * canvas (rows of canvas b at b*C).
 * DG_ESTATE without cfg.self_cond.  Asynchronous. */
int dg_set_self_cond(dg_handle* h, const float* d_z, int32_t rows, void* stream);

/* Stage 3 alone: append the causal-encoder K/V of a finished canvas
 * (device int32 [C]) at rows n_ctx..n_ctx+C-1; n_ctx += C, k_blk += 1. */
int dg_commit_canvas(dg_handle* h, const int32_t* d_canvas, void* stream);

/* Read and clear the handle's sticky error flags.  A pass whose logits
 * statistics were not finite sets one; an embedding of a token id outside
 * [0, V) (prompt, canvas or committed canvas ids) sets the other and reads a
 * zero row instead of the table.  Neither stops the passes queued after it.
 * Synchronises the stream.  DG_ETOKEN if an id was out of range, else
 * DG_ENONFINITE if statistics were not finite, else DG_OK. */
int dg_check_finite(dg_handle* h, void* stream);

/* Forget the context (n_ctx = 0, k_blk = 0).  Weights stay loaded. */
int dg_reset_context(dg_handle* h);

/* Current committed context length and canvas index. */
int dg_get_state(dg_handle* h, int64_t* n_ctx, int32_t* k_blk);

/* Declare the committed context: n_ctx rows of every layer's cache hold valid
 * K/V (restored with dg_set_kv from a saved cache, or injected) and the next
 * canvas has index k_blk.  With dg_get_state and dg_get_kv this saves and
 * resumes a context without re-running the encoder.  0 <= n_ctx, n_ctx + C <=
 * max_ctx, k_blk >= 0 (DG_EINVAL otherwise); afterwards the handle counts as
 * prefilled.  Synchronous only in that it waits for nothing. */
int dg_set_state(dg_handle* h, int64_t n_ctx, int32_t k_blk);

/* Replay the decoder-layer stack of dg_denoise_step as a HIP graph (enable = 1,
 * the default) or launch its kernels one by one (0).  The graph is captured
 * on first use for the current context length and replaced when n_ctx, the
 * weights or the context change; passes with per-layer captures
 * (DG_CAP_ROUTING, _HIDDEN, _ATTN, _ROUTER_LOGITS) or kernel timing enabled
 * run eagerly.  Both paths launch the same kernels with the same arguments,
 * so results are identical.  Waits for the device. */
int dg_set_graphs(dg_handle* h, int32_t enable);

/* Change which captures the following passes record (DG_CAP_* bits; 0 turns
 * them off).  Allocates the buffers a capture needs on first use; waits for
 * the device. */
int dg_set_capture(dg_handle* h, uint32_t capture_mask);

/* Copy a capture of the last denoise pass (see DG_CAP_*) into device memory
 * d_dst of exactly `bytes` bytes.  layer selects the layer for per-layer
 * captures.  DG_ESTATE if the capture was not enabled. */
int dg_get_capture(dg_handle* h, uint32_t what, int32_t layer, void* d_dst, size_t bytes,
                   void* stream);

/* Copy one layer's K or V cache rows [row0, row0+n) into device memory as
 * [Hkv, n, D] in act_dtype (which = 0 for K, 1 for V). */
int dg_get_kv(dg_handle* h, int32_t layer, int32_t which, int64_t row0, int64_t n, void* d_dst,
              void* stream);

/* Overwrite one layer's K or V cache rows [row0, row0+n) from device memory
 * laid out [Hkv, n, D] in act_dtype (which = 0 for K, 1 for V; K rows hold
 * the rotated keys).  Restores a saved cache or injects one computed
 * elsewhere; n_ctx is not changed.  row0 + n <= max_ctx. */
int dg_set_kv(dg_handle* h, int32_t layer, int32_t which, int64_t row0, int64_t n,
              const void* d_src, void* stream);

/* ---------------------------------------------------------------- kernel timing
 * HIP events recorded on the caller's stream around the launches of each
 * kernel class, for live per-kernel timing (the events themselves add no
 * host synchronisation).  dg_profile_begin enables recording for at most
 * max_launches launches; dg_profile_end synchronises the device, writes the
 * summed milliseconds and the launch count per class (arrays of DG_PROF_N)
 * and disables recording. */
#define DG_PROF_MOE_GEMM1 0   /* expert gate/up GEMM + SwiGLU */
#define DG_PROF_MOE_GEMM2 1   /* expert down GEMM */
#define DG_PROF_ATTENTION 2   /* attention incl. split combine */
#define DG_PROF_LM_HEAD 3     /* LM head with the streaming epilogue */
#define DG_PROF_DENSE 4       /* QKV, output and router projections */
#define DG_PROF_SELF_COND 5   /* self-conditioning: the p0 E contraction over the vocabulary */
#define DG_PROF_N 6
int dg_profile_begin(dg_handle* h, int32_t max_launches);
int dg_profile_end(dg_handle* h, double* total_ms, int32_t* counts);

/* ---------------------------------------------------------------- kernel-level entry points */

/* Attention for one batch of queries, the decoder's attention step
 * (technical-report summary, Method, generation pipeline: bidirectional
 * attention across the canvas and attention to the KV cache; alphasignal,
 * paragraph on bidirectional attention):
 *   O[m, h*D + t] = sum_j softmax_j(scale * q_h,m . k_g,j [+ mask]) v_g,j,t
 * with GQA group g = h / (Hq / Hkv).  d_q: [Hq, M, D]; d_k, d_v: [Hkv, S, D];
 * d_o: [M, Hq*D]; all dtype (DG_F32 or DG_BF16, bf16 requires D = 128).
 * causal != 0 masks key j for query m when j > q_pos0 + m (keys are at
 * positions 0..S-1); causal = 0 is the canvas' bidirectional attention.
 * d_workspace: caller-owned device scratch of at least the bytes
 * dg_attention_workspace_size reports for the same arguments (NULL allowed
 * when that is 0): the bf16 path packs a transposed, key-permuted copy of V
 * there and keeps the per-split partials of a key range split over
 * workgroups (binary16 split averages: |v| entries of 65520 and above
 * saturate at 65504).  Nothing is allocated.  A workspace must not be shared
 * by calls that may overlap.  DG_EINVAL for bad sizes or a short workspace,
 * before any work is enqueued.  Asynchronous. */
int dg_attention(const void* d_q, const void* d_k, const void* d_v, void* d_o, int32_t Hq,
                 int32_t Hkv, int32_t M, int32_t S, int32_t D, float scale, int32_t causal,
                 int32_t q_pos0, int32_t dtype, void* d_workspace, size_t workspace_bytes,
                 void* stream);

/* Workspace bytes dg_attention needs for these arguments (*bytes = 0: none).
 * Validates them as dg_attention does; touches no device. */
int dg_attention_workspace_size(int32_t Hq, int32_t Hkv, int32_t M, int32_t S, int32_t D,
                                int32_t causal, int32_t q_pos0, int32_t dtype, size_t* bytes);

/* dg_attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static device array of
 * 64 MiB (one per GPU, held until the process ends); calls whose workspace
 * (dg_attention_workspace_size) exceeds it fail with DG_EINVAL before any work
 * is enqueued.  The first call on a device resolves the array's address
 * (hipGetSymbolAddress).  Every call on one GPU shares the array, so calls
 * that may overlap on one GPU (other streams, other threads) race: the caller
 * orders them.  Nothing is allocated; results equal dg_attention's. */
int dg_attention_noalloc(const void* d_q, const void* d_k, const void* d_v, void* d_o,
                         int32_t Hq, int32_t Hkv, int32_t M, int32_t S, int32_t D, float scale,
                         int32_t causal, int32_t q_pos0, int32_t dtype, void* stream);

/* One MoE FFN layer on hidden states, the decoder's MoE step
 * (technical-report summary, Experiment: a mixture-of-experts transformer
 * with a small number of active experts among many), applied to its input
 * directly (no norm, no residual): router logits r = x Wr; top-k of
 * softmax(r) (ties to the lower expert id) with gates renormalised over the
 * k chosen; y = sum_j gate_j * (silu(x Wg_e) * (x Wu_e)) Wd_e, e = idx_j.
 * Uses layer `layer` of the handle's weights.  d_x: [n_tokens, d] act_dtype;
 * d_y: [n_tokens, d] act_dtype.  Optional d_idx (int32 [n_tokens, k]) and
 * d_gates (float [n_tokens, k]) receive the routing; pass NULL to skip.
 * n_tokens <= max(C, 4096), the handle's batch capacity.  Uses the
 * handle's workspace: calls on one handle must not overlap. */
int dg_moe_layer(dg_handle* h, int32_t layer, const void* d_x, int32_t n_tokens, void* d_y,
                 int32_t* d_idx, float* d_gates, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
