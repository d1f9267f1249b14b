"""The canvas denoiser, plainly, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
  * Three stages ([TR] Method, generation pipeline paragraph): (1) the prompt
    goes through the causal encoder to fill the KV cache; (2) the decoder
    refines a noisy canvas with bidirectional attention across the canvas and
    attention to the KV cache; (3) the finished canvas goes back through the
    causal encoder and is appended to the KV cache.  Encoder and decoder share
    weights ([TR] Method, architecture paragraph).
  * Block-autoregressive generation over canvases of 256 tokens, sequence
    layout P prompt tokens + K canvases of C tokens ([TR] Dataset, "Example
    and sequence structure"; Method, block-autoregressive paragraph).
  * Decoder logits L_t in R^{C x V} ([TR] Method, decoder equation) and the
    tempered posterior p0 = Softmax(L_t / tau) ([TR] Method, update equations,
    first line); the next canvas is drawn by a Step map from (x_t, p0)
    ([TR] Method, Step equation and third update line).
  * Canvas initialised with random tokens; each pass locks in high-confidence
    tokens and refines the rest; the block resolves after T passes ([AS] "How
    text diffusion actually works", steps 1-3).
  * Every canvas position attends to every other ([AS], paragraph on
    bidirectional attention).
  * A mixture-of-experts transformer with a 262k vocabulary and a token
    embedding E in R^{V x d} ([TR] Experiment, architecture paragraph; Method,
    definition of E).

Readings where the pages are silent (the synthetic configurations fix the
sizes, "RMSNorm", "RoPE base 10000", "SwiGLU", top-k routing with
softmax-renormalised gates, and the lock / redraw schedule):
  * block: pre-norm, h += Attn(RMSNorm h); h += MoE(RMSNorm h); final RMSNorm;
    no biases, no extra norms, no embedding scaling;
  * LM head tied to E: logits = RMSNorm(h) E^T (E is the only vocabulary
    matrix the pages define);
  * GQA: query head h reads KV head floor(h / (Hq / Hkv)); scores scaled by
    1/sqrt(D); decoder attention unmasked, encoder attention causal;
  * router: softmax over all experts, top-k (ties to the lower expert id),
    gates renormalised over the k chosen;
  * self-conditioning input z_t: zero unless the workload enables the
    self-conditioning block; then z = FFW(p0 E) of the previous pass is added
    to the canvas embedding and the first pass of a block takes z = 0 (see
    ``self_cond`` for the readings);
  * confidence = log of the largest tempered probability, m - lse;
  * schedule: pass s locks n_s = min(ceil(C/T), #unlocked) unlocked positions
    with the highest confidence (ties to the lower position), all remaining
    ones at s = T - 1; a newly locked position takes its argmax token (ties to
    the lower id); every other unlocked position is redrawn from p0 by the
    Gumbel-max rule with Philox uniforms (see ``philox``); locked positions are
    never written;
  * precision plan for the bf16 configurations: values are rounded to bf16
    where they are stored in bf16 (normed activations, Q/K/V, attention
    output, SwiGLU output, KV cache); the residual stream, router logits,
    expert outputs and all statistics stay in full precision.  For fp8
    experts, the expert inputs (normed activation, SwiGLU output) are rounded
    to e4m3 (saturating, no scale) and the weights are code * column scale;
    MX FP4 experts take the same e4m3 inputs and weights E2M1 value * E8M0
    block scale.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .numerics import rmsnorm, rope, round_bf16, e4m3_round, softmax, silu
from .philox import init_canvas, gumbel_uniforms
from . import eb_sampler as eb
from .self_cond import SelfCond, next_signal


# =========================================================================== pieces
def attention(q, k, v, causal: bool = False, q_pos=None, k_pos=None, scale=None) -> np.ndarray:
    """O = softmax(Q K^T * scale [+ causal mask]) V per query head, dense, two-pass.

    q [Hq, M, D]; k, v [Hkv, S, D].  With ``causal`` a key at position k_pos[j]
    is visible to a query at q_pos[i] iff k_pos[j] <= q_pos[i].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Hq, M, D = q.shape
    Hkv, S, _ = k.shape
    group = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    out = np.empty((Hq, M, D), np.float64)
    if causal:
        visible = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]
    for h in range(Hq):
        kh = h // group
        s = (q[h] @ k[kh].T) * scale
        if causal:
            s = np.where(visible, s, -np.inf)
        out[h] = softmax(s, axis=-1) @ v[kh]
    return out


def route_topk(r, k: int):
    """Top-k routing of router logits r [M, E].

    Returns (idx [M, k] in descending probability, ties to the lower expert id;
    gates [M, k] = p / sum of the chosen p; margin [M] = logit gap between the
    k-th and (k+1)-th largest logits, +inf when k == E).
    """
    r = np.asarray(r, np.float64)
    M, E = r.shape
    p = softmax(r, axis=-1)
    order = np.argsort(-p, axis=-1, kind="stable")
    idx = order[:, :k]
    ps = np.take_along_axis(p, idx, axis=-1)
    gates = ps / ps.sum(axis=-1, keepdims=True)
    rs = np.take_along_axis(r, order, axis=-1)
    margin = rs[:, k - 1] - rs[:, k] if k < E else np.full(M, np.inf)
    return idx.astype(np.int32), gates, margin


def moe_ffn(b, idx, gates, expert_weights, expert_round=None, hidden_round=None):
    """y[t] = sum over the chosen experts (slot order) of g * (SwiGLU_e(b[t]) Wd_e).

    ``expert_weights(e)`` returns (Wg [d, F], Wu [d, F], Wd [F, d]) in float64.
    ``expert_round`` rounds the expert input, ``hidden_round`` the SwiGLU output.
    """
    b = np.asarray(b, np.float64)
    M, d = b.shape
    k = idx.shape[1]
    xr = expert_round(b) if expert_round is not None else b
    contrib = np.zeros((M, k, d), np.float64)
    for e in np.unique(idx):
        rows, slots = np.nonzero(idx == e)
        wg, wu, wd = expert_weights(int(e))
        xe = xr[rows]
        with np.errstate(over="ignore"):
            hmid = silu(xe @ wg) * (xe @ wu)
        if hidden_round is not None:
            hmid = hidden_round(hmid)
        contrib[rows, slots] = hmid @ wd
    y = np.zeros((M, d), np.float64)
    for j in range(k):
        y += gates[:, j:j + 1] * contrib[:, j]
    return y


@dataclass
class HeadStats:
    m: np.ndarray          # max tempered logit            [C]
    argmax: np.ndarray     # lowest id attaining m          [C] int32
    lse: np.ndarray        # log-sum-exp of tempered logits [C]
    conf: np.ndarray       # m - lse = log max p0           [C]
    top2_gap: np.ndarray   # m minus the runner-up logit    [C]


def lm_head_stats(z) -> HeadStats:
    """Per-position statistics of the tempered logits z [C, V] (materialised)."""
    z = np.asarray(z, np.float64)
    a = np.argmax(z, axis=-1)                       # first index of the max
    m = z[np.arange(z.shape[0]), a]
    lse = m + np.log(np.sum(np.exp(z - m[:, None]), axis=-1))
    part = np.partition(z, z.shape[1] - 2, axis=-1)[:, -2:] if z.shape[1] > 1 else None
    gap = (m - part[:, 0]) if part is not None else np.full(z.shape[0], np.inf)
    return HeadStats(m=m, argmax=a.astype(np.int32), lse=lse, conf=m - lse, top2_gap=gap)


def gumbel_noise(u) -> np.ndarray:
    """G = -log(-log u): adding it to logits and taking the argmax draws from the softmax."""
    return -np.log(-np.log(np.asarray(u, np.float64)))


def gumbel_draw(z_rows, u_rows):
    """argmax_v (z + G) per row (ties to the lower id) and the best-minus-second gap."""
    s = np.asarray(z_rows, np.float64) + gumbel_noise(u_rows)
    w = np.argmax(s, axis=-1)
    best = s[np.arange(s.shape[0]), w]
    if s.shape[1] > 1:
        second = np.partition(s, s.shape[1] - 2, axis=-1)[:, -2]
    else:
        second = np.full(s.shape[0], -np.inf)
    return w.astype(np.int32), best - second


def lock_count(s: int, T: int, C: int, n_unlocked: int) -> int:
    """Positions locked at pass s: ceil(C/T) capped by what is left; all at the last pass."""
    if s == T - 1:
        return n_unlocked
    return min(-(-C // T), n_unlocked)


@dataclass
class SamplerResult:
    canvas: np.ndarray
    mask: np.ndarray
    new_locks: np.ndarray     # positions locked at this pass (sorted by rank)
    redrawn: np.ndarray       # unlocked positions redrawn at this pass
    cut_low: float            # confidence of the last position locked (or +inf)
    cut_high: float           # confidence of the best position left unlocked (or -inf)


def sampler_update(canvas, mask, conf, argmax, redraw_tokens, s: int, T: int) -> SamplerResult:
    """One Step: lock the most confident unlocked positions, redraw the rest.

    Ranking is by confidence descending, ties to the lower position.
    """
    canvas = np.array(canvas, dtype=np.int32, copy=True)
    mask = np.array(mask, dtype=np.uint8, copy=True)
    C = canvas.shape[0]
    unlocked = np.flatnonzero(mask == 0)
    n = lock_count(s, T, C, unlocked.size)
    conf = np.asarray(conf, np.float64)
    order = unlocked[np.lexsort((unlocked, -conf[unlocked]))]
    new = order[:n]
    rest = order[n:]
    canvas[new] = np.asarray(argmax)[new]
    mask[new] = 1
    canvas[rest] = np.asarray(redraw_tokens)[rest]
    lo = conf[new[-1]] if n > 0 else np.inf
    hi = conf[rest[0]] if rest.size > 0 else -np.inf
    return SamplerResult(canvas, mask, new, rest, lo, hi)


# =========================================================================== model
@dataclass
class StepResult:
    canvas: np.ndarray
    mask: np.ndarray
    stats: HeadStats
    redraw: np.ndarray            # Gumbel winner per position (-1 where not drawn)
    redraw_gap: np.ndarray        # best - second perturbed score (nan where not drawn)
    sampler: SamplerResult
    route_idx: list               # per layer [C, k]
    route_gates: list             # per layer [C, k]
    route_margin: list            # per layer [C]
    logits: np.ndarray | None = None
    hidden: list = field(default_factory=list)   # per layer residual after the layer
    sc: SelfCond | None = None    # the next pass's self-conditioning signal


class OracleModel:
    """Prefill / denoise step / commit of the shared-weight denoiser, float64."""

    def __init__(self, w, weights, capture_hidden: bool = False):
        self.w = w
        self.W = weights
        self.L = w.n_layers
        self.K = [None] * self.L      # per layer [Hkv, n_ctx, D]
        self.V = [None] * self.L
        self.n_ctx = 0
        self.k_blk = 0
        self.enc_route_margin = [np.zeros(0) for _ in range(self.L)]   # per layer, per row
        self.capture_hidden = capture_hidden
        self.bf16 = w.act == "bf16"
        self.fp8 = w.experts in ("fp8", "mxfp4")     # e4m3 expert inputs either way

    # ------------------------------------------------------------ precision plan
    def _act(self, x):
        return round_bf16(x) if self.bf16 else np.asarray(x, np.float64)

    def _expert_in(self, x):
        return e4m3_round(x) if self.fp8 else None

    # ------------------------------------------------------------ one layer
    def _qkv(self, l, a, positions):
        w = self.w
        M = a.shape[0]
        q = (a @ self.W.dense("wq", l)).reshape(M, w.n_q_heads, w.head_dim).transpose(1, 0, 2)
        q = self._act(rope(q, positions, w.rope_base))
        k, v = self.kv_rows(l, a, positions)
        return q, k, v

    def kv_rows(self, l, a, positions):
        """Cache rows of layer l for the normed rows a [M, d] at `positions`: the rotated
        keys and the values, [Hkv, M, D] each."""
        w = self.w
        M = a.shape[0]
        k = (a @ self.W.dense("wk", l)).reshape(M, w.n_kv_heads, w.head_dim).transpose(1, 0, 2)
        v = (a @ self.W.dense("wv", l)).reshape(M, w.n_kv_heads, w.head_dim).transpose(1, 0, 2)
        return self._act(rope(k, positions, w.rope_base)), self._act(v)

    def _moe(self, l, b):
        w = self.w
        r = b @ self.W.dense("wr", l)
        idx, gates, margin = route_topk(r, w.top_k)

        def ew(e):
            return (self.W.expert("wg", l, e), self.W.expert("wu", l, e),
                    self.W.expert("wd", l, e))

        if self.fp8:
            y = moe_ffn(b, idx, gates, ew, expert_round=e4m3_round, hidden_round=e4m3_round)
        elif self.bf16:
            y = moe_ffn(b, idx, gates, ew, hidden_round=round_bf16)
        else:
            y = moe_ffn(b, idx, gates, ew)
        return y, idx, gates, margin

    def _layer(self, l, h, positions, k_ctx, v_ctx, causal, ctx_pos, need_output=True):
        """Returns (new h or None, k_new, v_new, routing)."""
        w = self.w
        a = self._act(rmsnorm(h, w.rms_eps))
        q, k, v = self._qkv(l, a, positions)
        if not need_output:
            return None, k, v, None
        kk = np.concatenate([k_ctx, k], axis=1) if k_ctx is not None else k
        vv = np.concatenate([v_ctx, v], axis=1) if v_ctx is not None else v
        kpos = np.concatenate([ctx_pos, positions]) if k_ctx is not None else positions
        o = attention(q, kk, vv, causal=causal, q_pos=positions, k_pos=kpos)
        o = self._act(o.transpose(1, 0, 2).reshape(h.shape[0], w.n_q_heads * w.head_dim))
        h = h + o @ self.W.dense("wo", l)
        b = self._act(rmsnorm(h, w.rms_eps))
        y, idx, gates, margin = self._moe(l, b)
        return h + y, k, v, (idx, gates, margin)

    def encoder_layer_rows(self, l, h, positions):
        """Causal encoder layer l applied to some rows only: h [n, d] are the layer's input
        rows at `positions`, and the cache of layer l (self.K[l], self.V[l], rows at
        positions 0, 1, ...) already holds every position up to max(positions), these rows'
        own keys included.  Each row attends to the cached keys at positions <= its own.
        Returns (output rows [n, d], routing margin of each row)."""
        w = self.w
        positions = np.asarray(positions)
        a = self._act(rmsnorm(h, w.rms_eps))
        q = (a @ self.W.dense("wq", l)).reshape(len(positions), w.n_q_heads,
                                                w.head_dim).transpose(1, 0, 2)
        q = self._act(rope(q, positions, w.rope_base))
        S = self.K[l].shape[1]
        o = attention(q, self.K[l], self.V[l], causal=True, q_pos=positions, k_pos=np.arange(S))
        o = self._act(o.transpose(1, 0, 2).reshape(len(positions), w.n_q_heads * w.head_dim))
        h = h + o @ self.W.dense("wo", l)
        b = self._act(rmsnorm(h, w.rms_eps))
        y, _, _, margin = self._moe(l, b)
        return h + y, margin

    # ------------------------------------------------------------ stage 1 / stage 3
    def _encode(self, ids, start):
        """Causal encoder over ids at positions start..; appends K/V to the cache."""
        E = self.W.embed()
        h = E[np.asarray(ids)]
        positions = np.arange(start, start + len(ids))
        ctx_pos = np.arange(start)
        for l in range(self.L):
            last = l == self.L - 1
            kc = self.K[l] if start > 0 else None
            vc = self.V[l] if start > 0 else None
            h, k, v, rt = self._layer(l, h, positions, kc, vc, causal=True, ctx_pos=ctx_pos,
                                      need_output=not last)
            if rt is not None:
                self.enc_route_margin[l] = np.concatenate([self.enc_route_margin[l][:start],
                                                           rt[2]])
            self.K[l] = k if kc is None else np.concatenate([kc, k], axis=1)
            self.V[l] = v if vc is None else np.concatenate([vc, v], axis=1)
        self.n_ctx = start + len(ids)

    def prefill(self, ids):
        self.K = [None] * self.L
        self.V = [None] * self.L
        self.enc_route_margin = [np.zeros(0) for _ in range(self.L)]
        self.k_blk = 0
        self._encode(ids, 0)

    def commit(self, canvas):
        self._encode(canvas, self.n_ctx)
        self.k_blk += 1

    # ------------------------------------------------------------ stage 2
    def decoder_layer(self, l: int, h):
        """One decoder layer over the canvas rows h [C, d] (positions n_ctx..n_ctx+C-1,
        bidirectional over the context cache and the canvas).  Returns (h, routing)."""
        C = h.shape[0]
        positions = np.arange(self.n_ctx, self.n_ctx + C)
        ctx_pos = np.arange(self.n_ctx)
        kc = self.K[l] if self.n_ctx > 0 else None
        vc = self.V[l] if self.n_ctx > 0 else None
        h, _, _, rt = self._layer(l, h, positions, kc, vc, causal=False, ctx_pos=ctx_pos)
        return h, rt

    def head_logits(self, h):
        """Final RMSNorm and the tied LM head: logits [C, V] (before the temperature)."""
        hn = self._act(rmsnorm(h, self.w.rms_eps))
        return hn @ self.W.embed().T

    def decoder_logits(self, canvas, z_in=None):
        """Logits of the canvas; z_in [C, d] is the self-conditioning signal added to the
        token embedding (None: zero)."""
        h = self.W.embed()[np.asarray(canvas)]
        if z_in is not None:
            h = h + np.asarray(z_in, np.float64)
        routes = []
        hidden = []
        for l in range(self.L):
            h, rt = self.decoder_layer(l, h)
            routes.append(rt)
            if self.capture_hidden:
                hidden.append(h.copy())
        return self.head_logits(h), routes, hidden

    def next_signal(self, z) -> SelfCond:
        """Self-conditioning signal for the next pass from the tempered logits z."""
        W = self.W
        return next_signal(z, W.embed(), W.dense("sc_wg"), W.dense("sc_wu"), W.dense("sc_wd"),
                           self.bf16)

    def denoise_step(self, canvas, mask, s: int, T: int, seed: int, keep_logits=False,
                     row0: int = 0, z_in=None, want_signal: bool | None = None):
        """One pass over the canvas at positions n_ctx..n_ctx+C-1.  row0 offsets the rows
        its Gumbel uniforms are drawn for (canvas b of a batch draws as rows b C ..).
        z_in: the self-conditioning signal of this pass (None: zero); with the
        self-conditioning block the result carries the next pass's signal (.sc) unless
        want_signal is False."""
        w = self.w
        logits, routes, hidden = self.decoder_logits(canvas, z_in)
        z = logits / w.temperature
        st = lm_head_stats(z)
        C = len(canvas)
        redraw = np.full(C, -1, np.int32)
        gap = np.full(C, np.nan)
        unlocked = np.flatnonzero(np.asarray(mask) == 0)
        if unlocked.size:
            chunk = max(1, (1 << 24) // w.vocab)
            for c0 in range(0, unlocked.size, chunk):
                pos = unlocked[c0:c0 + chunk]
                u = gumbel_uniforms(seed, self.k_blk, s, pos + row0, w.vocab)
                redraw[pos], gap[pos] = gumbel_draw(z[pos], u)
        sr = sampler_update(canvas, mask, st.conf, st.argmax, redraw, s, T)
        sc = None
        if w.self_cond and (want_signal if want_signal is not None else True):
            sc = self.next_signal(z)
        return StepResult(canvas=sr.canvas, mask=sr.mask, stats=st, redraw=redraw,
                          redraw_gap=gap, sampler=sr,
                          route_idx=[r[0] for r in routes], route_gates=[r[1] for r in routes],
                          route_margin=[r[2] for r in routes],
                          logits=z if keep_logits else None, hidden=hidden, sc=sc)

    def denoise_step_batch(self, canvases, masks, s: int, T: int, seed: int,
                           keep_logits=False, z_ins=None):
        """A batch of canvases continuing the same context at the same positions: each
        canvas is a pass of its own (it attends to the context and to itself only), the
        lock schedule runs per canvas, and canvas b draws its Gumbel uniforms as rows
        b C .. b C + C - 1 of one long canvas.  z_ins: per canvas self-conditioning
        signal (None: zero).  Returns one StepResult per canvas."""
        C = self.w.canvas
        zs = z_ins if z_ins is not None else [None] * len(canvases)
        return [self.denoise_step(c, m, s, T, seed, keep_logits=keep_logits, row0=b * C,
                                  z_in=zs[b])
                for b, (c, m) in enumerate(zip(canvases, masks))]

    def init_canvas_batch(self, seed: int, B: int):
        """The initial canvases of a batch: B C positions of one long canvas, [B, C]."""
        C = self.w.canvas
        return init_canvas(seed, self.k_blk, B * C, self.w.vocab).reshape(B, C)

    def _draws(self, z, mask, s: int, seed: int):
        C = z.shape[0]
        redraw = np.full(C, -1, np.int32)
        gap = np.full(C, np.nan)
        unlocked = np.flatnonzero(np.asarray(mask) == 0)
        chunk = max(1, (1 << 24) // self.w.vocab)
        for c0 in range(0, unlocked.size, chunk):
            pos = unlocked[c0:c0 + chunk]
            u = gumbel_uniforms(seed, self.k_blk, s, pos, self.w.vocab)
            redraw[pos], gap[pos] = gumbel_draw(z[pos], u)
        return redraw, gap

    def denoise_step_eb(self, canvas, mask, prev_argmax, s: int, p, seed: int,
                        keep_logits=False, z_in=None):
        """One pass of the entropy-bounded sampler (``eb_sampler``): logits tempered at
        tau_s, per-position entropy, Gumbel draws for unlocked positions, then the update.
        With the self-conditioning block, p0 of the next signal is tempered at tau_s too.
        Returns (StepResult, EbResult, entropies)."""
        logits, routes, _ = self.decoder_logits(canvas, z_in)
        z = logits / eb.tau_at(s, p)
        st = lm_head_stats(z)
        H = eb.entropy(z)
        redraw, gap = self._draws(z, mask, s, seed)
        er = eb.eb_update(canvas, mask, H, st.argmax, redraw, prev_argmax, s, p, seed,
                          self.k_blk, self.w.vocab)
        res = StepResult(canvas=er.canvas, mask=er.mask, stats=st, redraw=redraw,
                         redraw_gap=gap, sampler=None,
                         route_idx=[r[0] for r in routes], route_gates=[r[1] for r in routes],
                         route_margin=[r[2] for r in routes],
                         logits=z if keep_logits else None,
                         sc=self.next_signal(z) if self.w.self_cond else None)
        return res, er, H

    def generate_block_eb(self, p, seed: int, commit: bool = True, on_step=None):
        """Passes of the entropy-bounded sampler until it ends the block; returns
        (canvas, number of passes)."""
        w = self.w
        canvas = init_canvas(seed, self.k_blk, w.canvas, w.vocab)
        mask = np.zeros(w.canvas, np.uint8)
        prev = None
        n = 0
        zs = None
        for s in range(p.max_steps):
            res, er, H = self.denoise_step_eb(canvas, mask, prev, s, p, seed, z_in=zs)
            if on_step is not None:
                on_step(s, canvas, mask, res, er, H)
            canvas, mask, prev = er.canvas, er.mask, res.stats.argmax
            zs = res.sc.z if res.sc is not None else None
            n = s + 1
            if er.done:
                break
        if commit:
            self.commit(canvas)
        return canvas, n

    def generate_block(self, T: int, seed: int, commit: bool = True, on_step=None):
        w = self.w
        canvas = init_canvas(seed, self.k_blk, w.canvas, w.vocab)
        mask = np.zeros(w.canvas, np.uint8)
        zs = None
        for s in range(T):
            # the last pass's signal would feed no pass: it is not formed
            res = self.denoise_step(canvas, mask, s, T, seed, z_in=zs, want_signal=s < T - 1)
            if on_step is not None:
                on_step(s, canvas, mask, res)
            canvas, mask = res.canvas, res.mask
            zs = res.sc.z if res.sc is not None else None
        if commit:
            self.commit(canvas)
        return canvas
