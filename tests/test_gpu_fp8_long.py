"""GPU parity of the long-context, multi-canvas variant of the 26B-class denoiser with fp8
experts (e4m3 weights with per-output-column fp32 scales, fp8 MFMA; attention and
activations in bf16), prompt P = 131072, truncated to layer 0:

  * prompt K/V of layer 0 at 64 sampled positions of the 131072 against the oracle's
    stored values (tests/golden/moe26b_fp8_long_1layer.npz), and the canvas init;
  * canvas 0, pass 0, stage by stage: the attention output against the oracle's attention
    of the canvas queries over the GPU's cache (131328 keys), the layer output against the
    oracle's output projection + MoE on the GPU's attention output, and the LM head,
    statistics and decisions against the oracle head on the GPU's layer output;
  * commit of the oracle's canvas-0 output (K/V appended at P..P+C-1), then canvas 1 (block
    index 1), pass 0, the same way: the canvas attends to the prompt and to the committed
    canvas.

Continuous values use the fp8 tolerance (2e-2 absolute + 5e-2 relative) or the bf16 one
for the bf16 attention output; decisions are exact outside the decision gate.  End to end
(against the stored oracle pass) the logit differences are logged: a bf16 rounding flip of
a normed activation moves its e4m3 code by a whole step (12.5 %) for ~1 in 15 of the
flipped elements, so element-wise end-to-end agreement is not a property fp8 inputs keep.
"""
import os

import numpy as np
import pytest
import torch

import fixtures as fx
from fixtures.dg_glue import build_handle
from parity import GATE, TOL, assert_close, routing_sets, worst_mismatch_margin
from parity import gated_mismatches as _gated
from parity import lock_set_check as _lock_check
from gpu_util import (i32_dev, kv_read, log, logits_capture, need_gpu, routing_capture,
                      stats_capture, u8_dev)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "moe26b_fp8_long_1layer.npz")
W = fx.MOE26B_FP8_LONG.with_(name="moe26b_fp8_long_1layer", n_layers=1)
DELTA = GATE["fp8"]


def gated_mismatches(gpu, ref, margin):
    bad, n, in_band = _gated(gpu, ref, margin, DELTA)
    if in_band or bad:
        log(f"disagreements {bad + in_band}, largest oracle margin among them "
            f"{worst_mismatch_margin(gpu, ref, margin):.4f} (gate {DELTA})")
    return bad, n, in_band


@pytest.fixture(scope="module")
def env():
    dg = need_gpu()
    g = dict(np.load(GOLDEN))
    log("building the 1-layer fp8-expert model, prompt 131072")
    caps = dg.DG_CAP_LOGITS | dg.DG_CAP_STATS | dg.DG_CAP_ROUTING
    h = build_handle(dg, W, capture_mask=caps, max_ctx=W.prompt_len + W.n_canvases * W.canvas)
    dg.dg_prefill_prompt_kv(h, i32_dev(fx.prompt_ids(W)), W.prompt_len)
    torch.cuda.synchronize()
    log("prefilled")
    yield dg, h, g
    dg.dg_destroy(h)


def test_prefill_kv_samples(env):
    dg, h, g = env
    pos = g["kv_pos"]
    for which, key in ((0, "k_0"), (1, "v_0")):
        full = kv_read(dg, h, 0, which, 0, W.prompt_len, W.n_kv_heads, W.head_dim, torch.bfloat16)
        assert_close(key, full[:, pos, :], g[key], *TOL["bf16"])


def _oracle():
    from oracle.model import OracleModel
    from oracle.weights import FixtureWeights
    return OracleModel(W, FixtureWeights(W))


def _check_pass(dg, h, g, m, b):
    """Canvas b, pass 0: GPU pass, then each stage against the oracle on the GPU's input."""
    from oracle.model import attention, lm_head_stats, sampler_update, gumbel_draw
    from oracle.numerics import rmsnorm
    from oracle.philox import gumbel_uniforms
    C, k, d = W.canvas, W.top_k, W.d_model
    canvas = torch.empty(C, dtype=torch.int32, device="cuda")
    mask = torch.empty(C, dtype=torch.uint8, device="cuda")
    dg.dg_init_canvas(h, canvas, mask, int(g["seed"]))
    torch.cuda.synchronize()
    cin = canvas.cpu().numpy().copy()
    assert np.array_equal(cin, g[f"b{b}_canvas_in"]), "canvas init differs"
    mask_in = mask.cpu().numpy().copy()
    n_ctx, _ = dg.dg_get_state(h)
    dg.dg_denoise_step(h, canvas, mask, 0, int(g["T"]), int(g["seed"]))
    torch.cuda.synchronize()
    attn = torch.empty(C, W.n_q_heads * W.head_dim, dtype=torch.bfloat16, device="cuda")
    dg.dg_get_capture(h, dg.DG_CAP_ATTN, 0, attn)
    hid = torch.empty(C, d, dtype=torch.float32, device="cuda")
    dg.dg_get_capture(h, dg.DG_CAP_HIDDEN, 0, hid)
    torch.cuda.synchronize()
    attn = attn.float().cpu().numpy().astype(np.float64)
    hid = hid.cpu().numpy().astype(np.float64)
    gi, _ = routing_capture(dg, h, 0, C, k)
    z = logits_capture(dg, h, C, W.vocab)
    st = stats_capture(dg, h, C)

    # attention: canvas queries over the GPU's cache rows (prompt, committed canvases, canvas)
    Kc = kv_read(dg, h, 0, 0, 0, n_ctx + C, W.n_kv_heads, W.head_dim, torch.bfloat16)
    Vc = kv_read(dg, h, 0, 1, 0, n_ctx + C, W.n_kv_heads, W.head_dim, torch.bfloat16)
    x0 = m.W.embed()[cin]
    a = m._act(rmsnorm(x0, W.rms_eps))
    q, _, _ = m._qkv(0, a, np.arange(n_ctx, n_ctx + C))
    o = m._act(attention(q, Kc, Vc).transpose(1, 0, 2).reshape(C, -1))
    del Kc, Vc
    err = assert_close("attention output", attn, o, *TOL["bf16"])
    log(f"canvas {b}: attention over {n_ctx + C} keys, max abs err {err:.3g}")

    # output projection + MoE on the GPU's attention output
    h1 = x0 + attn @ m.W.dense("wo", 0)
    bn = m._act(rmsnorm(h1, W.rms_eps))
    y, ridx, _, margin = m._moe(0, bn)
    gs, rs = routing_sets(gi), routing_sets(ridx)
    bad, n, _ = gated_mismatches(gs, rs, margin)
    assert bad == 0, f"{bad} of {n} gated routing decisions differ"
    ok = ~np.any(gs != rs, axis=1)
    err = assert_close("layer output", hid[ok], (h1 + y)[ok], *TOL["fp8"])
    log(f"canvas {b}: layer output max abs err {err:.3g}, in-band routing rows {int((~ok).sum())}")

    # LM head and statistics on the GPU's layer output
    zr = m.head_logits(hid) / W.temperature
    rows, cols = g[f"b{b}_logit_rows"], g[f"b{b}_logit_cols"]
    zs = z[torch.from_numpy(rows).long().cuda(), torch.from_numpy(cols).long().cuda()].cpu().numpy()
    err = assert_close("logits", zs, zr[rows, cols], *TOL["fp8"])
    e2e = np.abs(zs - g[f"b{b}_logit_vals"])
    log(f"canvas {b}: head logits max abs err {err:.3g}; end to end vs the stored oracle pass: "
        f"median {np.median(e2e):.3g}, p99 {np.quantile(e2e, 0.99):.3g}, max {e2e.max():.3g}")
    sr = lm_head_stats(zr)
    for key in ("m", "lse", "conf"):
        assert_close(key, st[key], getattr(sr, key), *TOL["fp8"])
    bad, n, _ = gated_mismatches(st["argmax"], sr.argmax, sr.top2_gap)
    assert bad == 0, f"{bad} of {n} gated argmax decisions differ"
    # redraws of 32 positions (the Gumbel noise of all 256 x 262144 would dominate the run)
    pos = np.arange(0, C, 8)
    red, gap = gumbel_draw(zr[pos], gumbel_uniforms(int(g["seed"]), b, 0, pos, W.vocab))
    bad, n, _ = gated_mismatches(st["redraw"][pos], red, gap)
    assert bad == 0, f"{bad} of {n} gated redraws differ"
    ref = sampler_update(cin, mask_in, sr.conf, st["argmax"], st["redraw"], 0, int(g["T"]))
    _lock_check(mask.cpu().numpy(), ref.mask, mask_in, sr.conf, ref.cut_low, ref.cut_high,
                delta=DELTA)


def test_canvas0_then_commit_then_canvas1(env):
    dg, h, g = env
    caps = dg.DG_CAP_LOGITS | dg.DG_CAP_STATS | dg.DG_CAP_ROUTING | dg.DG_CAP_HIDDEN | dg.DG_CAP_ATTN
    dg.dg_set_capture(h, caps)
    m = _oracle()
    _check_pass(dg, h, g, m, 0)
    dg.dg_commit_canvas(h, i32_dev(g["commit_tokens"]))
    torch.cuda.synchronize()
    n_ctx, k_blk = dg.dg_get_state(h)
    assert (n_ctx, k_blk) == (W.prompt_len + W.canvas, 1)
    _check_pass(dg, h, g, m, 1)
