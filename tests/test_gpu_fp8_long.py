"""GPU parity of the long-context, multi-canvas variant of the 26B-class denoiser with fp8
experts (e4m3 weights with per-output-column fp32 scales, fp8 MFMA; attention and
activations in bf16), prompt P = 131072, truncated to layers 0-1:

  * prompt cache: layer 0 at 64 sampled positions of the 131072, and layer 1 at the same
    positions (the oracle runs layer 0 at those rows against its whole layer-0 cache),
    against tests/golden/moe26b_fp8_long_2layer.npz; layer-1 rows are compared where the
    row's layer-0 routing is not a near tie;
  * canvas 0, pass 0, stage by stage, each stage on the GPU's own input: per layer the
    attention output (canvas queries over the GPU's cache, 131328 keys) and the layer
    output (output projection + fp8 MoE on the GPU's attention output); then the LM head,
    statistics and decisions on the GPU's final residual stream;
  * canvas 0, pass 0, end to end: the oracle from the embeddings through both layers over
    the GPU's context cache, gated decisions exact, logits within a statistical bound;
  * commit of block 0's initial canvas: the appended cache rows of both layers against the
    oracle's (sampled rows);
  * canvas 1 (block index 1), pass 0, stage by stage and end to end: the canvas attends to
    the prompt and to the committed canvas.

Continuous values use the fp8 tolerance (2e-2 absolute + 5e-2 relative) or the bf16 one
for the bf16 attention output and cache rows; decisions on a stage's own input are exact
outside the 1e-2 gate.  Comparisons across fp8 layers assert the measured noise envelope
of e4m3 inputs (see E2E_* below), decisions end to end outside a 0.25 gate.  In-band counts and the
end-to-end error quantiles go to the parity record moe26b_fp8_long_2layer.
"""
import os

import numpy as np
import pytest
import torch

import fixtures as fx
from fixtures.dg_glue import build_handle
from parity import E2E_GATE, GATE, TOL, assert_close, routing_sets, worst_mismatch_margin
from parity import gated_mismatches as _gated
from parity import lock_set_check as _lock_check
from gpu_util import (i32_dev, kv_read, log, logits_capture, need_gpu, record, routing_capture,
                      stats_capture)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "moe26b_fp8_long_2layer.npz")
W = fx.MOE26B_FP8_LONG.with_(name="moe26b_fp8_long_2layer", n_layers=2)
DELTA = GATE["fp8"]
DELTA_E2E = E2E_GATE["fp8"]
# a layer-1 cache row is compared where its token's layer-0 routing is no near tie; that
# routing sits upstream of any fp8 layer, so the bf16 end-to-end gate applies to it
DELTA_ROUTE0 = E2E_GATE["bf16"]
# End to end, fp8 inputs amplify upstream rounding differences: an expert input or a
# SwiGLU output that differs at bf16-rounding level crosses an e4m3 rounding boundary for
# about 1 in 15 elements and then moves by a whole code step (12.5 %).  Every stage meets
# the fp8 bound on every element on its own input; comparisons across fp8 layers assert
# the noise envelope measured on this workload (both canvases):
#   * cache rows after one fp8 layer: 94.5-97.4 % within the bound, at most 3.8 x it;
#   * logits after two fp8 layers: 73.8-74.1 % within the bound, at most 7.5 x it;
#   * decisions: the largest disagreeing oracle margin was 0.152 (gate 0.25).
E2E_KV_FRAC, E2E_KV_CAP = 0.90, 5.0
E2E_LOGIT_FRAC, E2E_LOGIT_CAP = 0.70, 10.0
REC = {}


def gated(gpu, ref, margin, delta=DELTA):
    bad, n, in_band = _gated(gpu, ref, margin, delta)
    if in_band or bad:
        log(f"disagreements {bad + in_band}, largest oracle margin among them "
            f"{worst_mismatch_margin(gpu, ref, margin):.4f} (gate {delta})")
    return bad, n, in_band


@pytest.fixture(scope="module")
def env():
    dg = need_gpu()
    g = dict(np.load(GOLDEN))
    log("building the 2-layer fp8-expert model, prompt 131072")
    caps = dg.DG_CAP_LOGITS | dg.DG_CAP_STATS | dg.DG_CAP_ROUTING
    h = build_handle(dg, W, capture_mask=caps, max_ctx=W.prompt_len + W.n_canvases * W.canvas)
    dg.dg_prefill_prompt_kv(h, i32_dev(fx.prompt_ids(W)), W.prompt_len)
    torch.cuda.synchronize()
    log("prefilled")
    yield dg, h, g
    record("moe26b_fp8_long_2layer", REC)
    dg.dg_destroy(h)


def _kv_stats(name, got, ref):
    """Error figures of cache rows compared end to end through an fp8 layer."""
    err = np.abs(got - ref)
    bound = TOL["fp8"][0] + TOL["fp8"][1] * np.abs(ref)
    bf = TOL["bf16"][0] + TOL["bf16"][1] * np.abs(ref)
    return {"name": name, "n": int(err.size), "median": float(np.median(err)),
            "p99": float(np.quantile(err, 0.99)), "max": float(err.max()),
            "frac_within_bf16_bound": float(np.mean(err <= bf)),
            "frac_within_fp8_bound": float(np.mean(err <= bound)),
            "max_over_fp8_bound": float((err / bound).max())}


def _kv_e2e(name, got, ref):
    st = _kv_stats(name, got, ref)
    REC.setdefault("cache_rows_end_to_end", []).append(st)
    log(f"{name}: {st}")
    return [(f"{name} within the bound on {E2E_KV_FRAC:.0%}",
             st["frac_within_fp8_bound"] >= E2E_KV_FRAC),
            (f"{name} within {E2E_KV_CAP}x the bound", st["max_over_fp8_bound"] <= E2E_KV_CAP)]


def test_prefill_kv_samples(env):
    """Layer-0 rows depend on the embedded prompt only: the bf16 bound on every element.
    Layer-1 rows hold one fp8 MoE layer (and 131072-key causal attention) of difference:
    the end-to-end form of the fp8 bound."""
    dg, h, g = env
    pos = g["kv_pos"]
    trusted = g["kv_margin0"] > DELTA_ROUTE0
    REC["prefill_layer1_rows_compared"] = int(trusted.sum())
    for which, key in ((0, "k"), (1, "v")):
        full = kv_read(dg, h, 0, which, 0, W.prompt_len, W.n_kv_heads, W.head_dim, torch.bfloat16)
        assert_close(f"layer 0 {key}", full[:, pos, :], g[f"{key}_0"], *TOL["bf16"])
    checks = []
    for which, key in ((0, "k"), (1, "v")):
        full = kv_read(dg, h, 1, which, 0, W.prompt_len, W.n_kv_heads, W.head_dim, torch.bfloat16)
        checks += _kv_e2e(f"prefill layer 1 {key}", full[:, pos[trusted], :],
                          g[f"{key}_1"][:, trusted, :])
    failed = [name for name, good in checks if not good]
    assert not failed, failed


def _capture(dg, h, what, layer, shape, dtype):
    t = torch.empty(*shape, dtype=dtype, device="cuda")
    dg.dg_get_capture(h, what, layer, t)
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64)


def _check_pass(dg, h, g, m, b):
    """Canvas b, pass 0: the GPU pass, each stage against the oracle on the GPU's input of
    that stage, then the oracle end to end over the GPU's context cache."""
    from oracle.model import attention, gumbel_draw, lm_head_stats, sampler_update
    from oracle.numerics import rmsnorm
    from oracle.philox import gumbel_uniforms
    C, k, d, L = W.canvas, W.top_k, W.d_model, W.n_layers
    rec = REC.setdefault(f"canvas{b}", {"stage": [], "gate": DELTA, "gate_e2e": DELTA_E2E})
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
    attn = [_capture(dg, h, dg.DG_CAP_ATTN, l, (C, W.n_q_heads * W.head_dim), torch.bfloat16)
            for l in range(L)]
    hid = [_capture(dg, h, dg.DG_CAP_HIDDEN, l, (C, d), torch.float32) for l in range(L)]
    routes = [routing_capture(dg, h, l, C, k)[0] for l in range(L)]
    z = logits_capture(dg, h, C, W.vocab)
    st = stats_capture(dg, h, C)
    positions = np.arange(n_ctx, n_ctx + C)

    m.n_ctx = n_ctx
    e2e_route_bad = 0
    x = m.W.embed()[cin]
    for l in range(L):
        # attention of the canvas queries over the GPU's cache (context and canvas rows)
        Kc = kv_read(dg, h, l, 0, 0, n_ctx + C, W.n_kv_heads, W.head_dim, torch.bfloat16)
        Vc = kv_read(dg, h, l, 1, 0, n_ctx + C, W.n_kv_heads, W.head_dim, torch.bfloat16)
        a = m._act(rmsnorm(x, W.rms_eps))
        q, _, _ = m._qkv(l, a, positions)
        o = m._act(attention(q, Kc, Vc).transpose(1, 0, 2).reshape(C, -1))
        # the canvas's own cache rows of this layer, from the GPU's layer input
        kr, vr = m.kv_rows(l, a, positions)
        assert_close(f"layer {l} canvas K rows", Kc[:, n_ctx:], kr, *TOL["bf16"])
        assert_close(f"layer {l} canvas V rows", Vc[:, n_ctx:], vr, *TOL["bf16"])
        m.K[l], m.V[l] = Kc[:, :n_ctx], Vc[:, :n_ctx]     # the context, for the end-to-end run
        del Kc, Vc
        err_a = assert_close(f"layer {l} attention output", attn[l], o, *TOL["bf16"])
        # output projection + MoE on the GPU's attention output
        h1 = x + attn[l] @ m.W.dense("wo", l)
        bn = m._act(rmsnorm(h1, W.rms_eps))
        y, ridx, _, margin = m._moe(l, bn)
        gs, rs = routing_sets(routes[l]), routing_sets(ridx)
        bad, n, in_band = gated(gs, rs, margin)
        assert bad == 0, f"layer {l}: {bad} of {n} gated routing decisions differ"
        ok = ~np.any(gs != rs, axis=1)
        err = assert_close(f"layer {l} output", hid[l][ok], (h1 + y)[ok], *TOL["fp8"])
        rec["stage"].append({"layer": l, "attention_max_abs_err": err_a, "output_max_abs_err": err,
                             "routing_in_band": in_band, "routing_gated": n})
        log(f"canvas {b} layer {l}: attention over {n_ctx + C} keys max abs err {err_a:.3g}, "
            f"output max abs err {err:.3g}, in-band routing rows {int((~ok).sum())}")
        x = hid[l]

    # LM head and statistics on the GPU's final residual stream
    zr = m.head_logits(x) / W.temperature
    rng = np.random.default_rng(20264 + b)
    rows = np.concatenate([rng.integers(0, C, 16384), np.arange(C)])
    cols = np.concatenate([rng.integers(0, W.vocab, 16384), st["argmax"]])
    zs = z[torch.from_numpy(rows).long().cuda(), torch.from_numpy(cols).long().cuda()].cpu().numpy()
    err = assert_close("logits", zs, zr[rows, cols], *TOL["fp8"])
    sr = lm_head_stats(zr)
    for key in ("m", "lse", "conf"):
        assert_close(key, st[key], getattr(sr, key), *TOL["fp8"])
    bad, n, in_band = gated(st["argmax"], sr.argmax, sr.top2_gap)
    assert bad == 0, f"{bad} of {n} gated argmax decisions differ"
    rec["head"] = {"logits_max_abs_err": err, "argmax_in_band": in_band, "argmax_gated": n}
    # redraws of 32 positions (the Gumbel noise of all 256 x 262144 would dominate the run)
    pos = np.arange(0, C, 8)
    red, gap = gumbel_draw(zr[pos], gumbel_uniforms(int(g["seed"]), b, 0, pos, W.vocab))
    bad, n, in_band = gated(st["redraw"][pos], red, gap)
    assert bad == 0, f"{bad} of {n} gated redraws differ"
    rec["head"].update(redraw_in_band=in_band, redraw_gated=n)
    ref = sampler_update(cin, mask_in, sr.conf, st["argmax"], st["redraw"], 0, int(g["T"]))
    rec["head"]["lock_in_band"] = _lock_check(mask.cpu().numpy(), ref.mask, mask_in, sr.conf,
                                              ref.cut_low, ref.cut_high, delta=DELTA)
    log(f"canvas {b}: head logits max abs err {err:.3g}")

    # end to end: the oracle from the embeddings over the GPU's context cache
    xe = m.W.embed()[cin]
    affected = np.zeros(C, bool)
    for l in range(L):
        xe, (ri, _, margin) = m.decoder_layer(l, xe)
        gs, rs = routing_sets(routes[l]), routing_sets(ri)
        keep = ~affected
        bad, n, in_band = gated(gs[keep], rs[keep], margin[keep], DELTA_E2E)
        e2e_route_bad += bad
        affected |= np.any(gs != rs, axis=1)
        diff_rows = np.any(gs != rs, axis=1) & keep
        rec.setdefault("e2e_routing_largest_disagreeing_margin", []).append(
            float(margin[diff_rows].max(initial=0.0)))
        rec.setdefault("e2e_routing", []).append({"layer": l, "in_band": in_band, "gated": n,
                                                  "rows_affected": int(affected.sum())})
    ze = m.head_logits(xe) / W.temperature
    ok = ~affected
    se = lm_head_stats(ze)
    sel = ok[rows]
    diff = np.abs(zs[sel] - ze[rows, cols][sel])
    bound = TOL["fp8"][0] + TOL["fp8"][1] * np.abs(ze[rows, cols][sel])
    bad, n, in_band = gated(st["argmax"][ok], se.argmax[ok], se.top2_gap[ok], DELTA_E2E)
    dis = st["argmax"][ok] != se.argmax[ok]
    rec["end_to_end"] = {"rows_unaffected": int(ok.sum()),
                         "logit_err_median": float(np.median(diff)),
                         "logit_err_p99": float(np.quantile(diff, 0.99)),
                         "logit_err_max": float(diff.max()),
                         "logit_err_max_over_bound": float((diff / bound).max()),
                         "frac_within_bound": float(np.mean(diff <= bound)),
                         "argmax_in_band": in_band, "argmax_gated": n, "argmax_gated_bad": bad,
                         "argmax_largest_disagreeing_margin":
                             float(se.top2_gap[ok][dis].max(initial=0.0))}
    log(f"canvas {b} end to end: {rec['end_to_end']}")
    rec["end_to_end"]["routing_gated_bad"] = e2e_route_bad
    return [(f"canvas {b}: end-to-end gated routing", e2e_route_bad == 0),
            (f"canvas {b}: end-to-end gated argmax", bad == 0),
            (f"canvas {b}: end-to-end logits within the bound on {E2E_LOGIT_FRAC:.0%}",
             np.mean(diff <= bound) >= E2E_LOGIT_FRAC),
            (f"canvas {b}: end-to-end logits within {E2E_LOGIT_CAP}x the bound",
             bool(np.all(diff <= E2E_LOGIT_CAP * bound)))]


def _oracle():
    from oracle.model import OracleModel
    from oracle.weights import FixtureWeights
    m = OracleModel(W, FixtureWeights(W, cache_experts=False))
    m.K, m.V = [None] * W.n_layers, [None] * W.n_layers
    return m


def test_canvas0_commit_canvas1(env):
    dg, h, g = env
    caps = dg.DG_CAP_LOGITS | dg.DG_CAP_STATS | dg.DG_CAP_ROUTING | dg.DG_CAP_HIDDEN | dg.DG_CAP_ATTN
    dg.dg_set_capture(h, caps)
    m = _oracle()
    checks = _check_pass(dg, h, g, m, 0)      # end-to-end checks, asserted at the end
    m.k_blk = 1
    # commit of block 0's initial canvas: the appended rows of both layers
    dg.dg_commit_canvas(h, i32_dev(g["commit_tokens"]))
    torch.cuda.synchronize()
    n_ctx, k_blk = dg.dg_get_state(h)
    assert (n_ctx, k_blk) == (W.prompt_len + W.canvas, 1)
    rows = g["commit_rows"]
    trusted = g["commit_margin0"] > DELTA_ROUTE0
    REC["commit_layer1_rows_compared"] = int(trusted.sum())
    for which, key in ((0, "k"), (1, "v")):
        got = kv_read(dg, h, 0, which, W.prompt_len, W.canvas, W.n_kv_heads, W.head_dim,
                      torch.bfloat16)
        assert_close(f"commit layer 0 {key}", got[:, rows], g[f"commit_{key}_0"], *TOL["bf16"])
        got = kv_read(dg, h, 1, which, W.prompt_len, W.canvas, W.n_kv_heads, W.head_dim,
                      torch.bfloat16)
        checks += _kv_e2e(f"commit layer 1 {key}", got[:, rows[trusted]],
                          g[f"commit_{key}_1"][:, trusted])
    log("commit rows of layer 0 match")
    checks += _check_pass(dg, h, g, m, 1)
    failed = [name for name, good in checks if not good]
    assert not failed, failed
