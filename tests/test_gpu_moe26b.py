"""GPU parity of the 26B-class bf16 MoE denoiser at full widths (d=2816, 128 experts top-8,
V=262144, P=8192).

  * layers 0-1 (the model truncated to its first two layers): prefill K/V samples, canvas
    init, pass 0 and pass 1 (teacher-forced from the oracle's state) against the oracle's
    stored values in tests/golden/moe26b_2layer.npz, end to end;
  * the same passes stage by stage: each layer and the LM head against the oracle run on
    the GPU's own input to that stage (the oracle's prompt cache computed on the host);
  * all 30 layers: one whole 12-pass block checked by the properties that hold at any size
    (lock schedule, locked tokens never change, all locked at the end, finite statistics,
    determinism of a repeated pass).
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

DELTA = GATE["bf16"]          # stage by stage: decisions on the GPU's own stage input
DELTA_E2E = E2E_GATE["bf16"]  # end to end through bf16 layers
E2E_BAD_FRAC = 1e-3   # end-to-end logits: fraction of samples allowed past the stated bound
E2E_CAP = 3.0         # end-to-end logits: every sample within this multiple of the bound


def gated_mismatches(gpu, ref, margin, delta=DELTA):
    bad, n, in_band = _gated(gpu, ref, margin, delta)
    if in_band or bad:
        log(f"disagreements {bad + in_band}, largest oracle margin among them "
            f"{worst_mismatch_margin(gpu, ref, margin):.4f} (gate {delta})")
    return bad, n, in_band


def lock_set_check(*args, delta=DELTA):
    return _lock_check(*args, delta=delta)
from gpu_util import (i32_dev, kv_read, log, logits_capture, need_gpu, record,
                      routing_capture, stats_capture, u8_dev)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "moe26b_2layer.npz")
W2 = fx.MOE26B.with_(name="moe26b_2layer", n_layers=2)


@pytest.fixture(scope="module")
def env2():
    dg = need_gpu()
    g = dict(np.load(GOLDEN))
    log("building the 2-layer full-width model")
    caps = dg.DG_CAP_LOGITS | dg.DG_CAP_STATS | dg.DG_CAP_ROUTING
    h = build_handle(dg, W2, capture_mask=caps)
    dg.dg_prefill_prompt_kv(h, i32_dev(fx.prompt_ids(W2)), W2.prompt_len)
    torch.cuda.synchronize()
    log("prefilled")
    yield dg, h, g
    dg.dg_destroy(h)


def test_prefill_kv_samples(env2):
    dg, h, g = env2
    pos = g["kv_pos"]
    # layer-1 rows depend on the token's layer-0 routing: compare the rows whose routing
    # margin in the oracle exceeds the decision gate
    trusted = {0: np.ones(pos.size, bool), 1: g["kv_margin0"] > DELTA_E2E}
    for l in range(W2.n_layers):
        for which, key in ((0, "k"), (1, "v")):
            full = kv_read(dg, h, l, which, 0, W2.prompt_len, W2.n_kv_heads, W2.head_dim,
                           torch.bfloat16)
            sel = trusted[l]
            assert_close(f"layer {l} {key}", full[:, pos[sel], :], g[f"{key}_{l}"][:, sel, :],
                         *TOL["bf16"])


@pytest.fixture(scope="module")
def forced(env2):
    """Teacher forcing of the prompt cache: the GPU gets the oracle's prompt K/V (computed
    here on the host, the same prefill the stored pass values were computed from), so a
    near-tie routing that the two prefills resolve differently cannot leak into the passes."""
    from oracle.model import OracleModel
    from oracle.weights import FixtureWeights

    dg, h, g = env2
    log("oracle prefill of the 2-layer model on the host")
    oracle = OracleModel(W2, FixtureWeights(W2))
    oracle.prefill(fx.prompt_ids(W2))
    log("oracle prefill done")
    for l in range(W2.n_layers):
        for which, ref in ((0, oracle.K[l]), (1, oracle.V[l])):
            src = torch.from_numpy(np.ascontiguousarray(ref.astype(np.float32))).to(torch.bfloat16).cuda()
            dg.dg_set_kv(h, l, which, 0, W2.prompt_len, src)
    torch.cuda.synchronize()
    return dg, h, g, oracle


def test_canvas_init(env2):
    dg, h, g = env2
    c = torch.empty(W2.canvas, dtype=torch.int32, device="cuda")
    dg.dg_init_canvas(h, c, None, int(g["seed"]))
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), g["canvas_in_0"])


@pytest.mark.parametrize("s", [0, 1])
def test_pass(forced, s):
    dg, h, g, _ = forced
    canvas, mask = g[f"canvas_in_{s}"], g[f"mask_in_{s}"]
    cd, md = i32_dev(canvas), u8_dev(mask)
    log(f"pass {s}")
    dg.dg_denoise_step(h, cd, md, s, int(g["T"]), int(g["seed"]))
    torch.cuda.synchronize()
    p = f"s{s}"
    C, k = W2.canvas, W2.top_k
    # routing: gated decisions exact; rows with an in-band difference are excluded below
    affected = np.zeros(C, bool)
    for l in range(W2.n_layers):
        gi, _ = routing_capture(dg, h, l, C, k)
        gi, ri = routing_sets(gi), routing_sets(g[f"{p}_route_idx_{l}"])
        # rows whose routing already differed upstream (in band) carry other inputs here
        keep = ~affected
        bad, n, in_band = gated_mismatches(gi[keep], ri[keep], g[f"{p}_route_margin_{l}"][keep],
                                         DELTA_E2E)
        assert bad == 0, f"layer {l}: {bad} of {n} gated routing decisions differ"
        affected |= np.any(gi != ri, axis=1)
    log(f"positions with in-band routing differences: {int(affected.sum())}")
    ok = ~affected
    z = logits_capture(dg, h, C, W2.vocab)
    rows, cols = g[f"{p}_logit_rows"], g[f"{p}_logit_cols"]
    zs = z[torch.from_numpy(rows).long().cuda(), torch.from_numpy(cols).long().cuda()].cpu().numpy()
    sel = ok[rows]
    # end to end through both layers: the stated bound on 99.9 % of the samples and
    # three times it on every sample (in-band bf16 rounding decisions accumulate over
    # the layers; the strict bound holds stage by stage, test_pass_stagewise)
    err = assert_close("logits", zs[sel], g[f"{p}_logit_vals"][sel], *TOL["bf16"],
                       max_bad_frac=E2E_BAD_FRAC)
    assert_close("logits (cap)", zs[sel], g[f"{p}_logit_vals"][sel],
                 *(E2E_CAP * t for t in TOL["bf16"]))
    log(f"logits max abs err {err:.3g}")
    st = stats_capture(dg, h, C)
    for key in ("m", "lse", "conf"):
        assert_close(key, st[key][ok], g[f"{p}_{key}"][ok], *TOL["bf16"])
    bad, n, _ = gated_mismatches(st["argmax"][ok], g[f"{p}_argmax"][ok], g[f"{p}_top2_gap"][ok],
                                 DELTA_E2E)
    assert bad == 0, f"{bad} of {n} gated argmax decisions differ"
    unl = (mask == 0) & ok
    bad, n, _ = gated_mismatches(st["redraw"][unl], g[f"{p}_redraw"][unl], g[f"{p}_redraw_gap"][unl],
                                 DELTA_E2E)
    assert bad == 0, f"{bad} of {n} gated redraws differ"
    mo, co = md.cpu().numpy(), cd.cpu().numpy()
    # the lock set is ranked over all positions: rows whose inputs legitimately differ
    # (in-band routing upstream) enter the reference ranking with the GPU's confidence
    from oracle.model import sampler_update
    conf_ref = np.where(ok, g[f"{p}_conf"], st["conf"])
    ref = sampler_update(canvas, mask, conf_ref, st["argmax"], st["redraw"], s, int(g["T"]))
    if ok.all():
        assert np.array_equal(ref.mask, g[f"{p}_mask_out"])
    lock_set_check(mo, ref.mask, mask, conf_ref, ref.cut_low, ref.cut_high, delta=DELTA_E2E)
    assert np.array_equal(co[mask == 1], canvas[mask == 1])


def hidden_capture(dg, h, layer, C, d):
    buf = torch.empty(C, d, dtype=torch.float32, device="cuda")
    dg.dg_get_capture(h, dg.DG_CAP_HIDDEN, layer, buf)
    torch.cuda.synchronize()
    return buf.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("s", [0, 1])
def test_pass_stagewise(forced, s):
    """Every stage of a pass against the oracle applied to the GPU's own input of that
    stage: layer 0 from the embeddings, layer 1 from the GPU's layer-0 output, the LM
    head and its statistics from the GPU's final residual stream.  The stated bounds
    hold here on every element; routing and argmax decisions are exact outside the gate."""
    dg, h, g, oracle = forced
    C, d, k = W2.canvas, W2.d_model, W2.top_k
    canvas, mask = g[f"canvas_in_{s}"], g[f"mask_in_{s}"]
    caps = dg.DG_CAP_LOGITS | dg.DG_CAP_STATS | dg.DG_CAP_ROUTING | dg.DG_CAP_HIDDEN
    dg.dg_set_capture(h, caps)
    try:
        dg.dg_denoise_step(h, i32_dev(canvas), u8_dev(mask), s, int(g["T"]), int(g["seed"]))
        torch.cuda.synchronize()
        hid = [hidden_capture(dg, h, l, C, d) for l in range(W2.n_layers)]
        z = logits_capture(dg, h, C, W2.vocab)
        st = stats_capture(dg, h, C)
        routes = [routing_capture(dg, h, l, C, k)[0] for l in range(W2.n_layers)]
    finally:
        dg.dg_set_capture(h, dg.DG_CAP_LOGITS | dg.DG_CAP_STATS | dg.DG_CAP_ROUTING)
    assert oracle.n_ctx == W2.prompt_len
    x = oracle.W.embed()[np.asarray(canvas)]
    for l in range(W2.n_layers):
        ref, (ri, _, margin) = oracle.decoder_layer(l, x)
        gi, ri = routing_sets(routes[l]), routing_sets(ri)
        bad, n, in_band = gated_mismatches(gi, ri, margin)
        assert bad == 0, f"layer {l}: {bad} of {n} gated routing decisions differ"
        ok = ~np.any(gi != ri, axis=1)
        err = assert_close(f"layer {l} residual stream", hid[l][ok], ref[ok], *TOL["bf16"])
        log(f"layer {l}: residual max abs err {err:.3g}, in-band routing rows {int((~ok).sum())}")
        x = hid[l]                                   # the next stage starts from the GPU's output
    zr = oracle.head_logits(x) / W2.temperature
    rows, cols = g[f"s{s}_logit_rows"], g[f"s{s}_logit_cols"]
    zs = z[torch.from_numpy(rows).long().cuda(), torch.from_numpy(cols).long().cuda()].cpu().numpy()
    err = assert_close("logits", zs, zr[rows, cols], *TOL["bf16"])
    log(f"head: logits max abs err {err:.3g}")
    from oracle.model import lm_head_stats
    sr = lm_head_stats(zr)
    for key in ("m", "lse", "conf"):
        assert_close(key, st[key], getattr(sr, key), *TOL["bf16"])
    bad, n, _ = gated_mismatches(st["argmax"], sr.argmax, sr.top2_gap)
    assert bad == 0, f"{bad} of {n} gated argmax decisions differ"


# ------------------------------------------------------------------ all 30 layers
@pytest.fixture(scope="module")
def env30():
    dg = need_gpu()
    w = fx.MOE26B
    log("building the 30-layer model (48 GB of bf16 weights)")
    h = build_handle(dg, w, capture_mask=dg.DG_CAP_STATS)
    log("loaded; prefilling 8192 prompt tokens")
    dg.dg_prefill_prompt_kv(h, i32_dev(fx.prompt_ids(w)), w.prompt_len)
    torch.cuda.synchronize()
    yield dg, h, w
    dg.dg_destroy(h)


def test_full_model_block_invariants(env30):
    dg, h, w = env30
    C, T = w.canvas, w.T
    cd = torch.empty(C, dtype=torch.int32, device="cuda")
    md = torch.empty(C, dtype=torch.uint8, device="cuda")
    dg.dg_init_canvas(h, cd, md, 11)
    for s in range(T):
        before_c, before_m = cd.cpu().numpy(), md.cpu().numpy()
        dg.dg_denoise_step(h, cd, md, s, T, 11)
        torch.cuda.synchronize()
        c, m = cd.cpu().numpy(), md.cpu().numpy()
        n_new = int(m.sum() - before_m.sum())
        assert n_new == (22 if s < T - 1 else 14), (s, n_new)
        assert np.array_equal(c[before_m == 1], before_c[before_m == 1])
        assert c.min() >= 0 and c.max() < w.vocab
        st = stats_capture(dg, h, C)
        assert np.all(np.isfinite(st["lse"])) and np.all(st["m"] <= st["lse"] + 1e-6)
        assert np.all(st["lse"] <= st["m"] + np.log(w.vocab) + 1e-3)
        log(f"30-layer pass {s}: {n_new} new locks, mean conf {st['conf'].mean():.3f}")
    assert int(md.sum()) == C
    dg.dg_check_finite(h)


def test_full_model_pass_is_deterministic(env30):
    dg, h, w = env30
    outs = []
    for _ in range(2):
        cd = torch.empty(w.canvas, dtype=torch.int32, device="cuda")
        md = torch.empty(w.canvas, dtype=torch.uint8, device="cuda")
        dg.dg_init_canvas(h, cd, md, 3)
        dg.dg_denoise_step(h, cd, md, 0, w.T, 3)
        st = stats_capture(dg, h, w.canvas)
        outs.append((cd.cpu().numpy(), md.cpu().numpy(), st["lse"], st["conf"]))
    assert all(np.array_equal(a, b) for a, b in zip(*outs))


def _kv_f64(dg, h, l, which, w):
    return kv_read(dg, h, l, which, 0, w.prompt_len, w.n_kv_heads, w.head_dim, torch.bfloat16)


def test_full_model_pass0_vs_oracle(env30, forced):
    """Pass 0 of the 30-layer model, the benched workload, against the oracle.

    Prompt cache: layers 0-1 from the oracle's own prefill (written into the GPU's cache as
    well), layers 2-29 teacher-forced from the GPU's prefill into the oracle (the oracle's
    own prefill of 30 layers over 8192 tokens is out of its reach).  Both sides then hold
    the same cache.

      * Graph and eager: the pass replayed as a HIP graph (the benched path) and launched
        one by one with per-layer captures give the same bits.
      * Stage by stage: each layer against the oracle run on the GPU's own input of that
        layer.  Gated routing decisions are exact, the experts hit per layer are the same
        set (the bench's algorithmic bytes count them), and the residual stream meets the
        bf16 bound on every element of the rows whose routing agrees.  The head, its
        statistics, gated argmax and redraw decisions, and the lock set are checked on the
        GPU's final residual stream.
      * End to end: the oracle from the embeddings through all 30 layers.  Gated routing
        decisions are exact on rows not already moved by an in-band difference upstream;
        gated argmax decisions are exact; the logits of those rows meet the bf16 bound on
        every sample.  These comparisons gate at 3e-2 (upstream bf16 storage decisions
        legitimately differ); the stage-by-stage ones at 1e-2.
    In-band counts and per-layer figures go to the parity record moe26b_30layer_pass0."""
    from oracle.model import OracleModel, gumbel_draw, lm_head_stats, sampler_update
    from oracle.philox import gumbel_uniforms, init_canvas

    dg, h, w = env30
    _, _, g, o2 = forced
    C, d, k, L, V = w.canvas, w.d_model, w.top_k, w.n_layers, w.vocab
    seed, T = int(g["seed"]), int(g["T"])
    for l in range(2):
        for which, ref in ((0, o2.K[l]), (1, o2.V[l])):
            src = torch.from_numpy(np.ascontiguousarray(ref.astype(np.float32))).to(torch.bfloat16).cuda()
            dg.dg_set_kv(h, l, which, 0, w.prompt_len, src)
    canvas = init_canvas(seed, 0, C, V)
    mask = np.zeros(C, np.uint8)

    # the benched path (graph replay), then the same pass eagerly with per-layer captures
    dg.dg_set_capture(h, dg.DG_CAP_STATS)
    cd, md = i32_dev(canvas), u8_dev(mask)
    dg.dg_denoise_step(h, cd, md, 0, T, seed)
    st_graph = stats_capture(dg, h, C)
    out_graph = (cd.cpu().numpy(), md.cpu().numpy())
    caps = dg.DG_CAP_LOGITS | dg.DG_CAP_STATS | dg.DG_CAP_ROUTING | dg.DG_CAP_HIDDEN
    dg.dg_set_capture(h, caps)
    try:
        cd, md = i32_dev(canvas), u8_dev(mask)
        dg.dg_denoise_step(h, cd, md, 0, T, seed)
        torch.cuda.synchronize()
        hid = [hidden_capture(dg, h, l, C, d) for l in range(L)]
        routes = [routing_capture(dg, h, l, C, k)[0] for l in range(L)]
        z = logits_capture(dg, h, C, V)
        st = stats_capture(dg, h, C)
        out = (cd.cpu().numpy(), md.cpu().numpy())
    finally:
        dg.dg_set_capture(h, dg.DG_CAP_STATS)
    for key in st:
        assert np.array_equal(st[key], st_graph[key]), f"graph and eager passes differ in {key}"
    assert all(np.array_equal(a, b) for a, b in zip(out, out_graph))
    log("30-layer pass 0: graph replay and eager launches agree bitwise")

    m = OracleModel(w, o2.W)           # the weight generator serves every layer
    m.n_ctx = w.prompt_len
    m.K, m.V = [None] * L, [None] * L
    rec = {"layers": [], "gate": DELTA}
    x = m.W.embed()[canvas]
    for l in range(L):
        if l < 2:
            m.K[l], m.V[l] = o2.K[l], o2.V[l]
        else:
            m.K[l], m.V[l] = _kv_f64(dg, h, l, 0, w), _kv_f64(dg, h, l, 1, w)
        ref, (ri, _, margin) = m.decoder_layer(l, x)
        gs, rs = routing_sets(routes[l]), routing_sets(ri)
        bad, n, in_band = _gated(gs, rs, margin, DELTA)
        assert bad == 0, f"layer {l}: {bad} of {n} gated routing decisions differ"
        ok = ~np.any(gs != rs, axis=1)
        hit_gpu, hit_ref = np.unique(routes[l]), np.unique(ri)
        # the expert sets agree over the rows whose routing agrees; rows with an in-band
        # difference may add or drop an expert only among their own k
        assert np.array_equal(np.unique(routes[l][ok]), np.unique(ri[ok])), f"layer {l}: experts hit"
        assert abs(hit_gpu.size - hit_ref.size) <= k * int((~ok).sum())
        err = assert_close(f"layer {l} residual stream", hid[l][ok], ref[ok], *TOL["bf16"])
        rec["layers"].append({"layer": l, "experts_hit_gpu": int(hit_gpu.size),
                              "experts_hit_oracle": int(hit_ref.size),
                              "largest_expert_rows": int(np.bincount(ri.ravel()).max()),
                              "routing_in_band": in_band, "routing_gated": n,
                              "residual_max_abs_err": err})
        log(f"layer {l}: experts hit {hit_gpu.size} (oracle {hit_ref.size}), residual max abs "
            f"err {err:.3g}, in-band routing rows {int((~ok).sum())}")
        x = hid[l]
        if l >= 2:
            m.W.forget_layer(l)
    zr = m.head_logits(x) / w.temperature
    rng = np.random.default_rng(20262)
    rows = np.concatenate([rng.integers(0, C, 16384), np.arange(C)])
    cols = np.concatenate([rng.integers(0, V, 16384), st["argmax"]])
    zi = (torch.from_numpy(rows).long().cuda(), torch.from_numpy(cols).long().cuda())
    zs = z[zi].cpu().numpy()
    err = assert_close("logits", zs, zr[rows, cols], *TOL["bf16"])
    sr = lm_head_stats(zr)
    for key in ("m", "lse", "conf"):
        assert_close(key, st[key], getattr(sr, key), *TOL["bf16"])
    bad, n, in_band = _gated(st["argmax"], sr.argmax, sr.top2_gap, DELTA)
    assert bad == 0, f"{bad} of {n} gated argmax decisions differ"
    rec["head"] = {"logits_max_abs_err": err, "argmax_in_band": in_band, "argmax_gated": n}
    pos = np.arange(0, C, 8)           # 32 redraws (the noise of every position is large)
    red, gap = gumbel_draw(zr[pos], gumbel_uniforms(seed, 0, 0, pos, V))
    bad, n, in_band = _gated(st["redraw"][pos], red, gap, DELTA)
    assert bad == 0, f"{bad} of {n} gated redraws differ"
    rec["head"].update(redraw_in_band=in_band, redraw_gated=n)
    ref = sampler_update(canvas, mask, sr.conf, st["argmax"], st["redraw"], 0, T)
    rec["head"]["lock_in_band"] = lock_set_check(out[1], ref.mask, mask, sr.conf, ref.cut_low,
                                                 ref.cut_high)
    log(f"30-layer head: logits max abs err {err:.3g}")

    # end to end from the embeddings
    xe = m.W.embed()[canvas]
    affected = np.zeros(C, bool)
    e2e = []
    for l in range(L):
        xe, (ri, _, margin) = m.decoder_layer(l, xe)
        gs, rs = routing_sets(routes[l]), routing_sets(ri)
        keep = ~affected
        bad, n, in_band = _gated(gs[keep], rs[keep], margin[keep], DELTA_E2E)
        assert bad == 0, f"end to end, layer {l}: {bad} of {n} gated routing decisions differ"
        affected |= np.any(gs != rs, axis=1)
        e2e.append({"layer": l, "routing_in_band": in_band, "rows_affected": int(affected.sum()),
                    "residual_max_abs_err_unaffected": float(np.abs(hid[l] - xe)[~affected].max(initial=0))})
        if l >= 2:
            m.W.forget_layer(l)
        log(f"end to end layer {l}: rows moved by in-band routing so far {int(affected.sum())}")
    ze = m.head_logits(xe) / w.temperature
    ok = ~affected
    se = lm_head_stats(ze)
    sel = ok[rows]
    diff = np.abs(zs[sel] - ze[rows, cols][sel])
    bound = TOL["bf16"][0] + TOL["bf16"][1] * np.abs(ze[rows, cols][sel])
    rec["end_to_end"] = {"layers": e2e, "rows_unaffected": int(ok.sum()),
                         "logit_err_median": float(np.median(diff)) if diff.size else 0.0,
                         "logit_err_p999": float(np.quantile(diff, 0.999)) if diff.size else 0.0,
                         "logit_err_max": float(diff.max(initial=0)),
                         "frac_beyond_bound": float(np.mean(diff > bound)) if diff.size else 0.0}
    bad, n, in_band = _gated(st["argmax"][ok], se.argmax[ok], se.top2_gap[ok], DELTA_E2E)
    rec["end_to_end"].update(argmax_in_band=in_band, argmax_gated=n, argmax_gated_bad=bad,
                             gate=DELTA_E2E)
    record("moe26b_30layer_pass0", rec)
    log(f"end to end: {rec['end_to_end']}")
    assert bad == 0, f"end to end: {bad} of {n} gated argmax decisions differ"
    assert_close("end-to-end logits", zs[sel], ze[rows, cols][sel], *TOL["bf16"])
