"""Batched canvases: B canvases denoised in one pass over a shared context (each attends to
the context and to itself only; canvas b draws its uniforms as rows b C .. of one long
canvas), against the oracle's per-canvas passes.

  * small bf16 model (2 layers, d=256, 64 experts top-4, V=1024) with a 4288-token prompt,
    batches of 3: the initial canvases bit-exact; two teacher-forced passes, each canvas's
    logits, statistics and decisions against the oracle (end to end through two bf16
    layers, the prompt cache forced to the oracle's); each canvas's own cache rows;
  * a batch of one equals the single-canvas call bit for bit, and the batched pass replayed
    as a HIP graph equals its one-by-one launches;
  * tiny fp32 model, a whole block of 2 canvases (dg_generate_block_batch) against the
    oracle's blocks;
  * batch and capacity limits are checked before any work."""
import numpy as np
import pytest
import torch

import fixtures as fx
from fixtures.dg_glue import build_handle
from parity import E2E_GATE, TOL, assert_close, routing_sets, worst_mismatch_margin
from parity import gated_mismatches as _gated
from parity import lock_set_check as _lock_check
from gpu_util import (i32_dev, kv_read, log, logits_capture, need_gpu, routing_capture,
                      stats_capture, u8_dev)

pytestmark = pytest.mark.gpu
W = fx.SMALL_BF16.with_(name="small_bf16_P4288", prompt_len=4288)
B = 3
DELTA = E2E_GATE["bf16"]
E2E_BAD_FRAC, E2E_CAP = 1e-3, 3.0


def gated(gpu, ref, margin, delta=DELTA):
    bad, n, in_band = _gated(gpu, ref, margin, delta)
    if in_band or bad:
        log(f"disagreements {bad + in_band}, largest oracle margin among them "
            f"{worst_mismatch_margin(gpu, ref, margin):.4f} (gate {delta})")
    return bad, n, in_band


@pytest.fixture(scope="module")
def env():
    from oracle.model import OracleModel
    from oracle.weights import FixtureWeights
    dg = need_gpu()
    caps = dg.DG_CAP_LOGITS | dg.DG_CAP_STATS | dg.DG_CAP_ROUTING
    h = build_handle(dg, W, capture_mask=caps, max_ctx=W.prompt_len + B * W.canvas, max_batch=B)
    oracle = OracleModel(W, FixtureWeights(W))
    ids = fx.prompt_ids(W)
    oracle.prefill(ids)
    dg.dg_prefill_prompt_kv(h, i32_dev(ids), W.prompt_len)
    for l in range(W.n_layers):      # the oracle's prompt cache on both sides
        for which, ref in ((0, oracle.K[l]), (1, oracle.V[l])):
            src = torch.from_numpy(np.ascontiguousarray(ref.astype(np.float32))).to(torch.bfloat16).cuda()
            dg.dg_set_kv(h, l, which, 0, W.prompt_len, src)
    torch.cuda.synchronize()
    yield dg, h, oracle
    dg.dg_destroy(h)


def test_batch_limits(env):
    dg, h, _ = env
    c = torch.zeros((B + 1) * W.canvas, dtype=torch.int32, device="cuda")
    m = torch.zeros((B + 1) * W.canvas, dtype=torch.uint8, device="cuda")
    for bad_b in (0, B + 1, -1):
        with pytest.raises(dg.DGError) as ei:
            dg.dg_denoise_step_batch(h, c, m, bad_b, 0, W.T, 1)
        assert ei.value.code == dg.DG_EINVAL


def test_initial_canvases_bit_exact(env):
    dg, h, oracle = env
    c = torch.empty(B * W.canvas, dtype=torch.int32, device="cuda")
    m = torch.full((B * W.canvas,), 7, dtype=torch.uint8, device="cuda")
    dg.dg_init_canvas_batch(h, c, m, B, 31)
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy().reshape(B, -1), oracle.init_canvas_batch(31, B))
    assert not m.cpu().numpy().any()


@pytest.mark.parametrize("s", [0, 1])
def test_batched_pass_against_oracle(env, s):
    dg, h, oracle = env
    C, k, seed = W.canvas, W.top_k, 31
    canv = oracle.init_canvas_batch(seed, B)
    masks = np.zeros((B, C), np.uint8)
    if s == 1:      # pass 1 from the oracle's pass-0 output (teacher forcing)
        res = oracle.denoise_step_batch(canv, masks, 0, W.T, seed)
        canv = np.stack([r.canvas for r in res])
        masks = np.stack([r.mask for r in res])
    ref = oracle.denoise_step_batch(canv, masks, s, W.T, seed, keep_logits=True)
    cd, md = i32_dev(canv.ravel()), u8_dev(masks.ravel())
    log(f"batched pass {s}, {B} canvases")
    dg.dg_denoise_step_batch(h, cd, md, B, s, W.T, seed)
    torch.cuda.synchronize()
    st = stats_capture(dg, h, B * C)
    z = logits_capture(dg, h, B * C, W.vocab).cpu().numpy()
    routes = [routing_capture(dg, h, l, B * C, k)[0] for l in range(W.n_layers)]
    co, mo = cd.cpu().numpy().reshape(B, C), md.cpu().numpy().reshape(B, C)
    for b in range(B):
        r = ref[b]
        rows = slice(b * C, (b + 1) * C)
        affected = np.zeros(C, bool)
        for l in range(W.n_layers):
            gs, rs = routing_sets(routes[l][rows]), routing_sets(r.route_idx[l])
            keep = ~affected
            bad, n, _ = gated(gs[keep], rs[keep], r.route_margin[l][keep])
            assert bad == 0, f"canvas {b} layer {l}: {bad} of {n} gated routing decisions differ"
            affected |= np.any(gs != rs, axis=1)
        ok = ~affected
        assert_close(f"canvas {b} logits", z[rows][ok], r.logits[ok], *TOL["bf16"],
                     max_bad_frac=E2E_BAD_FRAC)
        assert_close(f"canvas {b} logits (cap)", z[rows][ok], r.logits[ok],
                     *(E2E_CAP * t for t in TOL["bf16"]))
        for key in ("m", "lse", "conf"):
            assert_close(f"canvas {b} {key}", st[key][rows][ok], getattr(r.stats, key)[ok],
                         *TOL["bf16"])
        bad, n, _ = gated(st["argmax"][rows][ok], r.stats.argmax[ok], r.stats.top2_gap[ok])
        assert bad == 0, f"canvas {b}: {bad} of {n} gated argmax decisions differ"
        unl = (masks[b] == 0) & ok
        bad, n, _ = gated(st["redraw"][rows][unl], r.redraw[unl], r.redraw_gap[unl])
        assert bad == 0, f"canvas {b}: {bad} of {n} gated redraws differ"
        from oracle.model import sampler_update
        conf_ref = np.where(ok, r.stats.conf, st["conf"][rows])
        sr = sampler_update(canv[b], masks[b], conf_ref, st["argmax"][rows], st["redraw"][rows],
                            s, W.T)
        _lock_check(mo[b], sr.mask, masks[b], conf_ref, sr.cut_low, sr.cut_high, delta=DELTA)
        assert np.array_equal(co[b][masks[b] == 1], canv[b][masks[b] == 1])
        log(f"canvas {b}: rows moved by in-band routing {int(affected.sum())}")


def test_canvas_cache_rows(env):
    """Each canvas's K/V rows of layer 0 (n_ctx + b C + i): the projection of its own
    embedded tokens at positions n_ctx + i."""
    from oracle.numerics import rmsnorm
    dg, h, oracle = env
    C, seed = W.canvas, 77
    canv = oracle.init_canvas_batch(seed, B)
    cd, md = i32_dev(canv.ravel()), u8_dev(np.zeros(B * C))
    dg.dg_denoise_step_batch(h, cd, md, B, 0, W.T, seed)
    torch.cuda.synchronize()
    pos = np.arange(W.prompt_len, W.prompt_len + C)
    for which in (0, 1):
        got = kv_read(dg, h, 0, which, W.prompt_len, B * C, W.n_kv_heads, W.head_dim,
                      torch.bfloat16)
        for b in range(B):
            a = oracle._act(rmsnorm(oracle.W.embed()[canv[b]], W.rms_eps))
            ref = oracle.kv_rows(0, a, pos)[which]
            assert_close(f"canvas {b} layer-0 {'KV'[which]} rows", got[:, b * C:(b + 1) * C], ref,
                         *TOL["bf16"])


def test_batch_of_one_equals_single_and_graph_equals_eager(env):
    dg, h, oracle = env
    C, seed = W.canvas, 5
    canv = oracle.init_canvas_batch(seed, B)

    def run(fn):
        cd, md = i32_dev(canv.ravel()), u8_dev(np.zeros(B * C))
        out = []
        for s in range(2):
            fn(cd, md, s)
            torch.cuda.synchronize()
            out.append((cd.cpu().numpy().copy(), md.cpu().numpy().copy()))
        return out

    one = run(lambda cd, md, s: dg.dg_denoise_step_batch(h, cd[:C], md[:C], 1, s, W.T, seed))
    single = run(lambda cd, md, s: dg.dg_denoise_step(h, cd[:C], md[:C], s, W.T, seed))
    for a, b in zip(one, single):
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    dg.dg_set_capture(h, 0)           # per-layer captures off: the batched pass replays a graph
    try:
        dg.dg_set_graphs(h, 1)
        graph = run(lambda cd, md, s: dg.dg_denoise_step_batch(h, cd, md, B, s, W.T, seed))
        dg.dg_set_graphs(h, 0)
        eager = run(lambda cd, md, s: dg.dg_denoise_step_batch(h, cd, md, B, s, W.T, seed))
    finally:
        dg.dg_set_graphs(h, 1)
        dg.dg_set_capture(h, dg.DG_CAP_LOGITS | dg.DG_CAP_STATS | dg.DG_CAP_ROUTING)
    for a, b in zip(graph, eager):
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_tiny_fp32_batched_blocks():
    """Two whole blocks at once on the tiny fp32 model against two oracle blocks: equal
    unless a decision of the oracle sits within 1e-3 of a tie."""
    from oracle.model import OracleModel
    from oracle.weights import FixtureWeights
    dg = need_gpu()
    w = fx.TINY_FP32
    h = build_handle(dg, w, max_ctx=w.prompt_len + 2 * w.canvas, max_batch=2)
    try:
        oracle = OracleModel(w, FixtureWeights(w))
        ids = fx.prompt_ids(w)
        oracle.prefill(ids)
        dg.dg_prefill_prompt_kv(h, i32_dev(ids), w.prompt_len)
        out = torch.empty(2 * w.canvas, dtype=torch.int32, device="cuda")
        seed = 99
        dg.dg_generate_block_batch(h, out, 2, w.T, seed)
        got = out.cpu().numpy().reshape(2, -1)
        canv = oracle.init_canvas_batch(seed, 2)
        masks = np.zeros((2, w.canvas), np.uint8)
        margin = np.inf
        for s in range(w.T):
            res = oracle.denoise_step_batch(canv, masks, s, w.T, seed)
            for r, m in zip(res, masks):
                unl = m == 0
                margin = min(margin, r.stats.top2_gap[unl].min(initial=np.inf),
                             np.nanmin(np.where(unl, r.redraw_gap, np.inf)),
                             abs(r.sampler.cut_low - r.sampler.cut_high))
            canv = np.stack([r.canvas for r in res])
            masks = np.stack([r.mask for r in res])
        assert masks.all()
        if not np.array_equal(got, canv):
            assert margin < 1e-3, "batched blocks diverged without a near-tie decision"
            log(f"near-tie decision (margin {margin:.2e}): trajectories diverged")
        assert got.min() >= 0 and got.max() < w.vocab
        log(f"tiny fp32, 2 canvases: {int((got == canv).sum())} of {got.size} tokens equal")
    finally:
        dg.dg_destroy(h)
