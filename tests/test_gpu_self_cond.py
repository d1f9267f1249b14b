"""GPU parity of the self-conditioning signal z = FFW(Softmax(L/tau) E), fed into the next pass
(technical-report summary, Method: decoder and update equations), against the oracle:
  * tiny fp32 model: every pass of a block teacher-forced (canvas, mask and the incoming signal
    from the oracle): logits with the signal injected, decisions, u = p0 E and the next signal;
    the last pass of a block forms none; a free-running block equals the chain of single passes
    and the oracle's block (unless a decision sits at a near tie); a batch of two canvases with
    a signal per canvas;
  * small bf16 model (the MFMA path: posterior rows from the LM-head epilogue, the stream-K
    contraction over the vocabulary, the feed-forward block in fragment order): teacher-forced
    passes, graph == eager bitwise;
  * the benched model's dimensions (V = 262144, d = Fsc = 2816, one layer): u and z of sampled
    rows of pass 0 for one canvas and for a batch of two (two 256-row blocks in the contraction).
"""
import numpy as np
import pytest
import torch

import fixtures as fx
from fixtures.dg_glue import build_handle
from gpu_util import (i32_dev, log, logits_capture, need_gpu, record, routing_capture,
                      stats_capture, u8_dev)
from oracle.model import OracleModel
from oracle.philox import init_canvas
from oracle.weights import FixtureWeights
from parity import (E2E_GATE, GATE, TOL, assert_close, gated_mismatches, lock_set_check,
                    routing_sets)

pytestmark = pytest.mark.gpu


def f32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32))).cuda()


def sc_capture(dg, h, rows, d):
    """(u, z) of the last pass that formed a signal, float64 [rows, d] each."""
    u = torch.empty(rows, d, dtype=torch.float32, device="cuda")
    z = torch.empty(rows, d, dtype=torch.float32, device="cuda")
    dg.dg_get_capture(h, dg.DG_CAP_SELFCOND, 0, u)
    dg.dg_get_capture(h, dg.DG_CAP_SELFCOND, 1, z)
    torch.cuda.synchronize()
    return u.cpu().numpy().astype(np.float64), z.cpu().numpy().astype(np.float64)


def row_rel_err(got, ref):
    """Per row ||got - ref|| / ||ref||."""
    return np.linalg.norm(got - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-300)


def check_decisions(tag, st, res, canvas, mask, co, mo, delta, rows=None):
    """Decisions of one pass; rows (bool mask) restricts the per-position ones to rows whose
    inputs agree (the lock set is checked on the oracle's confidences of those rows and the
    GPU's own elsewhere)."""
    rows = np.ones(len(canvas), bool) if rows is None else rows
    bad, n, _ = gated_mismatches(st["argmax"][rows], res.stats.argmax[rows],
                                 res.stats.top2_gap[rows], delta)
    assert bad == 0, f"{tag}: {bad} argmax mismatches"
    unl = (mask == 0) & rows
    bad, n, _ = gated_mismatches(st["redraw"][unl], res.redraw[unl], res.redraw_gap[unl], delta)
    assert bad == 0, f"{tag}: {bad} redraw mismatches"
    conf = np.where(rows, res.stats.conf, st["conf"])
    lock_set_check(mo, res.mask, mask, conf, res.sampler.cut_low, res.sampler.cut_high,
                   delta=delta)
    assert np.array_equal(co[mask == 1], canvas[mask == 1]), f"{tag}: a locked token changed"
    ok = (mo == res.mask) & ((res.mask == 0) | (res.stats.top2_gap > delta)) & rows
    ok &= ~((res.mask == 0) & ~(np.nan_to_num(res.redraw_gap, nan=np.inf) > delta))
    assert np.array_equal(co[ok], res.canvas[ok]), f"{tag}: tokens differ"


# =================================================================== tiny fp32
TINY = fx.TINY_FP32_SC


@pytest.fixture(scope="module")
def tiny():
    dg = need_gpu()
    h = build_handle(dg, TINY, capture_mask=dg.DG_CAP_LOGITS | dg.DG_CAP_STATS)
    oracle = OracleModel(TINY, FixtureWeights(TINY))
    ids = fx.prompt_ids(TINY)
    oracle.prefill(ids)
    dg.dg_prefill_prompt_kv(h, i32_dev(ids), TINY.prompt_len)
    torch.cuda.synchronize()
    yield dg, h, oracle
    dg.dg_destroy(h)


def test_tiny_passes_teacher_forced(tiny):
    dg, h, oracle = tiny
    W = TINY
    seed = 21
    canvas = init_canvas(seed, 0, W.canvas, W.vocab)
    mask = np.zeros(W.canvas, np.uint8)
    z = None
    worst = {"logits": 0.0, "u": 0.0, "z": 0.0}
    for s in range(W.T):
        log(f"tiny fp32 self-conditioned pass {s}")
        res = oracle.denoise_step(canvas, mask, s, W.T, seed, keep_logits=True, z_in=z,
                                  want_signal=s < W.T - 1)
        if z is not None:
            dg.dg_set_self_cond(h, f32_dev(z), W.canvas)
        cd, md = i32_dev(canvas), u8_dev(mask)
        dg.dg_denoise_step(h, cd, md, s, W.T, seed)
        torch.cuda.synchronize()
        lg = logits_capture(dg, h, W.canvas, W.vocab).cpu().numpy()
        worst["logits"] = max(worst["logits"],
                              assert_close(f"pass {s} logits", lg, res.logits, *TOL["f32"]))
        st = stats_capture(dg, h, W.canvas)
        check_decisions(f"pass {s}", st, res, canvas, mask, cd.cpu().numpy(), md.cpu().numpy(),
                        GATE["f32"])
        u, zg = sc_capture(dg, h, W.canvas, W.d_model)
        if s < W.T - 1:
            for name, got, ref in (("u", u, res.sc.u), ("z", zg, res.sc.z)):
                scale = np.abs(ref).max()
                worst[name] = max(worst[name], assert_close(f"pass {s} {name}", got, ref,
                                                            1e-4 * scale, 1e-4) / scale)
        else:   # the last pass forms no signal: the one set for it is still there
            assert res.sc is None
            assert np.array_equal(zg, z.astype(np.float32).astype(np.float64))
        canvas, mask, z = res.canvas, res.mask, (res.sc.z if res.sc is not None else None)
    log(f"largest errors: logits {worst['logits']:.2e}, u {worst['u']:.2e} and z "
        f"{worst['z']:.2e} of the largest value")
    assert mask.sum() == W.canvas


def test_tiny_signal_moves_the_logits(tiny):
    """Pass 1 with the signal of pass 0 differs from pass 1 with a zero signal by far more than
    the tolerance (the injection is visible), and a zero signal set by hand gives exactly the
    logits of pass 1 of a model without self-conditioning (a pass with z = 0)."""
    dg, h, oracle = tiny
    W = TINY
    seed = 5
    canvas = init_canvas(seed, 0, W.canvas, W.vocab)
    mask = np.zeros(W.canvas, np.uint8)
    r0 = oracle.denoise_step(canvas, mask, 0, W.T, seed)
    outs = []
    for zin in (r0.sc.z, np.zeros((W.canvas, W.d_model))):
        dg.dg_set_self_cond(h, f32_dev(zin), W.canvas)
        dg.dg_denoise_step(h, i32_dev(r0.canvas), u8_dev(r0.mask), 1, W.T, seed)
        outs.append(logits_capture(dg, h, W.canvas, W.vocab).cpu().numpy())
    assert np.abs(outs[0] - outs[1]).max() > 100 * TOL["f32"][0]
    ref0 = oracle.denoise_step(r0.canvas, r0.mask, 1, W.T, seed, keep_logits=True)
    assert_close("zero signal logits", outs[1], ref0.logits, *TOL["f32"])


def test_tiny_block_chain_and_oracle(tiny):
    dg, h, oracle = tiny
    W = TINY
    seed = 99
    cd = torch.empty(W.canvas, dtype=torch.int32, device="cuda")
    md = torch.empty(W.canvas, dtype=torch.uint8, device="cuda")
    dg.dg_init_canvas(h, cd, md, seed)
    for s in range(W.T):
        dg.dg_denoise_step(h, cd, md, s, W.T, seed)
    out = torch.empty(W.canvas, dtype=torch.int32, device="cuda")
    dg.dg_generate_block(h, out, W.T, seed, False)
    torch.cuda.synchronize()
    chain, block = cd.cpu().numpy(), out.cpu().numpy()
    assert np.array_equal(chain, block), "generate_block differs from its chain of passes"
    margins = []

    def cb(s, c, m, res):
        unl = m == 0
        margins.append(min(res.stats.top2_gap[unl].min(initial=np.inf),
                           np.nanmin(np.where(unl, res.redraw_gap, np.inf)),
                           abs(res.sampler.cut_low - res.sampler.cut_high)))

    ref = oracle.generate_block(W.T, seed, commit=False, on_step=cb)
    if not np.array_equal(block, ref):
        assert min(margins) < 1e-3, "free-running block diverged without a near-tie decision"
        log(f"near-tie decision (margin {min(margins):.2e}): trajectories diverged")


def test_tiny_batch_of_two_signals():
    dg = need_gpu()
    W = TINY
    B = 2
    h = build_handle(dg, W, capture_mask=dg.DG_CAP_STATS, max_batch=B,
                     max_ctx=W.prompt_len + B * W.canvas)
    try:
        oracle = OracleModel(W, FixtureWeights(W))
        ids = fx.prompt_ids(W)
        oracle.prefill(ids)
        dg.dg_prefill_prompt_kv(h, i32_dev(ids), W.prompt_len)
        seed = 17
        canvases = list(oracle.init_canvas_batch(seed, B))
        masks = [np.zeros(W.canvas, np.uint8) for _ in range(B)]
        zs = None
        for s in range(3):
            res = oracle.denoise_step_batch(canvases, masks, s, W.T, seed, z_ins=zs)
            if zs is not None:
                dg.dg_set_self_cond(h, f32_dev(np.concatenate(zs)), B * W.canvas)
            cd, md = i32_dev(np.concatenate(canvases)), u8_dev(np.concatenate(masks))
            dg.dg_denoise_step_batch(h, cd, md, B, s, W.T, seed)
            torch.cuda.synchronize()
            st = stats_capture(dg, h, B * W.canvas)
            u, zg = sc_capture(dg, h, B * W.canvas, W.d_model)
            co, mo = cd.cpu().numpy(), md.cpu().numpy()
            for b in range(B):
                rows = slice(b * W.canvas, (b + 1) * W.canvas)
                stb = {k: v[rows] for k, v in st.items()}
                check_decisions(f"pass {s} canvas {b}", stb, res[b], canvases[b], masks[b],
                                co[rows], mo[rows], GATE["f32"])
                for name, got, ref in (("u", u[rows], res[b].sc.u), ("z", zg[rows], res[b].sc.z)):
                    assert_close(f"pass {s} canvas {b} {name}", got, ref,
                                 1e-4 * np.abs(ref).max(), 1e-4)
            canvases = [r.canvas for r in res]
            masks = [r.mask for r in res]
            zs = [r.sc.z for r in res]
    finally:
        dg.dg_destroy(h)


# =================================================================== small bf16
SMALL = fx.SMALL_BF16_SC
DELTA = E2E_GATE["bf16"]      # decisions end to end through two bf16 layers
SC_REL = 3e-2                 # per-row relative error of u and z, end to end (see below)


@pytest.fixture(scope="module")
def small():
    dg = need_gpu()
    h = build_handle(dg, SMALL, capture_mask=dg.DG_CAP_LOGITS | dg.DG_CAP_STATS |
                     dg.DG_CAP_ROUTING)
    oracle = OracleModel(SMALL, FixtureWeights(SMALL))
    ids = fx.prompt_ids(SMALL)
    oracle.prefill(ids)
    dg.dg_prefill_prompt_kv(h, i32_dev(ids), SMALL.prompt_len)
    # the oracle's prompt cache, so that the passes below see the oracle's context
    for l in range(SMALL.n_layers):
        for which, ref in ((0, oracle.K[l]), (1, oracle.V[l])):
            src = torch.from_numpy(np.ascontiguousarray(ref.astype(np.float32))).to(
                torch.bfloat16).cuda()
            dg.dg_set_kv(h, l, which, 0, SMALL.prompt_len, src)
    torch.cuda.synchronize()
    yield dg, h, oracle
    dg.dg_destroy(h)


def test_small_bf16_passes_teacher_forced(small):
    """Rows whose expert set differs from the oracle's in some layer (a routing near tie, gated
    at the end-to-end bound) carry other inputs from there on and are left out of the row-wise
    comparisons.  u = p0 E and z are compared per row by relative norm: both sides form p0 from
    their own logits, which agree within the bf16 end-to-end bound, so the error of u and z is
    that of the logits carried through the softmax (relative change of p0 ~ the absolute change
    of the tempered logit), averaged over the vocabulary; 3e-2 is the bf16 end-to-end decision
    gate read as a relative bound."""
    dg, h, oracle = small
    W = SMALL
    seed = 8
    canvas = init_canvas(seed, 0, W.canvas, W.vocab)
    mask = np.zeros(W.canvas, np.uint8)
    z = None
    worst = {"u": 0.0, "z": 0.0}
    for s in range(3):
        log(f"small bf16 self-conditioned pass {s}")
        res = oracle.denoise_step(canvas, mask, s, W.T, seed, keep_logits=True, z_in=z)
        if z is not None:
            dg.dg_set_self_cond(h, f32_dev(z), W.canvas)
        cd, md = i32_dev(canvas), u8_dev(mask)
        dg.dg_denoise_step(h, cd, md, s, W.T, seed)
        torch.cuda.synchronize()
        affected = np.zeros(W.canvas, bool)
        for l in range(W.n_layers):
            gi, _ = routing_capture(dg, h, l, W.canvas, W.top_k)
            gi, ri = routing_sets(gi), routing_sets(res.route_idx[l])
            bad, n, _ = gated_mismatches(gi[~affected], ri[~affected],
                                         res.route_margin[l][~affected], DELTA)
            assert bad == 0, f"pass {s} layer {l}: {bad} gated routing mismatches"
            affected |= np.any(gi != ri, axis=1)
        ok = ~affected
        log(f"pass {s}: {int(affected.sum())} rows behind a routing near tie")
        lg = logits_capture(dg, h, W.canvas, W.vocab).cpu().numpy()
        assert_close(f"pass {s} logits", lg[ok], res.logits[ok], *TOL["bf16"])
        st = stats_capture(dg, h, W.canvas)
        check_decisions(f"pass {s}", st, res, canvas, mask, cd.cpu().numpy(), md.cpu().numpy(),
                        DELTA, rows=ok)
        u, zg = sc_capture(dg, h, W.canvas, W.d_model)
        for name, got, ref in (("u", u[ok], res.sc.u[ok]), ("z", zg[ok], res.sc.z[ok])):
            e = row_rel_err(got, ref)
            worst[name] = max(worst[name], float(e.max()))
            assert e.max() < SC_REL, f"pass {s} {name}: row {int(e.argmax())} off by {e.max():.3g}"
        canvas, mask, z = res.canvas, res.mask, res.sc.z
    log(f"largest per-row relative error: u {worst['u']:.2e}, z {worst['z']:.2e}")
    record("small_bf16_selfcond", {"u_row_rel_max": worst["u"], "z_row_rel_max": worst["z"]})


def test_small_bf16_graph_equals_eager(small):
    dg, h, oracle = small
    W = SMALL
    canvas = init_canvas(3, 0, W.canvas, W.vocab)
    zin = np.random.default_rng(0).standard_normal((W.canvas, W.d_model)) * 0.02
    outs = []
    for graphs in (True, False):
        dg.dg_set_graphs(h, graphs)
        dg.dg_set_self_cond(h, f32_dev(zin), W.canvas)
        cd, md = i32_dev(canvas), u8_dev(np.zeros(W.canvas))
        dg.dg_denoise_step(h, cd, md, 1, W.T, 3)
        u, zg = sc_capture(dg, h, W.canvas, W.d_model)
        outs.append((cd.cpu().numpy(), md.cpu().numpy(), u, zg))
    dg.dg_set_graphs(h, True)
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


# =================================================================== full size
BIG = fx.MOE26B_SC_1L


def _sample_rows(C, rng):
    return np.unique(np.concatenate([[0, 1, 15, 16, 127, 128, C - 1], rng.choice(C, 9, False)]))


def test_benched_dimensions_pass0_signal():
    """Pass 0 of the benched dimensions with one layer: the oracle runs the decoder over the
    whole canvas (bidirectional) and the head and signal on sampled rows only; the GPU's u and
    z of those rows, for one canvas and for each canvas of a batch of two, within the per-row
    relative bound of the bf16 path."""
    dg = need_gpu()
    W = BIG
    B = 2
    log("building the one-layer model of the benched dimensions")
    h = build_handle(dg, W, capture_mask=dg.DG_CAP_ROUTING, max_batch=B,
                     max_ctx=W.prompt_len + B * W.canvas)
    try:
        ids = fx.prompt_ids(W)
        dg.dg_prefill_prompt_kv(h, i32_dev(ids), W.prompt_len)
        oracle = OracleModel(W, FixtureWeights(W, cache_experts=False))
        oracle.prefill(ids)
        seed = 4
        canvases = oracle.init_canvas_batch(seed, B)
        rng = np.random.default_rng(1)
        worst = {}
        for batch in (1, 2):
            cd = i32_dev(canvases[:batch].reshape(-1))
            md = u8_dev(np.zeros(batch * W.canvas))
            log(f"GPU pass 0, batch of {batch}")
            if batch == 1:
                dg.dg_denoise_step(h, cd, md, 0, W.T, seed)
            else:
                dg.dg_denoise_step_batch(h, cd, md, batch, 0, W.T, seed)
            u, zg = sc_capture(dg, h, batch * W.canvas, W.d_model)
            routes = [routing_capture(dg, h, l, batch * W.canvas, W.top_k)[0]
                      for l in range(W.n_layers)]
            for b in range(batch):
                rows = _sample_rows(W.canvas, rng)
                log(f"oracle decoder, canvas {b}, rows {rows.tolist()}")
                x = oracle.W.embed()[canvases[b]]
                keep = np.ones(W.canvas, bool)
                for l in range(W.n_layers):
                    x, rt = oracle.decoder_layer(l, x)
                    gi = routing_sets(routes[l][b * W.canvas:(b + 1) * W.canvas])
                    ri = routing_sets(rt[0])
                    bad, n, _ = gated_mismatches(gi[keep], ri[keep], rt[2][keep], DELTA)
                    assert bad == 0, f"batch {batch} canvas {b} layer {l}: routing differs"
                    keep &= ~np.any(gi != ri, axis=1)
                rows = rows[keep[rows]]          # rows behind a routing near tie are left out
                zt = oracle.head_logits(x[rows]) / W.temperature
                ref = oracle.next_signal(zt)
                for name, got, r in (("u", u[b * W.canvas + rows], ref.u),
                                     ("z", zg[b * W.canvas + rows], ref.z)):
                    e = row_rel_err(got, r)
                    key = f"batch{batch}_canvas{b}_{name}"
                    worst[key] = float(e.max())
                    assert e.max() < SC_REL, f"{key}: row {int(rows[e.argmax()])} off by {e.max():.3g}"
        log(f"per-row relative errors: {worst}")
        record("moe26b_1L_selfcond_pass0", worst)
    finally:
        dg.dg_destroy(h)
