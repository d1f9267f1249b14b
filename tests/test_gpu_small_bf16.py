"""GPU parity of a small bf16 denoiser (2 layers, d=256, 64 experts top-4, V=1024) through the
same MFMA kernels as the large models, with a 4296-token prompt that spans two prefill chunks:
prefill K/V of every row, per-layer hidden states, routing, logits and decisions of
teacher-forced passes, and a committed canvas."""
import numpy as np
import pytest
import torch

import fixtures as fx
from fixtures.dg_glue import build_handle
from oracle.model import OracleModel
from oracle.philox import init_canvas
from oracle.weights import FixtureWeights
from parity import E2E_GATE, TOL, assert_close, routing_sets, worst_mismatch_margin
from parity import gated_mismatches as _gated
from parity import lock_set_check as _lock_check

DELTA = E2E_GATE["bf16"]   # passes end to end through two bf16 layers


def gated_mismatches(gpu, ref, margin):
    bad, n, in_band = _gated(gpu, ref, margin, DELTA)
    if in_band or bad:
        log(f"disagreements {bad + in_band}, largest oracle margin among them "
            f"{worst_mismatch_margin(gpu, ref, margin):.4f} (gate {DELTA})")
    return bad, n, in_band


def lock_set_check(*args):
    return _lock_check(*args, delta=DELTA)
from gpu_util import (i32_dev, kv_read, log, logits_capture, need_gpu, routing_capture,
                      stats_capture, u8_dev)

pytestmark = pytest.mark.gpu
W = fx.SMALL_BF16


@pytest.fixture(scope="module")
def env():
    dg = need_gpu()
    caps = dg.DG_CAP_LOGITS | dg.DG_CAP_STATS | dg.DG_CAP_ROUTING | dg.DG_CAP_HIDDEN
    h = build_handle(dg, W, capture_mask=caps)
    oracle = OracleModel(W, FixtureWeights(W), capture_hidden=True)
    ids = fx.prompt_ids(W)
    oracle.prefill(ids)
    dg.dg_prefill_prompt_kv(h, i32_dev(ids), W.prompt_len)
    torch.cuda.synchronize()
    yield dg, h, oracle
    dg.dg_destroy(h)


def test_prefill_kv_every_row(env):
    dg, h, oracle = env
    # a row of layer l is determined when its token's routing in layers < l is not a near tie
    trusted = np.ones(W.prompt_len, bool)
    for l in range(W.n_layers):
        for which, ref in ((0, oracle.K[l]), (1, oracle.V[l])):
            got = kv_read(dg, h, l, which, 0, W.prompt_len, W.n_kv_heads, W.head_dim,
                          torch.bfloat16)
            err = np.abs(got - ref)
            bad = err > 2e-2 + 1e-2 * np.abs(ref)
            rows = np.flatnonzero(bad.any(axis=(0, 2)) & trusted)
            assert rows.size == 0, (f"layer {l} {'KV'[which]}: {rows.size} rows differ, first "
                                    f"{rows[:10].tolist()}, max err {err.max():.3g}")
        log(f"layer {l}: {int((~trusted).sum())} rows behind a near-tie routing")
        if l < W.n_layers - 1:
            trusted &= oracle.enc_route_margin[l] > DELTA


def test_teacher_force_prompt_cache(env):
    """Give the GPU the oracle's prompt K/V, so the passes below see the oracle's context."""
    dg, h, oracle = env
    for l in range(W.n_layers):
        for which, ref in ((0, oracle.K[l]), (1, oracle.V[l])):
            src = torch.from_numpy(np.ascontiguousarray(ref.astype(np.float32))).to(torch.bfloat16).cuda()
            dg.dg_set_kv(h, l, which, 0, W.prompt_len, src)
            back = kv_read(dg, h, l, which, 0, W.prompt_len, W.n_kv_heads, W.head_dim,
                           torch.bfloat16)
            assert np.array_equal(back, ref)


def test_passes_teacher_forced(env):
    dg, h, oracle = env
    seed = 4
    canvas = init_canvas(seed, 0, W.canvas, W.vocab)
    mask = np.zeros(W.canvas, np.uint8)
    for s in range(3):
        log(f"small bf16 pass {s}")
        res = oracle.denoise_step(canvas, mask, s, W.T, seed, keep_logits=True)
        cd, md = i32_dev(canvas), u8_dev(mask)
        dg.dg_denoise_step(h, cd, md, s, W.T, seed)
        torch.cuda.synchronize()
        affected = np.zeros(W.canvas, bool)
        for l in range(W.n_layers):
            gi, gg = routing_capture(dg, h, l, W.canvas, W.top_k)
            gi, ri = routing_sets(gi), routing_sets(res.route_idx[l])
            keep = ~affected   # rows whose routing differed upstream carry other inputs
            bad, n, _ = gated_mismatches(gi[keep], ri[keep], res.route_margin[l][keep])
            hid = torch.empty(W.canvas, W.d_model, dtype=torch.float32, device="cuda")
            dg.dg_get_capture(h, dg.DG_CAP_HIDDEN, l, hid)
            hg = hid.cpu().numpy().astype(np.float64)
            rows_bad = np.flatnonzero((np.abs(hg - res.hidden[l]) >
                                       2e-2 + 1e-2 * np.abs(res.hidden[l])).any(axis=1))
            assert bad == 0, (f"pass {s} layer {l}: {bad}/{n} gated routing differ; "
                              f"hidden rows off: {rows_bad[:20].tolist()}")
            affected |= np.any(gi != ri, axis=1)
            ok_rows = ~affected
            assert_close(f"pass {s} layer {l} hidden", hg[ok_rows], res.hidden[l][ok_rows],
                         *TOL["bf16"])
        ok = ~affected
        z = logits_capture(dg, h, W.canvas, W.vocab).cpu().numpy()
        assert_close(f"pass {s} logits", z[ok], res.logits[ok], *TOL["bf16"])
        st = stats_capture(dg, h, W.canvas)
        bad, n, _ = gated_mismatches(st["argmax"][ok], res.stats.argmax[ok], res.stats.top2_gap[ok])
        assert bad == 0
        unl = (mask == 0) & ok
        bad, n, _ = gated_mismatches(st["redraw"][unl], res.redraw[unl], res.redraw_gap[unl])
        assert bad == 0
        mo = md.cpu().numpy()
        conf_ref = np.where(ok, res.stats.conf, st["conf"])
        lock_set_check(mo, res.mask, mask, conf_ref, res.sampler.cut_low, res.sampler.cut_high)
        canvas, mask = res.canvas, res.mask


def test_commit_rows(env):
    dg, h, oracle = env
    canvas = init_canvas(9, 0, W.canvas, W.vocab)
    dg.dg_commit_canvas(h, i32_dev(canvas))
    oracle.commit(canvas)
    torch.cuda.synchronize()
    trusted = np.ones(W.canvas, bool)
    for l in range(W.n_layers):
        for which, ref_kv, name in ((0, oracle.K[l], "K"), (1, oracle.V[l], "V")):
            got = kv_read(dg, h, l, which, W.prompt_len, W.canvas, W.n_kv_heads, W.head_dim,
                          torch.bfloat16)
            assert_close(f"commit layer {l} {name}", got[:, trusted],
                         ref_kv[:, W.prompt_len:][:, trusted], *TOL["bf16"])
        if l < W.n_layers - 1:
            trusted &= oracle.enc_route_margin[l][W.prompt_len:] > DELTA
    n_ctx, k_blk = dg.dg_get_state(h)
    assert (n_ctx, k_blk) == (W.prompt_len + W.canvas, 1)
