"""GPU parity of the whole fp32 tiny denoiser (2 layers, d=256, V=1024, P=64) against the oracle:
prefill K/V, canvas init, all 12 passes teacher-forced, a free-running block, and commit."""
import numpy as np
import pytest
import torch

import fixtures as fx
from fixtures.dg_glue import build_handle
from oracle.model import OracleModel
from oracle.philox import init_canvas
from oracle.weights import FixtureWeights
from parity import DELTA, TOL, assert_close, gated_mismatches, lock_set_check, routing_sets
from gpu_util import (i32_dev, kv_read, log, logits_capture, need_gpu, routing_capture,
                      stats_capture, u8_dev)

pytestmark = pytest.mark.gpu
W = fx.TINY_FP32


@pytest.fixture(scope="module")
def env():
    dg = need_gpu()
    caps = dg.DG_CAP_LOGITS | dg.DG_CAP_STATS | dg.DG_CAP_ROUTING
    h = build_handle(dg, W, capture_mask=caps)
    oracle = OracleModel(W, FixtureWeights(W))
    ids = fx.prompt_ids(W)
    oracle.prefill(ids)
    dg.dg_prefill_prompt_kv(h, i32_dev(ids), W.prompt_len)
    torch.cuda.synchronize()
    yield dg, h, oracle
    dg.dg_destroy(h)


def test_prefill_kv_matches(env):
    dg, h, oracle = env
    for l in range(W.n_layers):
        for which, ref in ((0, oracle.K[l]), (1, oracle.V[l])):
            got = kv_read(dg, h, l, which, 0, W.prompt_len, W.n_kv_heads, W.head_dim, torch.float32)
            assert_close(f"layer {l} {'KV'[which]}", got, ref, *TOL["f32"])


def test_canvas_init_bit_exact(env):
    dg, h, _ = env
    c = torch.empty(W.canvas, dtype=torch.int32, device="cuda")
    m = torch.full((W.canvas,), 7, dtype=torch.uint8, device="cuda")
    dg.dg_init_canvas(h, c, m, 12345)
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), init_canvas(12345, 0, W.canvas, W.vocab))
    assert int(m.sum()) == 0


def _check_pass(dg, h, oracle, canvas, mask, s, seed):
    res = oracle.denoise_step(canvas, mask, s, W.T, seed, keep_logits=True)
    cd, md = i32_dev(canvas), u8_dev(mask)
    dg.dg_denoise_step(h, cd, md, s, W.T, seed)
    torch.cuda.synchronize()
    z = logits_capture(dg, h, W.canvas, W.vocab).cpu().numpy()
    assert_close(f"pass {s} logits", z, res.logits, *TOL["f32"])
    st = stats_capture(dg, h, W.canvas)
    for key in ("m", "lse", "conf"):
        assert_close(f"pass {s} {key}", st[key], getattr(res.stats, key), *TOL["f32"])
    bad, n, _ = gated_mismatches(st["argmax"], res.stats.argmax, res.stats.top2_gap)
    assert bad == 0, f"pass {s}: {bad} argmax mismatches"
    for l in range(W.n_layers):
        gi, gg = routing_capture(dg, h, l, W.canvas, W.top_k)
        bad, n, _ = gated_mismatches(routing_sets(gi), routing_sets(res.route_idx[l]),
                                     res.route_margin[l])
        assert bad == 0, f"pass {s} layer {l}: {bad} routing mismatches"
    unl = mask == 0
    gap = np.where(unl, res.redraw_gap, -np.inf)
    bad, n, _ = gated_mismatches(st["redraw"][unl], res.redraw[unl], gap[unl])
    assert bad == 0, f"pass {s}: {bad} redraw mismatches"
    assert np.all(st["redraw"][~unl] == -1)
    mo, co = md.cpu().numpy(), cd.cpu().numpy()
    lock_set_check(mo, res.mask, mask, res.stats.conf, res.sampler.cut_low, res.sampler.cut_high)
    assert np.array_equal(co[mask == 1], canvas[mask == 1]), "a locked token changed"
    agree = (mo == res.mask)
    ok_tok = agree & ((res.mask == 0) | (res.stats.top2_gap > DELTA))
    ok_tok &= ~((res.mask == 0) & ~(np.nan_to_num(res.redraw_gap, nan=np.inf) > DELTA))
    assert np.array_equal(co[ok_tok], res.canvas[ok_tok])
    return res


def test_all_passes_teacher_forced(env):
    dg, h, oracle = env
    seed = W.seed
    canvas = init_canvas(seed, 0, W.canvas, W.vocab)
    mask = np.zeros(W.canvas, np.uint8)
    for s in range(W.T):
        log(f"tiny fp32 pass {s}")
        res = _check_pass(dg, h, oracle, canvas, mask, s, seed)
        canvas, mask = res.canvas, res.mask
    assert mask.sum() == W.canvas


def test_free_running_block_and_commit(env):
    """One whole block on each side from the same seed.  The trajectories are equal unless a
    decision of the oracle sits within 1e-3 of a tie (then the free run may legitimately
    diverge, and the GPU's block is checked by its invariants).  The commit is checked on the
    GPU's own tokens either way: K and V rows of every layer against the oracle's encoder."""
    dg, h, oracle = env
    seed = 777
    out = torch.empty(W.canvas, dtype=torch.int32, device="cuda")
    dg.dg_generate_block(h, out, W.T, seed, True)
    torch.cuda.synchronize()
    margins = []

    def cb(s, c, m, res):
        unl = m == 0
        margins.append(min(res.stats.top2_gap[unl].min(initial=np.inf),
                           np.nanmin(np.where(unl, res.redraw_gap, np.inf)),
                           abs(res.sampler.cut_low - res.sampler.cut_high)))

    ref = oracle.generate_block(W.T, seed, commit=False, on_step=cb)
    got = out.cpu().numpy()
    if not np.array_equal(got, ref):
        assert min(margins) < 1e-3, "free-running block diverged without a near-tie decision"
        log(f"near-tie decision (margin {min(margins):.2e}): trajectories diverged")
    assert got.min() >= 0 and got.max() < W.vocab
    oracle.commit(got)
    n_ctx, k_blk = dg.dg_get_state(h)
    assert (n_ctx, k_blk) == (W.prompt_len + W.canvas, 1) == (oracle.n_ctx, oracle.k_blk)
    for l in range(W.n_layers):
        for which, ref_kv, name in ((0, oracle.K[l], "K"), (1, oracle.V[l], "V")):
            got_kv = kv_read(dg, h, l, which, W.prompt_len, W.canvas, W.n_kv_heads, W.head_dim,
                             torch.float32)
            assert_close(f"commit layer {l} {name}", got_kv, ref_kv[:, W.prompt_len:], *TOL["f32"])


def test_determinism_repeat_pass(env):
    dg, h, oracle = env
    # the previous test committed a canvas and filled the cache: a full cache is refused
    with pytest.raises(dg.DGError) as ei:
        dg.dg_denoise_step(h, i32_dev(np.zeros(W.canvas)), u8_dev(np.zeros(W.canvas)), 0, W.T, 5)
    assert ei.value.code == dg.DG_ECAPACITY
    dg.dg_prefill_prompt_kv(h, i32_dev(fx.prompt_ids(W)), W.prompt_len)
    canvas = init_canvas(5, 0, W.canvas, W.vocab)
    outs = []
    for _ in range(2):
        cd, md = i32_dev(canvas), u8_dev(np.zeros(W.canvas))
        dg.dg_denoise_step(h, cd, md, 0, W.T, 5)
        z = logits_capture(dg, h, W.canvas, W.vocab)
        outs.append((cd.cpu().numpy(), md.cpu().numpy(), z.cpu().numpy()))
    assert all(np.array_equal(a, b) for a, b in zip(outs[0], outs[1]))
