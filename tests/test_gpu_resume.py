"""Resume from the middle of a block: passes 0-5 on one handle, the canvas and lock mask
copied to host memory, the handle destroyed, a new handle created, loaded and prefilled
with the same prompt, passes 6-11 there.  The result equals a block run straight through on
a third handle, bit for bit (the pass is a pure function of weights, cache, canvas, mask,
step and seed), and so does a resumed entropy-bounded block.  Small bf16 model (2 layers,
d=256, 64 experts top-4, V=1024, prompt 4296)."""
import numpy as np
import pytest
import torch

import fixtures as fx
from fixtures.dg_glue import build_handle
from gpu_util import i32_dev, log, need_gpu, stats_capture, u8_dev

pytestmark = pytest.mark.gpu
W = fx.SMALL_BF16
SEED = 4242


def _handle(dg):
    h = build_handle(dg, W, capture_mask=dg.DG_CAP_STATS)
    dg.dg_prefill_prompt_kv(h, i32_dev(fx.prompt_ids(W)), W.prompt_len)
    return h


def _run(dg, h, canvas, mask, steps):
    cd, md = i32_dev(canvas), u8_dev(mask)
    for s in steps:
        dg.dg_denoise_step(h, cd, md, s, W.T, SEED)
    torch.cuda.synchronize()
    return cd.cpu().numpy(), md.cpu().numpy(), stats_capture(dg, h, W.canvas)


def test_resume_after_destroy_equals_straight_run():
    dg = need_gpu()
    init = torch.empty(W.canvas, dtype=torch.int32, device="cuda")
    h = _handle(dg)
    try:
        dg.dg_init_canvas(h, init, None, SEED)
        torch.cuda.synchronize()
        canvas0 = init.cpu().numpy()
        mask0 = np.zeros(W.canvas, np.uint8)
        straight = _run(dg, h, canvas0, mask0, range(W.T))
    finally:
        dg.dg_destroy(h)
    h = _handle(dg)
    try:
        c6, m6, _ = _run(dg, h, canvas0, mask0, range(6))
    finally:
        dg.dg_destroy(h)
    assert int(m6.sum()) == 6 * 22
    h = _handle(dg)
    try:
        resumed = _run(dg, h, c6, m6, range(6, W.T))
    finally:
        dg.dg_destroy(h)
    assert np.array_equal(resumed[0], straight[0]), "resumed canvas differs"
    assert np.array_equal(resumed[1], straight[1]) and int(resumed[1].sum()) == W.canvas
    for key in straight[2]:
        assert np.array_equal(resumed[2][key].view(np.uint8), straight[2][key].view(np.uint8)), key
    log("block resumed after pass 5 on a fresh handle: bitwise equal to the straight run")


def test_resume_entropy_bounded_block():
    """The entropy-bounded sampler keeps the previous pass's argmax in the handle (for its
    stop test): a fresh handle rebuilds it by running the last pass before the resume
    point again from the saved state, which gives that pass's canvas again."""
    dg = need_gpu()
    p = dg.eb_params(max_steps=16)

    def eb_passes(h, canvas, mask, steps):
        cd, md = i32_dev(canvas), u8_dev(mask)
        info = torch.zeros(4, dtype=torch.int32, device="cuda")
        for s in steps:
            dg.dg_denoise_step_eb(h, cd, md, s, p, SEED, info)
        torch.cuda.synchronize()
        return cd.cpu().numpy(), md.cpu().numpy(), info.cpu().numpy()

    h = _handle(dg)
    try:
        init = torch.empty(W.canvas, dtype=torch.int32, device="cuda")
        dg.dg_init_canvas(h, init, None, SEED)
        torch.cuda.synchronize()
        canvas0, mask0 = init.cpu().numpy(), np.zeros(W.canvas, np.uint8)
        straight = eb_passes(h, canvas0, mask0, range(8))
        c3, m3, _ = eb_passes(h, canvas0, mask0, range(3))      # state before pass 3
        c4, m4, _ = eb_passes(h, c3, m3, range(3, 4))
    finally:
        dg.dg_destroy(h)
    h = _handle(dg)
    try:
        # pass 3 again from the saved state before it restores the previous argmax, whose
        # canvas update must equal the first run's
        c4b, m4b, _ = eb_passes(h, c3, m3, range(3, 4))
        assert np.array_equal(c4b, c4) and np.array_equal(m4b, m4)
        resumed = eb_passes(h, c4, m4, range(4, 8))
    finally:
        dg.dg_destroy(h)
    assert np.array_equal(resumed[0], straight[0]) and np.array_equal(resumed[1], straight[1])
    assert np.array_equal(resumed[2], straight[2])
    log("entropy-bounded block resumed after pass 3: bitwise equal to the straight run")


def test_resume_from_a_saved_cache():
    """The cache saved with dg_get_kv (every layer, K and V, the prompt's rows) and restored
    into a fresh handle with dg_set_kv + dg_set_state instead of a prefill: passes 6-11 equal
    the straight run bit for bit."""
    dg = need_gpu()
    h = _handle(dg)
    try:
        init = torch.empty(W.canvas, dtype=torch.int32, device="cuda")
        dg.dg_init_canvas(h, init, None, SEED)
        torch.cuda.synchronize()
        canvas0, mask0 = init.cpu().numpy(), np.zeros(W.canvas, np.uint8)
        straight = _run(dg, h, canvas0, mask0, range(W.T))
        c6, m6, _ = _run(dg, h, canvas0, mask0, range(6))
        n_ctx, k_blk = dg.dg_get_state(h)
        saved = []
        for l in range(W.n_layers):
            for which in (0, 1):
                t = torch.empty(W.n_kv_heads, n_ctx, W.head_dim, dtype=torch.bfloat16,
                                device="cuda")
                dg.dg_get_kv(h, l, which, 0, n_ctx, t)
                saved.append(t.cpu())
        torch.cuda.synchronize()
    finally:
        dg.dg_destroy(h)
    h = build_handle(dg, W, capture_mask=dg.DG_CAP_STATS)
    try:
        with pytest.raises(dg.DGError):            # no context yet
            _run(dg, h, c6, m6, range(6, 7))
        i = 0
        for l in range(W.n_layers):
            for which in (0, 1):
                dg.dg_set_kv(h, l, which, 0, n_ctx, saved[i].cuda())
                i += 1
        with pytest.raises(dg.DGError) as ei:
            dg.dg_set_state(h, W.max_ctx, 0)         # no room for a canvas
        assert ei.value.code == dg.DG_EINVAL
        dg.dg_set_state(h, n_ctx, k_blk)
        resumed = _run(dg, h, c6, m6, range(6, W.T))
    finally:
        dg.dg_destroy(h)
    assert np.array_equal(resumed[0], straight[0]) and np.array_equal(resumed[1], straight[1])
    for key in straight[2]:
        assert np.array_equal(resumed[2][key].view(np.uint8), straight[2][key].view(np.uint8)), key
    log("block resumed from a saved cache (no prefill): bitwise equal to the straight run")


def test_resume_self_conditioned_block():
    """With self-conditioning the handle also carries the signal between passes: it is saved
    with the DG_CAP_SELFCOND capture and restored with dg_set_self_cond."""
    dg = need_gpu()
    Ws = fx.SMALL_BF16_SC

    def handle():
        h = build_handle(dg, Ws, capture_mask=dg.DG_CAP_STATS)
        dg.dg_prefill_prompt_kv(h, i32_dev(fx.prompt_ids(Ws)), Ws.prompt_len)
        return h

    def passes(h, canvas, mask, steps):
        cd, md = i32_dev(canvas), u8_dev(mask)
        for s in steps:
            dg.dg_denoise_step(h, cd, md, s, Ws.T, SEED)
        torch.cuda.synchronize()
        return cd.cpu().numpy(), md.cpu().numpy()

    h = handle()
    try:
        init = torch.empty(Ws.canvas, dtype=torch.int32, device="cuda")
        dg.dg_init_canvas(h, init, None, SEED)
        torch.cuda.synchronize()
        canvas0, mask0 = init.cpu().numpy(), np.zeros(Ws.canvas, np.uint8)
        straight = passes(h, canvas0, mask0, range(Ws.T))
        c6, m6 = passes(h, canvas0, mask0, range(6))
        z = torch.empty(Ws.canvas, Ws.d_model, dtype=torch.float32, device="cuda")
        dg.dg_get_capture(h, dg.DG_CAP_SELFCOND, 1, z)
        z_saved = z.cpu()
    finally:
        dg.dg_destroy(h)
    h = handle()
    try:
        dg.dg_set_self_cond(h, z_saved.cuda(), Ws.canvas)
        resumed = passes(h, c6, m6, range(6, Ws.T))
    finally:
        dg.dg_destroy(h)
    assert np.array_equal(resumed[0], straight[0]) and np.array_equal(resumed[1], straight[1])
    log("self-conditioned block resumed after pass 5 with its saved signal: bitwise equal")
