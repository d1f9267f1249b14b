"""Bad data from the caller or from the weights is reported, never read out of bounds.

A token id outside [0, V) in the prompt or the canvas embeds as a zero row and
sets the handle's token flag (DG_ETOKEN from dg_check_finite); NaN router
weights give NaN router logits, whose top-k still names experts in [0, E), and
the NaN logits set the non-finite flag (DG_ENONFINITE).  The handle stays
usable: flags are cleared by the read.  Small bf16 model (2 layers, d=256,
64 experts top-4, V=1024, prompt 4296)."""
import numpy as np
import pytest
import torch

import fixtures as fx
from fixtures.dg_glue import build_handle
from gpu_util import i32_dev, log, need_gpu

pytestmark = pytest.mark.gpu
W = fx.SMALL_BF16


def _flag(dg, h):
    """Code that dg_check_finite returns (DG_OK or the error code it raises)."""
    try:
        dg.dg_check_finite(h)
        return dg.DG_OK
    except dg.DGError as e:
        return e.code


@pytest.fixture(scope="module")
def dg():
    return need_gpu()


def test_out_of_range_canvas_ids(dg):
    h = build_handle(dg, W)
    try:
        dg.dg_prefill_prompt_kv(h, i32_dev(fx.prompt_ids(W)), W.prompt_len)
        assert _flag(dg, h) == dg.DG_OK
        canvas = torch.empty(W.canvas, dtype=torch.int32, device="cuda")
        mask = torch.empty(W.canvas, dtype=torch.uint8, device="cuda")
        dg.dg_init_canvas(h, canvas, mask, 3)
        canvas[3] = W.vocab
        canvas[7] = -1
        canvas[11] = 2**31 - 1
        dg.dg_denoise_step(h, canvas, mask, 0, 4, 3)
        torch.cuda.synchronize()
        assert _flag(dg, h) == dg.DG_ETOKEN
        assert _flag(dg, h) == dg.DG_OK                      # cleared by the read
        c = canvas.cpu().numpy()
        assert c.min() >= 0 and c.max() < W.vocab            # every position was rewritten
        dg.dg_denoise_step(h, canvas, mask, 1, 4, 3)
        assert _flag(dg, h) == dg.DG_OK
        log("canvas ids V, -1, 2^31-1: DG_ETOKEN, then a clean pass")
    finally:
        dg.dg_destroy(h)


def test_out_of_range_prompt_id(dg):
    h = build_handle(dg, W)
    try:
        ids = fx.prompt_ids(W).copy()
        ids[100] = W.vocab + 5
        dg.dg_prefill_prompt_kv(h, i32_dev(ids), W.prompt_len)
        assert _flag(dg, h) == dg.DG_ETOKEN
        assert _flag(dg, h) == dg.DG_OK
    finally:
        dg.dg_destroy(h)


def test_nan_router_weights(dg):
    h = build_handle(dg, W, capture_mask=dg.DG_CAP_ROUTING)
    try:
        nan = np.full(fx.tensor_shape(W, "wr"), 0x7FC0, dtype=np.uint16)   # bf16 quiet NaN
        dg.dg_load_tensor(h, dg.DG_T_WR, 0, 0, nan)
        dg.dg_prefill_prompt_kv(h, i32_dev(fx.prompt_ids(W)), W.prompt_len)
        canvas = torch.empty(W.canvas, dtype=torch.int32, device="cuda")
        mask = torch.empty(W.canvas, dtype=torch.uint8, device="cuda")
        dg.dg_init_canvas(h, canvas, mask, 5)
        dg.dg_denoise_step(h, canvas, mask, 0, 4, 5)
        torch.cuda.synchronize()
        idx = torch.empty(2 * W.canvas * W.top_k, dtype=torch.int32, device="cuda")
        dg.dg_get_capture(h, dg.DG_CAP_ROUTING, 0, idx)
        torch.cuda.synchronize()
        ids = idx.cpu().numpy()[:W.canvas * W.top_k]
        assert ids.min() >= 0 and ids.max() < W.n_experts
        assert _flag(dg, h) == dg.DG_ENONFINITE
        dg.dg_denoise_step(h, canvas, mask, 1, 4, 5)         # canvas now holds no valid id
        assert _flag(dg, h) == dg.DG_ETOKEN
        log("NaN router weights: expert ids in range, DG_ENONFINITE, then DG_ETOKEN")
    finally:
        dg.dg_destroy(h)


def test_nan_expert_weights_reach_the_flag(dg):
    """NaN in the second expert GEMM's weights: the binary16 expert outputs keep the NaN
    (saturation applies to finite values only), so the pass's statistics flag it."""
    h = build_handle(dg, W)
    try:
        nan = np.full(fx.tensor_shape(W, "wd"), 0x7FC0, dtype=np.uint16)   # bf16 quiet NaN
        dg.dg_load_tensor(h, dg.DG_T_WD, 0, -1, nan)
        dg.dg_prefill_prompt_kv(h, i32_dev(fx.prompt_ids(W)), W.prompt_len)
        canvas = torch.empty(W.canvas, dtype=torch.int32, device="cuda")
        mask = torch.empty(W.canvas, dtype=torch.uint8, device="cuda")
        dg.dg_init_canvas(h, canvas, mask, 9)
        dg.dg_denoise_step(h, canvas, mask, 0, 4, 9)
        torch.cuda.synchronize()
        assert _flag(dg, h) in (dg.DG_ENONFINITE, dg.DG_ETOKEN)
        log("NaN expert weights: flagged")
    finally:
        dg.dg_destroy(h)


def test_binary16_saturation_is_flagged(dg):
    """Expert outputs are stored as binary16 for the combine.  Down-projection weights of
    2^20 push finite expert outputs far beyond its range (|y| >= 65520): they saturate at
    65504 and the range bit makes dg_check_finite report DG_ENONFINITE with its own message,
    in the prefill and again in a denoise pass."""
    h = build_handle(dg, W)
    try:
        big = np.full(fx.tensor_shape(W, "wd"), 0x4980, dtype=np.uint16)   # bf16 2^20
        dg.dg_load_tensor(h, dg.DG_T_WD, 0, -1, big)
        dg.dg_prefill_prompt_kv(h, i32_dev(fx.prompt_ids(W)), W.prompt_len)
        assert _flag(dg, h) == dg.DG_ENONFINITE
        assert "binary16" in dg.dg_last_error()
        assert _flag(dg, h) == dg.DG_OK                      # cleared by the read
        canvas = torch.empty(W.canvas, dtype=torch.int32, device="cuda")
        mask = torch.empty(W.canvas, dtype=torch.uint8, device="cuda")
        dg.dg_init_canvas(h, canvas, mask, 11)
        dg.dg_denoise_step(h, canvas, mask, 0, 4, 11)
        torch.cuda.synchronize()
        assert _flag(dg, h) == dg.DG_ENONFINITE
        assert "binary16" in dg.dg_last_error()
        log("expert outputs beyond the binary16 range: flagged in prefill and pass")
    finally:
        dg.dg_destroy(h)
