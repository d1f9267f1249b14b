"""The decoder-layer stack of a denoise pass replayed as a HIP graph gives the same bits as the
same kernels launched one by one: canvas, lock mask, statistics and logits after every pass of
a block, across a commit (which changes the context length, so the graph is captured again),
on the small bf16 model (2 layers, d=256, 64 experts top-4, V=1024, prompt 4296).  Between the
graph replays the host runs eager work (LM head, sampler, copies) and synchronises."""
import numpy as np
import pytest
import torch

import fixtures as fx
from fixtures.dg_glue import build_handle
from gpu_util import i32_dev, log, logits_capture, need_gpu, stats_capture

pytestmark = pytest.mark.gpu
W = fx.SMALL_BF16


def _passes(dg, h, graphs, seed, n):
    """n passes from the initial canvas of `seed`; per pass (canvas, mask, stats, logits)."""
    dg.dg_set_graphs(h, graphs)
    canvas = torch.empty(W.canvas, dtype=torch.int32, device="cuda")
    mask = torch.empty(W.canvas, dtype=torch.uint8, device="cuda")
    dg.dg_init_canvas(h, canvas, mask, seed)
    out = []
    for s in range(n):
        dg.dg_denoise_step(h, canvas, mask, s, W.T, seed)
        torch.cuda.synchronize()
        st = stats_capture(dg, h, W.canvas)
        z = logits_capture(dg, h, W.canvas, W.vocab).cpu().numpy()
        out.append((canvas.cpu().numpy().copy(), mask.cpu().numpy().copy(), st, z))
    return out, canvas


def _same(a, b, what):
    for s, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x[0], y[0]), f"{what} pass {s}: canvas differs"
        assert np.array_equal(x[1], y[1]), f"{what} pass {s}: mask differs"
        for key in x[2]:
            assert np.array_equal(x[2][key].view(np.uint8), y[2][key].view(np.uint8)), \
                f"{what} pass {s}: statistic {key} differs"
        assert np.array_equal(x[3].view(np.uint32), y[3].view(np.uint32)), f"{what} pass {s}: logits differ"


@pytest.fixture(scope="module")
def env():
    dg = need_gpu()
    h = build_handle(dg, W, capture_mask=dg.DG_CAP_LOGITS | dg.DG_CAP_STATS,
                     max_ctx=W.prompt_len + 2 * W.canvas)
    dg.dg_prefill_prompt_kv(h, i32_dev(fx.prompt_ids(W)), W.prompt_len)
    torch.cuda.synchronize()
    yield dg, h
    dg.dg_destroy(h)


def test_graph_replays_match_eager(env):
    dg, h = env
    n = 4
    g0, _ = _passes(dg, h, True, 7, n)
    e0, _ = _passes(dg, h, False, 7, n)
    _same(g0, e0, "block 0")
    g1, _ = _passes(dg, h, True, 7, n)     # captured again after the eager passes
    _same(g1, e0, "block 0 again")
    log(f"{n} passes: graph and eager results identical")


def test_graph_after_commit(env):
    dg, h = env
    _, canvas = _passes(dg, h, True, 11, 2)
    n0, _ = dg.dg_get_state(h)
    dg.dg_commit_canvas(h, canvas)
    torch.cuda.synchronize()
    n1, k1 = dg.dg_get_state(h)
    assert n1 == n0 + W.canvas and k1 >= 1
    g, _ = _passes(dg, h, True, 12, 3)
    e, _ = _passes(dg, h, False, 12, 3)
    _same(g, e, "after commit")
    dg.dg_set_graphs(h, True)
