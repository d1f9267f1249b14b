"""dg_attention_noalloc (static device scratch, no allocation) gives the same bits as
dg_attention with a caller-owned workspace, on two calls in a row, the second smaller
(the scratch keeps the first call's contents), and refuses sizes beyond its scratch."""
import math

import numpy as np
import pytest
import torch

import fixtures as fx
from gpu_util import bf16_dev, log, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    return need_gpu()


def _inputs(Hq, Hkv, M, S, seed):
    q = bf16_dev(fx.normal(seed, 900, (Hq, M, 128), 1.0, "bf16"))
    k = bf16_dev(fx.normal(seed, 901, (Hkv, S, 128), 1.0, "bf16"))
    v = bf16_dev(fx.normal(seed, 902, (Hkv, S, 128), 1.0, "bf16"))
    return q, k, v


@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_workspace_call_twice(dg, causal):
    # first the 16/8-head, 4096 + 256-key shape, then a smaller ragged one
    for (Hq, Hkv, M, S, q_pos0, seed) in ((16, 8, 256, 4352, 4096, 3), (4, 2, 40, 300, 260, 4)):
        q, k, v = _inputs(Hq, Hkv, M, S, seed)
        qp = q_pos0 if causal else 0
        n = dg.dg_attention_workspace_size(Hq, Hkv, M, S, 128, causal, qp, dg.DG_BF16)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
        ref = torch.empty(M, Hq * 128, dtype=torch.bfloat16, device="cuda")
        got = torch.full((M, Hq * 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        log(f"noalloc attention Hq={Hq} Hkv={Hkv} M={M} S={S} causal={causal} ws={n}")
        scale = 1.0 / math.sqrt(128)
        dg.dg_attention(q, k, v, ref, Hq, Hkv, M, S, 128, scale, causal, qp, dg.DG_BF16, ws)
        dg.dg_attention_noalloc(q, k, v, got, Hq, Hkv, M, S, 128, scale, causal, qp, dg.DG_BF16)
        torch.cuda.synchronize()
        assert torch.isfinite(ref.float()).all()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_noalloc_rejects_sizes_beyond_its_scratch(dg):
    # a transposed V copy of 8 heads x 128 dims x 65536 keys alone is 128 MiB > 64 MiB
    Hq, Hkv, M, S = 16, 8, 256, 65536
    n = dg.dg_attention_workspace_size(Hq, Hkv, M, S, 128, False, 0, dg.DG_BF16)
    assert n > 64 << 20
    t = torch.empty(16, dtype=torch.bfloat16, device="cuda")     # never read: rejected first
    with pytest.raises(dg.DGError) as ei:
        dg.dg_attention_noalloc(t, t, t, t, Hq, Hkv, M, S, 128, 0.1, False, 0, dg.DG_BF16)
    assert ei.value.code == dg.DG_EINVAL and "scratch" in str(ei.value)
