"""GPU parity of the attention and MoE entry points against the CPU oracle."""
import math

import numpy as np
import pytest
import torch

import fixtures as fx
from oracle import model as om
from oracle.numerics import round_bf16, e4m3_round
from parity import DELTA, TOL, assert_close, gated_mismatches, routing_sets
from gpu_util import bf16_dev, bf16_host_f64, bits_f64, log, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    return need_gpu()


# ------------------------------------------------------------------ attention
def _workspace(dg, Hq, Hkv, M, S, D, causal, q_pos0, code):
    """Caller-owned workspace of the attention call (None when it needs none)."""
    n = dg.dg_attention_workspace_size(Hq, Hkv, M, S, D, causal, q_pos0, code)
    return torch.empty(n, dtype=torch.uint8, device="cuda") if n else None


def _attn_case(dg, Hq, Hkv, M, S, causal, q_pos0, seed, dtype="bf16", D=128):
    rng = np.random.default_rng(seed)
    if dtype == "bf16":
        q = fx.normal(seed, 900, (Hq, M, D), 1.0, "bf16")
        k = fx.normal(seed, 901, (Hkv, S, D), 1.0, "bf16")
        v = fx.normal(seed, 902, (Hkv, S, D), 1.0, "bf16")
        qd, kd, vd = bf16_dev(q), bf16_dev(k), bf16_dev(v)
        qf, kf, vf = bits_f64(q), bits_f64(k), bits_f64(v)
        o = torch.empty(M, Hq * D, dtype=torch.bfloat16, device="cuda")
        code = dg.DG_BF16
    else:
        qf = rng.standard_normal((Hq, M, D)).astype(np.float32)
        kf = rng.standard_normal((Hkv, S, D)).astype(np.float32)
        vf = rng.standard_normal((Hkv, S, D)).astype(np.float32)
        qd, kd, vd = (torch.from_numpy(a).cuda() for a in (qf, kf, vf))
        qf, kf, vf = (a.astype(np.float64) for a in (qf, kf, vf))
        o = torch.empty(M, Hq * D, dtype=torch.float32, device="cuda")
        code = dg.DG_F32
    log(f"attention Hq={Hq} Hkv={Hkv} M={M} S={S} causal={causal} q_pos0={q_pos0} {dtype}")
    ws = _workspace(dg, Hq, Hkv, M, S, D, causal, q_pos0, code)
    dg.dg_attention(qd, kd, vd, o, Hq, Hkv, M, S, D, 1.0 / math.sqrt(D), causal, q_pos0, code, ws)
    torch.cuda.synchronize()
    ref = om.attention(qf, kf, vf, causal=causal, q_pos=np.arange(q_pos0, q_pos0 + M),
                       k_pos=np.arange(S))
    ref = ref.transpose(1, 0, 2).reshape(M, Hq * D)
    if dtype == "bf16":
        got = bf16_host_f64(o)
        return assert_close("attention", got, round_bf16(ref), *TOL["bf16"])
    got = o.cpu().numpy().astype(np.float64)
    return assert_close("attention f32", got, ref, *TOL["f32"])


def test_attention_gqa_prompt4096_canvas256_bf16(dg):
    # 16 query / 8 KV heads of dim 128, 4096 cached prompt keys + 256 canvas keys, non-causal
    q, k, v = fx.attn_inputs(fx.ATTN)
    a = fx.ATTN
    o = torch.empty(a.canvas, a.n_q_heads * a.head_dim, dtype=torch.bfloat16, device="cuda")
    log("attention workload 16x8 heads, S=4352")
    ws = _workspace(dg, a.n_q_heads, a.n_kv_heads, a.canvas, a.seq, a.head_dim, False, 0,
                    dg.DG_BF16)
    dg.dg_attention(bf16_dev(q), bf16_dev(k), bf16_dev(v), o, a.n_q_heads, a.n_kv_heads,
                    a.canvas, a.seq, a.head_dim, 1.0 / math.sqrt(128), False, 0, dg.DG_BF16, ws)
    torch.cuda.synchronize()
    ref = om.attention(bits_f64(q), bits_f64(k), bits_f64(v))
    ref = ref.transpose(1, 0, 2).reshape(a.canvas, -1)
    err = assert_close("attention workload", bf16_host_f64(o), round_bf16(ref), *TOL["bf16"])
    log(f"max abs err {err:.3g}")


@pytest.mark.parametrize("Hq,Hkv,M,S,causal,q_pos0", [
    (4, 2, 40, 100, False, 0),        # ragged queries and keys, several key blocks
    (4, 2, 40, 100, True, 60),        # causal with context prefix (commit shape)
    (2, 2, 256, 17, False, 0),        # fewer keys than one block
    (16, 8, 256, 8448, True, 8192),   # commit at the end of an 8192-token prompt
    (16, 8, 128, 128, True, 0),       # prefill chunk from position 0
])
def test_attention_edge_cases_bf16(dg, Hq, Hkv, M, S, causal, q_pos0):
    _attn_case(dg, Hq, Hkv, M, S, causal, q_pos0, seed=3)


@pytest.mark.parametrize("D,causal", [(64, False), (64, True), (128, False)])
def test_attention_f32(dg, D, causal):
    _attn_case(dg, 4, 2, 70, 150 if not causal else 70 + 30, causal, 30 if causal else 0,
               seed=4, dtype="f32", D=D)


# ------------------------------------------------------------------ MoE layer
def _moe_handle(dg, d, E, k, F, expert_dtype, tokens):
    cfg = dg.make_cfg(1, d, 16, 8, 128, E, k, F, 128, 256, max(256, tokens),
                      act_dtype=dg.DG_BF16, expert_dtype=expert_dtype)
    return dg.dg_create(cfg)


def _run_moe(dg, x_bits, wr, wg, wu, wd, k, expert_dtype="bf16"):
    T, d = x_bits.shape
    E, _, F = wg.shape
    code = {"bf16": dg.DG_BF16, "fp8": dg.DG_FP8_E4M3}[expert_dtype]
    h = _moe_handle(dg, d, E, k, F, code, T)
    try:
        dg.dg_load_tensor(h, dg.DG_T_WR, 0, 0, wr)
        if expert_dtype == "bf16":
            for kind, w in ((dg.DG_T_WG, wg), (dg.DG_T_WU, wu), (dg.DG_T_WD, wd)):
                dg.dg_load_tensor(h, kind, 0, -1, np.ascontiguousarray(w))
            wfn = lambda e: (bits_f64(wg[e]), bits_f64(wu[e]), bits_f64(wd[e]))
        else:
            deq = {}
            for kind, w in ((dg.DG_T_WG, wg), (dg.DG_T_WU, wu), (dg.DG_T_WD, wd)):
                parts = [fx.quant_e4m3_cols(w[e]) for e in range(E)]
                codes = np.ascontiguousarray(np.stack([p[0] for p in parts]))
                scales = np.ascontiguousarray(np.stack([p[1] for p in parts]))
                dg.dg_load_tensor(h, kind, 0, -1, codes, scales)
                table = fx.e4m3_decode_table()
                deq[kind] = [table[codes[e]] * scales[e].astype(np.float64)[None, :] for e in range(E)]
            wfn = lambda e: (deq[dg.DG_T_WG][e], deq[dg.DG_T_WU][e], deq[dg.DG_T_WD][e])
        xd = bf16_dev(x_bits)
        y = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
        idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
        gates = torch.empty(T, k, dtype=torch.float32, device="cuda")
        dg.dg_moe_layer(h, 0, xd, T, y, idx, gates)
        torch.cuda.synchronize()
        y2 = torch.empty_like(y)
        dg.dg_moe_layer(h, 0, xd, T, y2)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "MoE layer not deterministic"
    finally:
        dg.dg_destroy(h)
    xf = bits_f64(x_bits)
    r = xf @ (bits_f64(wr) if wr.dtype == np.uint16 else wr)
    ridx, rg, margin = om.route_topk(r, k)
    if expert_dtype == "bf16":
        yref = om.moe_ffn(xf, ridx, rg, wfn, hidden_round=round_bf16)
    else:
        yref = om.moe_ffn(xf, ridx, rg, wfn, expert_round=e4m3_round, hidden_round=e4m3_round)
    gi = idx.cpu().numpy()
    bad, n_gated, in_band = gated_mismatches(routing_sets(gi), routing_sets(ridx), margin)
    assert bad == 0, f"{bad} gated routing mismatches of {n_gated}"
    same = np.all(routing_sets(gi) == routing_sets(ridx), axis=1)
    # gates per expert: order both sides by expert id
    og, orf = np.argsort(gi, axis=1), np.argsort(ridx, axis=1)
    g_gpu = np.take_along_axis(gates.cpu().numpy(), og, axis=1)
    g_ref = np.take_along_axis(rg, orf, axis=1)
    assert_close("gates", g_gpu[same], g_ref[same], 1e-5, 1e-4)
    tol = TOL["bf16"] if expert_dtype == "bf16" else TOL["fp8"]
    err = assert_close("moe y", bf16_host_f64(y)[same], round_bf16(yref)[same], *tol)
    return err, in_band, np.bincount(ridx.ravel(), minlength=E)


def test_moe_layer_256tok_d2816_E128_top8(dg):
    x, wr, wg, wu, wd = fx.moe_inputs(fx.MOE_LAYER)
    log("MoE workload d=2816 E=128 k=8 F=704")
    err, in_band, load = _run_moe(dg, x, wr, wg, wu, wd, 8)
    log(f"max abs err {err:.3g}; in-band routing differences {in_band}; "
        f"load min {load.min()} max {load.max()}")


def test_moe_layer_skewed_all_tokens_one_expert(dg):
    rng = np.random.default_rng(5)
    T, d, E, k, F = 256, 128, 64, 2, 128
    x = fx.normal(1, 910, (T, d), 1.0, "bf16")
    x = (x & np.uint16(0x7FFF))                              # |x|: all positive
    wr = fx.normal(1, 911, (d, E), 0.02, "bf16")
    wr[:, 5] = fx.bf16_encode_scalar(1.0)                    # expert 5 wins every token
    wg = fx.normal(1, 912, (E, d, F), 0.1, "bf16")
    wu = fx.normal(1, 913, (E, d, F), 0.1, "bf16")
    wd = fx.normal(1, 914, (E, F, d), 0.1, "bf16")
    err, in_band, load = _run_moe(dg, x, wr, wg, wu, wd, k)
    assert load[5] == T and (load == 0).sum() > 10


@pytest.mark.parametrize("T", [512, 520])
def test_moe_layer_routing_capacity(dg, T):
    """256 experts top-16 (the largest expert count and k the routing takes).  512 tokens give
    8192 entries, the most the one-block permutation takes (each of its 1024 threads holds 8);
    520 tokens take the chunked path (per-chunk counts, one scan, per-chunk scatter)."""
    d, E, k, F = 128, 256, 16, 128
    x = fx.normal(3, 930, (T, d), 1.0, "bf16")
    wr = fx.normal(3, 931, (d, E), 0.05, "bf16")
    wg = fx.normal(3, 932, (E, d, F), 0.05, "bf16")
    wu = fx.normal(3, 933, (E, d, F), 0.05, "bf16")
    wd = fx.normal(3, 934, (E, F, d), 0.05, "bf16")
    err, in_band, load = _run_moe(dg, x, wr, wg, wu, wd, k)
    assert load.sum() == T * k
    log(f"T={T} E={E} k={k}: max abs err {err:.3g}; in-band routing differences {in_band}; "
        f"experts hit {(load > 0).sum()}")


def test_moe_layer_fp8_experts(dg):
    T, d, E, k, F = 256, 256, 64, 4, 128
    x = fx.normal(2, 920, (T, d), 1.0, "bf16")
    wr = fx.normal(2, 921, (d, E), 0.02, "bf16")
    wg = fx.normal(2, 922, (E, d, F), 0.02, "f32")
    wu = fx.normal(2, 923, (E, d, F), 0.02, "f32")
    wd = fx.normal(2, 924, (E, F, d), 0.02, "f32")
    err, in_band, _ = _run_moe(dg, x, wr, wg, wu, wd, k, expert_dtype="fp8")
    log(f"fp8 MoE max abs err {err:.3g}")
